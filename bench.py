"""Benchmark of the block-sparse attention layer on one MI355X.

Workload: the Wan-14B-like layer (B=1, H=40, N=75600 = 21 x 45 x 80 tokens,
d=128, 128-token blocks), top-k key tiles at 95% sparsity, bf16 inputs from
the seeded generator (already resident in HBM when timing starts).

A step is one pass of the whole path: pool + classify, list compaction (and
the query-block run order, sla_row_order, timed with it), sparse attention (bf16 output written directly: this workload has no
marginal tiles, so the linear branch and the sum are empty).  Workloads
with marginal tiles (--config wan1p3b, long_clip_95, long_clip_90) run the
linear branch's preparation and then the fused sparse + linear kernel that
stores O once; --unfused times the separate sparse, linear and combine calls.

Printed JSON line:
  value        kept-block attention FLOP per step / step time (TFLOP/s),
               i.e. whole-layer effective throughput;
  roofline     the sparse-attention kernel alone: kept FLOP per launch /
               its average launch time (HIP events on its stream) against
               the bf16 dense MFMA peak; traffic = HBM bytes per launch from
               the committed counter summary of the same kernel source, else
               null;
  cpu_baseline the fp64 oracle on the host cores on a bounded sample, and
               (parity) the GPU's class map and bf16 output on those sampled
               heads and query blocks compared with it;
  extra        per-stage times, dense baselines (this library's dense kernel
               and torch SDPA) and ms/layer ratios, the inputs' SHA-256, the
               shader clock during the attention kernel (a probe wave on a
               second stream), and the pool + classify stage's HBM bytes and
               GB/s from its committed counter summary.

python bench.py [--gpus 1] [--steps K] [--warmup W] [--config wan14b]
                [--no-cpu-baseline] [--no-dense] [--profile] [--unfused]
                [--keep F]

--keep F replaces a top-k workload's kept fraction (the sparsity sweep that
checks the kernel's time and MFMA work scale with the kept tiles); the line
then describes that workload, not the headline one.
"""

import argparse
import json
import math
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2500.0   # MI355X dense bf16 MFMA
PEAK_HBM_GBS = 8000.0


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def kept_flop(crit_idx, crit_cnt, N, block, d):
    """Exact kept-pair FLOP: 4 * rows(i) * keys(j) * d over every kept pair."""
    import torch
    width = crit_idx.shape[-1]
    nqb = crit_idx.shape[-2]
    valid = torch.arange(width, device=crit_idx.device) < crit_cnt[..., None]
    j = torch.where(valid, crit_idx, torch.zeros_like(crit_idx)).long()
    keys = torch.clamp(N - j * block, max=block)
    keys = torch.where(valid, keys, torch.zeros_like(keys))
    rows = torch.clamp(N - torch.arange(nqb, device=j.device) * block, max=block)
    per = (keys.sum(-1) * rows).sum().item()
    return 4.0 * per * d


def pipe_mfma_flop(crit_idx, crit_cnt, N):
    """MFMA FLOP the d = 128, 128-token kernel issues for these lists: every
    kept tile runs its first 64-key half, and its second when that half holds
    a key below N; a half is 4 waves x 32 MFMAs of 32x32x16 (32768 FLOP), over
    all 128 rows of the query block (the rows past N of the last block too)."""
    import torch
    width = crit_idx.shape[-1]
    valid = torch.arange(width, device=crit_idx.device) < crit_cnt[..., None]
    j = torch.where(valid, crit_idx, torch.zeros_like(crit_idx)).long()
    halves = torch.where(valid, 1 + (j * 128 + 64 < N).long(), torch.zeros_like(j))
    return float(halves.sum().item()) * 4 * 32 * 32768


# Sources of the sparse-attention kernel; a counter summary applies only to the
# build whose sources hash to the value recorded in it.
KERNEL_SOURCES = ["sparse_attn.hip", "common.h", "linear_apply.h", "lists.h"]


def kernel_source_hash():
    import hashlib
    h = hashlib.sha256()
    for f in KERNEL_SOURCES:
        with open(os.path.join(ROOT, "block_sparse_attention_meanpool_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()


POOL_SOURCES = ["pool_classify.hip", "common.h"]


def pool_source_hash():
    import hashlib
    h = hashlib.sha256()
    for f in POOL_SOURCES:
        with open(os.path.join(ROOT, "block_sparse_attention_meanpool_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()


def _profile_fields(config_name):
    path = os.path.join(ROOT, "profiles", f"hbm_traffic_attn_{config_name}.md")
    fields = {}
    if os.path.exists(path):
        with open(path) as fh:
            for line in fh:
                if line.startswith("- ") and ": " in line:
                    key, val = line[2:].split(": ", 1)
                    fields[key.strip()] = val.strip().strip("`")
    return fields


def measured_pool_traffic(config_name):
    """HBM bytes per step of the pool + score + select kernels from the committed
    counter summary, or None when there is none or their sources have changed."""
    fields = _profile_fields(config_name)
    if fields.get("pool classify source sha256") != pool_source_hash():
        return None
    try:
        return {"fetch": float(fields["pool classify fetch bytes per step"]),
                "write": float(fields["pool classify write bytes per step"])}
    except (KeyError, ValueError):
        return None


def measured_traffic(config_name):
    """HBM bytes per launch of the sparse-attention kernel from the committed
    counter summary (FETCH_SIZE + WRITE_SIZE, copy-calibrated), or None when
    there is none for this workload or the kernel has changed since."""
    path = os.path.join(ROOT, "profiles", f"hbm_traffic_attn_{config_name}.md")
    if not os.path.exists(path):
        return None
    fields = {}
    with open(path) as fh:
        for line in fh:
            if line.startswith("- ") and ": " in line:
                key, val = line[2:].split(": ", 1)
                fields[key.strip()] = val.strip().strip("`")
    if fields.get("kernel source sha256") != kernel_source_hash():
        return None
    try:
        return {"fetch": float(fields["fetch bytes per launch"]),
                "write": float(fields["write bytes per launch"])}
    except (KeyError, ValueError):
        return None


def backward_timing(sla, torch, q, k, v, b, crit_idx, crit_cnt, marg_idx, marg_cnt, km, flop,
                    steps, stream, order=None):
    """Gradients of the whole layer (mask held fixed) for a seeded dO: the
    softmax branch's backward and, with marginal tiles, the linear branch's,
    each timed with HIP events on the launch stream.  The forward's O_s and
    LSE are computed first, outside the timed region."""
    g = torch.Generator(device=q.device).manual_seed(7)
    d_o = torch.randn(q.shape, generator=g, device=q.device, dtype=torch.float32).to(torch.bfloat16)
    o_s, lse = sla.sla_sparse_attn_fwd(q, k, v, b, crit_idx, crit_cnt, o_fp32=False,
                                       want_lse=True, row_order=order)
    dq, dk, dv = (torch.empty(q.shape, dtype=torch.float32, device=q.device) for _ in range(3))
    B, H, N, d = q.shape
    ws = torch.empty(sla.lib().sla_sparse_attn_bwd_ws_bytes(B, H, N, d, b), dtype=torch.uint8,
                     device=q.device)
    lin_ws = lws = None
    if km:
        lin_ws = sla.sla_linear_branch_prepare(k, v, b, marg_idx, marg_cnt)
        lws = torch.empty(sla.lib().sla_linear_branch_bwd_ws_bytes(B, H, N, d, b),
                          dtype=torch.uint8, device=q.device)

    def run(marks):
        if marks:
            marks[0].record(stream)
        sla.sla_sparse_attn_bwd(q, k, v, b, crit_idx, crit_cnt, o_s, lse, d_o, dq=dq, dk=dk, dv=dv,
                                ws=ws, row_order=order)
        if marks:
            marks[1].record(stream)
        if km:
            sla.sla_linear_branch_bwd(q, k, v, b, marg_idx, marg_cnt, d_o, lin_ws, dq, dk, dv,
                                      ws=lws)
            if marks:
                marks[2].record(stream)

    run(None)
    torch.cuda.synchronize()
    reps = max(1, min(steps, 5))
    all_marks = []
    for _ in range(reps):
        marks = [torch.cuda.Event(enable_timing=True) for _ in range(3)]
        run(marks)
        all_marks.append(marks)
    torch.cuda.synchronize()
    sm = float(np.mean([m[0].elapsed_time(m[1]) for m in all_marks]))
    out = {"sparse_bwd_ms": sm, "reps": reps,
           "sparse_bwd_tflops_2p5x": 2.5 * flop / (sm * 1e-3) / 1e12,
           "note": "2.5 x the kept forward FLOP, the usual accounting of an attention backward; "
                   "the kernels recompute S and dP in both passes (3.5 x executed)"}
    if km:
        out["linear_bwd_ms"] = float(np.mean([m[1].elapsed_time(m[2]) for m in all_marks]))
    del d_o, o_s, lse, dq, dk, dv, ws, lin_ws, lws
    return out


def describe(spec, kc, km):
    grid = f" ({'x'.join(str(x) for x in spec.grid)})" if spec.grid else ""
    if spec.mode == "topk":
        sel = (f"top-{kc} of {spec.nb} key tiles per query block "
               f"({100 * (1 - kc / spec.nb):.0f}% sparsity)")
    elif spec.mode == "cdf":
        sel = f"softmax-CDF cut at thr={spec.thr}"
    else:
        sel = (f"{kc} critical + {km} marginal (linear) of {spec.nb} key tiles per query block"
               + (" (mask given)" if spec.mode == "maskin" else ""))
    return (f"{spec.name}: B={spec.B} H={spec.H} N={spec.N}{grid} d={spec.d} "
            f"block={spec.block}, {sel}")


def cpu_baseline(spec, data, kc, km, budget_s=20.0, gpu=None):
    """Time the fp64 oracle on a bounded sample of the workload on the host cores.

    With `gpu` = (class map uint8 [B, H, nb, nb], bf16 output bits uint16 [B, H, N, d]) of the
    timed run, the sampled oracle rows are also compared with the GPU's: the class map of every
    sampled head bit for bit, and the output of every sampled query block (max-abs and rel-L2 of
    the bf16 output against the fp64 one)."""
    from oracle import sla as osla
    try:
        from threadpoolctl import threadpool_info
        cores = max((i.get("num_threads", 1) for i in threadpool_info()), default=1)
    except Exception:
        cores = os.cpu_count() or 1
    sel = "sla3" if spec.mode == "maskin" else spec.mode
    flop = 0.0
    blocks = 0
    t0 = time.perf_counter()
    g = np.random.default_rng(0)
    h = 0
    cmp = {"cls_mismatch": 0, "err2": 0.0, "ref2": 0.0, "max_abs": 0.0}
    check = 0.0
    while time.perf_counter() - t0 - check < budget_s and h < spec.H:
        q = osla.bf16_to_f64(data["q"][0, h])[None, None]
        k = osla.bf16_to_f64(data["k"][0, h])[None, None]
        v = osla.bf16_to_f64(data["v"][0, h])[None, None]
        cls, *_ = osla.class_map(q, k, spec.block, sel, spec.keep, spec.marg, spec.thr)
        rows = [(0, 0, int(i)) for i in g.choice(spec.nb, size=min(spec.nb, 128), replace=False)]
        res = osla.forward_rows(q, k, v, cls, spec.block, rows)
        for (_, _, i) in rows:
            lo, hi = osla.block_bounds(spec.N, spec.block, i)
            for j in np.nonzero(cls[0, 0, i] == osla.CRITICAL)[0]:
                klo, khi = osla.block_bounds(spec.N, spec.block, int(j))
                flop += 4.0 * (hi - lo) * (khi - klo) * spec.d
        blocks += len(rows)
        if gpu is not None:   # outside the timed work: compare with the GPU's rows
            t1 = time.perf_counter()
            g_cls, g_o = gpu
            cmp["cls_mismatch"] += int((g_cls[0, h] != cls[0, 0]).sum())
            for (_, _, i) in rows:
                lo, hi = osla.block_bounds(spec.N, spec.block, i)
                got = osla.bf16_to_f64(g_o[0, h, lo:hi])
                ref = res[(0, 0, i)][3]
                cmp["err2"] += float(((got - ref) ** 2).sum())
                cmp["ref2"] += float((ref ** 2).sum())
                cmp["max_abs"] = max(cmp["max_abs"], float(np.abs(got - ref).max()))
            check += time.perf_counter() - t1
        h += 1
    dt = time.perf_counter() - t0 - check
    single = None
    if spec.N * spec.H <= 4096:
        # a workload small enough for the whole oracle forward on one BLAS thread
        from threadpoolctl import threadpool_limits
        q, k, v = (osla.bf16_to_f64(data[t]) for t in "qkv")
        with threadpool_limits(1):
            t1 = time.perf_counter()
            cls, *_ = osla.class_map(q, k, spec.block, sel, spec.keep, spec.marg, spec.thr)
            osla.forward(q, k, v, cls, spec.block)
            single = time.perf_counter() - t1
    out = {"value": flop / dt / 1e12, "unit": "TFLOP/s", "cores": int(cores), "kind": "oracle",
            "sample": (f"fp64 numpy oracle: pool + score + top-k class map of {h} head(s) in full, "
                       f"then masked softmax attention of {blocks} sampled query blocks "
                       f"({min(spec.nb, 128)} per head); kept-block FLOP of those blocks / wall time "
                       f"({dt:.1f} s)")}
    if single is not None:
        out["single_core_full_forward_s"] = single
    if gpu is not None:
        out["parity"] = {
            "heads": h, "query_blocks": blocks,
            "class_map_mismatches": cmp["cls_mismatch"],
            "o_bf16_max_abs": cmp["max_abs"],
            "o_bf16_rel_l2": (cmp["err2"] / cmp["ref2"]) ** 0.5 if cmp["ref2"] > 0 else 0.0,
            "what": "GPU class map of the sampled heads vs the oracle's (bit-exact expected); "
                    "GPU bf16 output of the sampled query blocks vs the fp64 oracle"}
    return out


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--config", default="wan14b")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-dense", action="store_true")
    ap.add_argument("--profile", action="store_true", help="short run for a profiler")
    ap.add_argument("--profile-dense", action="store_true",
                    help="with --profile: one dense-kernel launch after the copy")
    ap.add_argument("--no-backward", action="store_true", help="skip the backward timing")
    ap.add_argument("--unfused", action="store_true",
                    help="with a linear branch: separate sparse, linear and combine calls")
    ap.add_argument("--keep", default=None,
                    help="kept fraction for a top-k workload, e.g. 1/10 (sparsity sweep)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only (asked for --gpus {args.gpus}); the path shards by "
              "head with no communication inside attention, so run one process per GPU instead.",
              file=sys.stderr)
        sys.exit(2)
    if args.profile:
        args.no_cpu_baseline = True
        args.no_dense = True
        args.no_backward = True

    import torch
    import block_sparse_attention_meanpool_amd as sla
    from synth import CONFIGS, generate

    spec = CONFIGS[args.config]
    if args.keep is not None:
        import dataclasses
        from fractions import Fraction
        if spec.mode != "topk":
            log("[bench] --keep applies to top-k workloads only")
            sys.exit(2)
        spec = dataclasses.replace(spec, keep=Fraction(args.keep))
    B, H, N, d, b, nb = spec.B, spec.H, spec.N, spec.d, spec.block, spec.nb
    sel = "sla3" if spec.mode == "maskin" else spec.mode
    kc, km = sla.counts_for(sel, nb, spec.keep, spec.marg)
    log(f"[bench] {spec.name}: B={B} H={H} N={N} d={d} block={b} nb={nb} k_crit={kc} k_marg={km}")
    t0 = time.time()
    data = generate(spec)
    log(f"[bench] generated inputs in {time.time() - t0:.1f} s")
    import hashlib
    input_sha = {t: hashlib.sha256(np.ascontiguousarray(data[t]).tobytes()).hexdigest()
                 for t in "qkv"}
    dev = torch.device("cuda:0")
    q, k, v = (torch.from_numpy(data[t].view(np.int16)).view(torch.bfloat16).to(dev) for t in "qkv")
    torch.cuda.synchronize()

    # every buffer allocated once, outside the timed region
    cls = torch.empty((B, H, nb, nb), dtype=torch.uint8, device=dev)
    ws = torch.empty(sla.lib().sla_pool_classify_ws_bytes(B, H, N, d, b, 0), dtype=torch.uint8,
                     device=dev)
    kc_max = nb if sel == "cdf" else kc
    crit_idx = torch.empty((B, H, nb, kc_max), dtype=torch.int32, device=dev)
    crit_cnt = torch.empty((B, H, nb), dtype=torch.int32, device=dev)
    marg_idx = marg_cnt = o_s = o_lin = lin_ws = None
    if km:
        marg_idx = torch.empty((B, H, nb, km), dtype=torch.int32, device=dev)
        marg_cnt = torch.empty((B, H, nb), dtype=torch.int32, device=dev)
        if args.unfused:
            o_s = torch.empty(q.shape, dtype=torch.float32, device=dev)
            o_lin = torch.empty(q.shape, dtype=torch.float32, device=dev)
        lin_ws = torch.empty(sla.lib().sla_linear_branch_ws_bytes(B, H, N, d, b), dtype=torch.uint8,
                             device=dev)
    o = torch.empty(q.shape, dtype=torch.bfloat16, device=dev)
    order = torch.empty((B, H, nb), dtype=torch.int32, device=dev)
    stream = torch.cuda.current_stream()

    fused = bool(km) and not args.unfused
    if fused:
        stages = ["pool_classify", "block_mask", "linear_prepare", "sparse_attn"]
    else:
        stages = ["pool_classify", "block_mask", "sparse_attn"] + (["linear_branch", "combine"] if km else [])
    ev = {s: [] for s in stages}

    def step(record):
        marks = [torch.cuda.Event(enable_timing=True) for _ in range(len(stages) + 1)] if record else None
        if record:
            marks[0].record(stream)
        sla.sla_pool_classify(q, k, b, sel, kc, km, spec.thr or 0.0, cls=cls, ws=ws)
        if record:
            marks[1].record(stream)
        sla.sla_block_mask(cls, kc_max, km, crit_idx, crit_cnt, marg_idx, marg_cnt)
        sla.sla_row_order(crit_idx, crit_cnt, order)
        if record:
            marks[2].record(stream)
        if fused:
            sla.sla_linear_branch_prepare(k, v, b, marg_idx, marg_cnt, ws=lin_ws)
            if record:
                marks[3].record(stream)
            sla.sla_sparse_linear_attn_fwd(q, k, v, b, crit_idx, crit_cnt, lin_ws, o=o,
                                           row_order=order)
            if record:
                marks[4].record(stream)
        elif km:
            sla.sla_sparse_attn_fwd(q, k, v, b, crit_idx, crit_cnt, o_s=o_s, row_order=order)
            if record:
                marks[3].record(stream)
            sla.sla_linear_branch_fwd(q, k, v, b, marg_idx, marg_cnt, o_lin=o_lin, ws=lin_ws)
            if record:
                marks[4].record(stream)
            sla.sla_combine(o_s, o_lin, o=o)
            if record:
                marks[5].record(stream)
        else:
            sla.sla_sparse_attn_fwd(q, k, v, b, crit_idx, crit_cnt, o_s=o, row_order=order)
            if record:
                marks[3].record(stream)
        if record:
            ev_list.append(marks)

    ev_list = []
    for _ in range(args.warmup):
        step(False)
    torch.cuda.synchronize()
    log(f"[bench] warmup {args.warmup} steps done")
    t_start = time.perf_counter()
    for _ in range(args.steps):
        step(True)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t_start
    for marks in ev_list:
        for i, s in enumerate(stages):
            ev[s].append(marks[i].elapsed_time(marks[i + 1]))
    ms_step = wall * 1e3 / args.steps
    stage_ms = {s: float(np.mean(ev[s])) for s in stages}
    stage_min = {s: float(np.min(ev[s])) for s in stages}
    stage_med = {s: float(np.median(ev[s])) for s in stages}
    log(f"[bench] timed {args.steps} steps: {ms_step:.3f} ms/step; stages {stage_ms}")
    # The attention kernel's shader clock: the probe waits on a second stream
    # while a few more launches of the kernel run (outside the timed steps).
    def attn_only():
        if fused:
            sla.sla_sparse_linear_attn_fwd(q, k, v, b, crit_idx, crit_cnt, lin_ws, o=o,
                                           row_order=order)
        else:
            sla.sla_sparse_attn_fwd(q, k, v, b, crit_idx, crit_cnt,
                                    o_s=o_s if km else o, row_order=order)
    attn_ms = stage_ms["sparse_attn"]
    n_clk = max(3, min(20, int(200.0 / max(attn_ms, 1e-3))))
    side = torch.cuda.Stream()
    probe, fixed_hz = sla.sla_clock_probe(int(min(0.8 * n_clk * attn_ms * 1e3, 1e6)), stream=side)
    for _ in range(n_clk):
        attn_only()
    torch.cuda.synchronize()
    attn_sclk = sla.probe_clock_hz(probe, fixed_hz) / 1e9
    log(f"[bench] shader clock during the attention kernel: {attn_sclk:.3f} GHz")
    # the timed run's class map and output, for the oracle comparison of the CPU-baseline leg
    gpu_result = None
    if not args.no_cpu_baseline:
        gpu_result = (cls.cpu().numpy(), o.cpu().view(torch.int16).numpy().view(np.uint16))

    if args.profile:
        # a plain 1 GiB device copy, the reference for scaling HBM counters
        src = torch.empty(1 << 30, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
        if d == 128 and b == 128:
            log(f"[bench] expected MFMA FLOP per sparse launch: "
                f"{pipe_mfma_flop(crit_idx, crit_cnt, N) * B:.6e}")
        if args.profile_dense:
            od = torch.empty(q.shape, dtype=torch.bfloat16, device=dev)
            sla.sla_dense_attn_fwd(q, k, v, b, o=od)
            torch.cuda.synchronize()
            if d == 128 and b == 128:
                every = torch.arange(nb, dtype=torch.int32, device=dev).expand(B, H, nb, nb)
                full = torch.full((B, H, nb), nb, dtype=torch.int32, device=dev)
                log(f"[bench] expected MFMA FLOP per dense launch: "
                    f"{pipe_mfma_flop(every, full, N) * B:.6e} "
                    f"(attention FLOP 4*H*N*N*d: {4.0 * B * H * N * N * d:.6e})")
            del od

    flop = kept_flop(crit_idx, crit_cnt, N, b, d) * B
    kept_frac = crit_cnt.double().mean().item() / nb
    sparse_ms = stage_ms["sparse_attn"]
    achieved = flop / (sparse_ms * 1e-3) / 1e12
    value = flop / (ms_step * 1e-3) / 1e12
    pool_bytes = 2 * B * H * N * d * 2 + 2 * B * H * nb * d * 4
    extra = {
        "stage_ms_mean": stage_ms, "stage_ms_median": stage_med, "stage_ms_min": stage_min,
        "kept_fraction": kept_frac, "kept_flop_per_step": flop,
        "input_sha256": input_sha,
        "attn_sclk_ghz": attn_sclk,
        "sparse_kernel_tflops": achieved,
        "pool_classify_gbs_algorithmic": pool_bytes / (stage_ms["pool_classify"] * 1e-3) / 1e9,
    }

    # per-head 3D tile order (run on Q, K, V before the path and on O after it)
    if spec.grid and not args.profile:
        shape = (2, 8, 8) if b == 128 else (1, 8, 8)
        if all(g % t == 0 for g, t in zip(spec.grid, shape)):
            y = torch.empty_like(q)
            sla.sla_tile_permute(q, spec.grid, [shape] * H, b, y=y)
            torch.cuda.synchronize()
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            for t in (q, k, v):
                sla.sla_tile_permute(t, spec.grid, [shape] * H, b, y=y)
            sla.sla_tile_permute(o, spec.grid, [shape] * H, b, inverse=True, y=y)
            e1.record(stream)
            torch.cuda.synchronize()
            ms = e0.elapsed_time(e1)
            extra["tile_permute"] = {"tile": shape, "ms_qkv_and_o": ms,
                                     "gbs": 8 * q.numel() * 2 / (ms * 1e-3) / 1e9}
            del y

    # mask quality of this step's critical tiles (outside the timed region)
    if not args.profile:
        rec = sla.sla_mask_recall(q, k, b, crit_idx, crit_cnt)
        torch.cuda.synchronize()
        extra["mask_recall"] = {"mean": float(rec.double().mean().item()),
                                "min": float(rec.min().item()),
                                "what": "share of each query's dense softmax mass on its critical tiles"}
        del rec

    if not args.no_backward:
        extra["backward"] = backward_timing(sla, torch, q, k, v, b, crit_idx, crit_cnt, marg_idx,
                                            marg_cnt, km, flop, args.steps, stream, order)
        log(f"[bench] backward: {extra['backward']}")

    if not args.no_dense:
        od = torch.empty(q.shape, dtype=torch.bfloat16, device=dev)
        sla.sla_dense_attn_fwd(q, k, v, b, o=od)
        torch.cuda.synchronize()
        reps = 2
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(reps):
            sla.sla_dense_attn_fwd(q, k, v, b, o=od)
        e1.record(stream)
        torch.cuda.synchronize()
        dense_ms = e0.elapsed_time(e1) / reps
        dense_flop = 4.0 * B * H * N * N * d
        extra["dense_kernel_ms"] = dense_ms
        extra["dense_kernel_tflops"] = dense_flop / (dense_ms * 1e-3) / 1e12
        del od
        try:
            import torch.nn.functional as Fn
            from torch.nn.attention import SDPBackend, sdpa_kernel
            # flash / memory-efficient kernels only: never the bf16 math path
            with torch.no_grad(), sdpa_kernel([SDPBackend.FLASH_ATTENTION,
                                               SDPBackend.EFFICIENT_ATTENTION]):
                Fn.scaled_dot_product_attention(q[:, :4], k[:, :4], v[:, :4])
                torch.cuda.synchronize()
                e0.record(stream)
                Fn.scaled_dot_product_attention(q, k, v)
                e1.record(stream)
                torch.cuda.synchronize()
            extra["torch_sdpa_ms"] = e0.elapsed_time(e1)
            extra["torch_sdpa_tflops"] = dense_flop / (extra["torch_sdpa_ms"] * 1e-3) / 1e12
        except Exception as exc:  # context only
            extra["torch_sdpa_error"] = str(exc)[:200]
        best_dense = min(x for x in (extra.get("dense_kernel_ms"), extra.get("torch_sdpa_ms")) if x)
        extra["dense_best_ms"] = best_dense
        extra["speedup_vs_best_dense"] = best_dense / ms_step
        log(f"[bench] dense: ours {extra['dense_kernel_ms']:.2f} ms, sdpa {extra.get('torch_sdpa_ms')}")

    pool_traffic = measured_pool_traffic(spec.name)
    if pool_traffic is not None:
        extra["pool_classify_hbm_bytes_per_step"] = pool_traffic
        extra["pool_classify_gbs_counted"] = ((pool_traffic["fetch"] + pool_traffic["write"]) /
                                              (stage_ms["pool_classify"] * 1e-3) / 1e9)
    traffic = measured_traffic(spec.name)
    if traffic is not None:
        extra["attn_hbm_bytes_per_launch"] = traffic
        extra["attn_hbm_gbs"] = (traffic["fetch"] + traffic["write"]) / (sparse_ms * 1e-3) / 1e9
    result = {
        "metric": "effective attn TFLOP/s on kept blocks; ms/layer vs dense at 95% sparsity",
        "value": value, "unit": "TFLOP/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": ms_step, "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "bf16", "data": "synthetic (seeded random-Fourier video-latent fields + noise)",
        "config": {"workload": describe(spec, kc, km), "global_batch": B, "seq_len": N,
                   "parallelism": "none (1 GPU)",
                   "path": "fused" if fused else ("unfused" if km else "sparse only")},
        "roofline": {"bound": "mfma", "achieved": achieved, "peak": PEAK_BF16_TFLOPS,
                     "unit": "TFLOP/s", "frac": achieved / PEAK_BF16_TFLOPS,
                     "traffic": None if traffic is None else traffic["fetch"] + traffic["write"]},
        "extra": extra,
    }
    if not args.no_cpu_baseline:
        log("[bench] timing the oracle on the host cores")
        result["cpu_baseline"] = cpu_baseline(spec, data, kc, km, gpu=gpu_result)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
