"""Write the margin-repair tables under synth/repairs (one per workload seed).

For every (batch, head) of a workload this script generates Q and K, pools
them and scores the block pairs with the oracle, audits every row against the
selection boundaries of every selection rule run on that data, and for each
failing query block asks the generator for successive noise attempts of
that block's Q tokens until the row passes (at most 4096 attempts), then
regenerates and re-audits the whole head with the repairs, and stores the
attempts.  The generator only reads the tables.

Run:  python -m oracle.make_repairs [workload-seed ...]
TEST INFRASTRUCTURE ONLY (see the package header).
"""

import math
import sys
import time
from concurrent.futures import ProcessPoolExecutor

from synth import CONFIGS
from synth.generate import generate_head, head_field, q_block_bits, save_repairs

from . import margin, sla

MAX_ATTEMPTS = 4096


def boundaries_for(specs, nkb):
    cuts, thr = set(), None
    for sp in specs:
        if sp.mode == "cdf":
            thr = sp.thr
            continue
        sel = "sla3" if sp.mode == "maskin" else sp.mode
        kc, km = sla.selection_counts(sel, nkb, sp.keep, sp.marg)
        cuts.add(kc)
        if km:
            cuts.add(kc + km)
    return sorted(cuts), thr


def _scores(spec, q_bits, kp):
    qp = sla.pool(sla.bf16_to_f64(q_bits), spec.block)
    return sla.pooled_scores(qp, kp, 1.0 / math.sqrt(spec.d))


def repair_head(spec, cuts, thr, b, h):
    """Redraw each failing query block until its row passes; verify the whole head."""
    part = generate_head(spec, b, h, ("q", "k"))
    kp = sla.pool(sla.bf16_to_f64(part["k"]), spec.block)
    s = _scores(spec, part["q"], kp)
    bad = [int(i[0]) for i in margin.failing_rows(s, cuts, thr)]
    field = head_field(spec, b, h) if (bad and spec.kind == "fourier") else None
    repairs = {}
    for i in bad:
        lo, hi = sla.block_bounds(spec.N, spec.block, i)
        fld = field[lo:hi] if field is not None else None
        for a in range(1, MAX_ATTEMPTS + 1):
            row = _scores(spec, q_block_bits(spec, b, h, i, a, fld), kp)[0]
            if margin.row_ok(row, cuts, thr):
                repairs[(b, h, i)] = a
                break
        else:
            raise RuntimeError(f"cfg {spec.cfg_id} head {h} block {i}: no margin after "
                               f"{MAX_ATTEMPTS} redraws")
    if repairs:
        q = generate_head(spec, b, h, ("q",), repairs)["q"]
        left = margin.failing_rows(_scores(spec, q, kp), cuts, thr)
        if left:
            raise RuntimeError(f"cfg {spec.cfg_id} head {h}: rows {left} still fail after repair")
    return repairs


def _job(args):
    spec, cuts, thr, b, h = args
    return repair_head(spec, cuts, thr, b, h)


def make(cfg_id, workers=8):
    specs = [s for s in CONFIGS.values() if s.cfg_id == cfg_id]
    spec = specs[0]
    cuts, thr = boundaries_for(specs, spec.nb)
    t0 = time.time()
    jobs = [(b, h) for b in range(spec.B) for h in range(spec.H)]
    # One process per worker: numpy's BLAS must not be entered from several
    # threads of one process at once (concurrent calls corrupt results).
    with ProcessPoolExecutor(max_workers=workers) as ex:
        parts = list(ex.map(_job, [(spec, cuts, thr, b, h) for b, h in jobs]))
    repairs = {}
    for p in parts:
        repairs.update(p)
    meta = {"workloads": [s.name for s in specs], "boundaries": cuts, "thr": thr,
            "gap": 2e-4, "mass_gap": 1e-4, "rows": spec.B * spec.H * spec.nb,
            "repaired_rows": len(repairs), "max_attempt": max(repairs.values(), default=0)}
    save_repairs(cfg_id, repairs, meta)
    print(f"cfg {cfg_id}: {len(repairs)} of {meta['rows']} rows repaired, "
          f"max attempt {meta['max_attempt']}, {time.time() - t0:.1f} s", flush=True)


if __name__ == "__main__":
    ids = [int(a) for a in sys.argv[1:]] or sorted({s.cfg_id for s in CONFIGS.values()})
    for cid in ids:
        make(cid)
