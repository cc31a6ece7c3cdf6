"""Seeded generator of bf16 Q, K, V.

Recipe (every value is produced in float32 and rounded once to bf16 with
round-to-nearest-even):

* kind "iid": each of Q, K, V is N(0, 1), one numpy PCG64 stream per
  (cfg_id, tensor, batch, head) from ``SeedSequence([cfg_id, t, b, h])`` with
  t = 0, 1, 2 for Q, K, V.
* kind "fourier": a field is the sum of 8 low-frequency 3D random-Fourier
  modes over the (t, y, x) token grid,
      F_c(t, y, x) = sum_f a[f, c] * cos(2 pi (u_f . (t/T, y/Y, x/X)) + ph[f, c])
  with u_f ~ U[-2, 2]^3 (cycles per axis extent), a ~ N(0, 1/4) (so F has unit
  variance) and ph ~ U[0, 2 pi).  Q and K share one field (stream
  ``[cfg_id, 10, b, h]``), V has its own (``[cfg_id, 11, b, h]``); each tensor
  adds 0.3 * N(0, 1) noise from its own stream ``[cfg_id, t, b, h]``.
  Sharing the field gives the pooled Q.K scores the spatial-temporal locality
  of a video latent.
* margin repairs: a repair table maps (b, h, i) -> attempt a >= 1.  The tokens
  of query block i of that head then take their Q noise (their whole Q value
  for kind "iid") from stream ``[cfg_id, 0, b, h, i, a]``.  K and V are never
  touched, so a repair changes one row of the block-score matrix only.  The
  tables are written by a script next to the oracle and stored under
  ``synth/repairs``; this module only applies them.
"""

import json
import os
from concurrent.futures import ThreadPoolExecutor

import numpy as np

from .configs import Spec

_REPAIR_DIR = os.path.join(os.path.dirname(os.path.abspath(__file__)), "repairs")
_TENSOR_ID = {"q": 0, "k": 1, "v": 2}
_N_MODES = 8
_NOISE = np.float32(0.3)


def _rng(*key):
    return np.random.default_rng(np.random.SeedSequence(list(key)))


def f32_to_bf16_bits(x):
    """Round float32 values to bf16 (round to nearest, ties to even); uint16 bits."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32)
    bias = ((u >> np.uint32(16)) & np.uint32(1)) + np.uint32(0x7FFF)
    return ((u + bias) >> np.uint32(16)).astype(np.uint16)


def _field(spec: Spec, stream_key, lo=0, hi=None):
    """Sum of 8 random-Fourier modes over tokens [lo, hi) of the grid, float32 [hi - lo, d].

    Elementwise numpy only (no BLAS), accumulated mode by mode in a fixed
    order, so the values do not depend on threading.
    """
    if hi is None:
        hi = spec.N
    T, Y, X = spec.grid
    rng = _rng(*stream_key)
    u = rng.uniform(-2.0, 2.0, size=(_N_MODES, 3))
    amp = rng.normal(0.0, 0.5, size=(_N_MODES, spec.d))
    ph = rng.uniform(0.0, 2.0 * np.pi, size=(_N_MODES, spec.d))
    n = np.arange(lo, hi, dtype=np.int64)
    x = (n % X) / X
    y = ((n // X) % Y) / Y
    t = (n // (X * Y)) / T
    wc = amp * np.cos(ph)                                   # [8, d]
    ws = amp * np.sin(ph)
    out = np.zeros((hi - lo, spec.d), dtype=np.float64)
    tmp = np.empty_like(out)
    for f in range(_N_MODES):
        theta = 2.0 * np.pi * (u[f, 0] * t + u[f, 1] * y + u[f, 2] * x)   # [n]
        # a cos(theta + ph) = (a cos ph) cos theta - (a sin ph) sin theta
        np.multiply(np.cos(theta)[:, None], wc[f][None, :], out=tmp)
        out += tmp
        np.multiply(np.sin(theta)[:, None], ws[f][None, :], out=tmp)
        out -= tmp
    return out.astype(np.float32)


def head_field(spec: Spec, b: int, h: int):
    """The Q/K field of one head, float32 [N, d] (kind "fourier" only)."""
    return _field(spec, (spec.cfg_id, 10, b, h))


def q_block_bits(spec: Spec, b: int, h: int, i: int, attempt: int, field=None):
    """Q tokens of query block i of one head under redraw `attempt` >= 1, bf16 bits.

    `field` may pass the head's precomputed Q/K field rows for the block.
    """
    if attempt < 1:
        raise ValueError("attempt 0 is the head's main noise stream")
    lo = i * spec.block
    hi = min(lo + spec.block, spec.N)
    noise = _rng(spec.cfg_id, 0, b, h, i, attempt).standard_normal((hi - lo, spec.d), dtype=np.float32)
    if spec.kind == "iid":
        return f32_to_bf16_bits(noise)
    if field is None:
        field = _field(spec, (spec.cfg_id, 10, b, h), lo, hi)
    return f32_to_bf16_bits(field + _NOISE * noise)


def generate_head(spec: Spec, b: int, h: int, tensors=("q", "k", "v"), repairs=None):
    """One (batch, head) slice: dict name -> uint16 bf16 bits [N, d]."""
    out = {}
    fields = {}
    for name in tensors:
        tid = _TENSOR_ID[name]
        noise = _rng(spec.cfg_id, tid, b, h).standard_normal((spec.N, spec.d), dtype=np.float32)
        if spec.kind == "iid":
            x32 = noise
        else:
            fid = 11 if name == "v" else 10
            if fid not in fields:
                fields[fid] = _field(spec, (spec.cfg_id, fid, b, h))
            x32 = fields[fid] + _NOISE * noise
        bits = f32_to_bf16_bits(x32)
        if name == "q" and repairs:
            for (rb, rh, i), attempt in repairs.items():
                if rb != b or rh != h or attempt == 0:
                    continue
                lo = i * spec.block
                hi = min(lo + spec.block, spec.N)
                fld = fields[10][lo:hi] if spec.kind == "fourier" else None
                bits[lo:hi] = q_block_bits(spec, b, h, i, attempt, fld)
        out[name] = bits
    return out


def generate(spec: Spec, tensors=("q", "k", "v"), repairs="stored", threads=None):
    """Full tensors: dict name -> uint16 bf16 bits [B, H, N, d].

    repairs: "stored" reads the committed table for spec.cfg_id (an empty table
    if none is stored), None applies none, or pass a dict (b, h, i) -> attempt.
    """
    if isinstance(repairs, str):
        repairs = load_repairs(spec.cfg_id)
    out = {name: np.empty((spec.B, spec.H, spec.N, spec.d), dtype=np.uint16) for name in tensors}

    def work(bh):
        b, h = bh
        part = generate_head(spec, b, h, tensors, repairs)
        for name in tensors:
            out[name][b, h] = part[name]

    jobs = [(b, h) for b in range(spec.B) for h in range(spec.H)]
    if threads is None:
        threads = min(16, os.cpu_count() or 1)
    if threads <= 1 or len(jobs) == 1:
        for j in jobs:
            work(j)
    else:
        with ThreadPoolExecutor(max_workers=threads) as ex:
            list(ex.map(work, jobs))
    return out


def repair_path(cfg_id: int) -> str:
    return os.path.join(_REPAIR_DIR, f"cfg{cfg_id}.json")


def load_repairs(cfg_id: int):
    """The stored margin-repair table for a workload seed: {(b, h, i): attempt}."""
    path = repair_path(cfg_id)
    if not os.path.exists(path):
        return {}
    with open(path) as f:
        doc = json.load(f)
    return {tuple(int(x) for x in key.split(",")): int(a) for key, a in doc["repairs"].items()}


def save_repairs(cfg_id: int, repairs, meta):
    doc = {"meta": meta,
           "repairs": {f"{b},{h},{i}": int(a) for (b, h, i), a in sorted(repairs.items()) if a}}
    os.makedirs(_REPAIR_DIR, exist_ok=True)
    with open(repair_path(cfg_id), "w") as f:
        json.dump(doc, f, indent=1, sort_keys=True)
        f.write("\n")
