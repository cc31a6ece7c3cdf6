"""Helpers for the GPU parity tests: device transfer of bf16 bits, seeded
small workloads with margin repairs from the oracle, and the comparison bars.

Bars (the ones stated for this path): block masks and lists bit-exact;
outputs within max-abs 2e-2 and relative L2 5e-3 of the fp64 oracle, evaluated
on the kernels' fp32 outputs before the final bf16 rounding; the bf16 output
must equal the round-to-nearest-even of that fp32 output.
"""

import math
import sys

import numpy as np
import torch

from oracle import sla as osla
from oracle.make_repairs import boundaries_for, repair_head
from synth import generate

MAX_ABS = 2e-2
REL_L2 = 5e-3
# The kernel's softmax normaliser sums the same bf16-rounded probabilities
# that enter the P.V product (so constant V gives exactly V).  bf16 keeps 8
# significant bits, so round-to-nearest-even moves each term by at most 2^-8
# relative, and ln(sum) by at most ln(1 + 2^-8) < 2^-8, plus fp32 error.
BF16_U = 2.0 ** -8
LSE_MAX_ABS = BF16_U + 5e-4
# The LSE error is the log of the normaliser's relative error, a weighted mean
# sum_i w_i delta_i of the roundings (weights w_i = p_i / sum p, |delta_i| <=
# 2^-8, independent, mean square at most 2^-16 / 3); its mean square is at
# most (2^-16 / 3) sum_i w_i^2 <= 2^-16 / 3.  So the root-mean-square error
# over the rows is held to 2^-8 / sqrt(3), plus the same fp32 slack scaled down.
LSE_RMS = BF16_U / math.sqrt(3.0) + 1e-4


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def to_dev(bits):
    """uint16 bf16 bits (numpy) -> torch.bfloat16 on cuda:0."""
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).to("cuda:0")


def bits_of(t):
    """torch.bfloat16 -> uint16 bits (numpy)."""
    return t.detach().cpu().contiguous().view(torch.int16).numpy().view(np.uint16)


def f64(t):
    return t.detach().cpu().to(torch.float64).numpy()


def small_inputs(spec):
    """Generate a small workload with margin repairs computed by the oracle."""
    cuts, thr = boundaries_for([spec], spec.nb)
    repairs = {}
    for b in range(spec.B):
        for h in range(spec.H):
            repairs.update(repair_head(spec, cuts, thr, b, h))
    return generate(spec, repairs=repairs, threads=1)


def counts(spec):
    sel = "sla3" if spec.mode == "maskin" else spec.mode
    return osla.selection_counts(sel, spec.nb, spec.keep, spec.marg)


def check_close(got, want, what, max_abs=MAX_ABS, rel_l2=REL_L2):
    got = np.asarray(got, dtype=np.float64)
    want = np.asarray(want, dtype=np.float64)
    assert got.shape == want.shape, (what, got.shape, want.shape)
    diff = np.abs(got - want)
    mabs = float(diff.max()) if diff.size else 0.0
    nrm = float(np.linalg.norm(want))
    rel = float(np.linalg.norm(got - want) / nrm) if nrm > 0 else float(np.linalg.norm(got - want))
    say(f"  {what}: max|d| = {mabs:.3e}, rel-L2 = {rel:.3e}, max|ref| = {float(np.abs(want).max()):.3f}")
    assert mabs <= max_abs, f"{what}: max-abs {mabs} > {max_abs}"
    assert rel <= rel_l2, f"{what}: rel-L2 {rel} > {rel_l2}"
    return mabs, rel


def check_lse(got, want, what="LSE"):
    """LSE against the oracle: every finite entry within LSE_MAX_ABS, their
    root-mean-square error within LSE_RMS; -inf exactly where the oracle has it."""
    got = np.asarray(got, dtype=np.float64)
    want = np.asarray(want, dtype=np.float64)
    assert got.shape == want.shape, (what, got.shape, want.shape)
    fin = np.isfinite(want)
    assert np.array_equal(np.isfinite(got), fin), f"{what}: -inf rows differ"
    assert (got[~fin] == want[~fin]).all(), f"{what}: non-finite values differ"
    diff = got[fin] - want[fin]
    mabs = float(np.abs(diff).max()) if diff.size else 0.0
    rms = float(np.sqrt(np.mean(diff ** 2))) if diff.size else 0.0
    say(f"  {what}: max|d| = {mabs:.3e}, rms = {rms:.3e} (bars {LSE_MAX_ABS:.2e}, {LSE_RMS:.2e})")
    assert mabs <= LSE_MAX_ABS, f"{what}: max-abs {mabs} > {LSE_MAX_ABS}"
    assert rms <= LSE_RMS, f"{what}: rms {rms} > {LSE_RMS}"
    return mabs, rms


def rne_bf16_bits(x32):
    """Round float32 values to bf16 bits (nearest even), independently of the kernels."""
    u = np.ascontiguousarray(x32, dtype=np.float32).view(np.uint32)
    return ((u + np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))) >> np.uint32(16)).astype(np.uint16)


def scale_of(d):
    return 1.0 / math.sqrt(d)
