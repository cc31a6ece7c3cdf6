"""GPU mask recall (sla_mask_recall) against the oracle's fp64 definition.

recall = exp(LSE_kept - LSE_all); each GPU LSE is within 2^-8 + 5e-4 of its
exact value (the LSE bar of the forward tests), so recall is within a
relative exp(2 (2^-8 + 5e-4)) - 1 of the oracle's; rows with no kept tile
are exactly 0.
"""

from fractions import Fraction as F

import numpy as np
import pytest
import torch

import block_sparse_attention_meanpool_amd as sla
from gpu_util import LSE_MAX_ABS, say, to_dev
from oracle import sla as osla
from synth import generate
from synth.configs import Spec

pytestmark = pytest.mark.gpu

REL = float(np.exp(2 * LSE_MAX_ABS) - 1)


def _check(got, want, what):
    empty = want == 0
    assert not got[empty].any(), what
    rel = np.abs(got[~empty] / want[~empty] - 1)
    say(f"  {what}: max rel = {rel.max():.3e} (bar {REL:.3e}), mean recall {want.mean():.4f}")
    assert rel.max() <= REL


@pytest.mark.parametrize("d,block", [(128, 128), (64, 64), (128, 64), (64, 128)])
def test_recall_small(d, block):
    spec = Spec(401, "recall", B=1, H=2, N=1000, d=d, block=block, kind="fourier",
                grid=(10, 10, 10), mode="topk", keep=F(1, 4))
    data = generate(spec, repairs=None, threads=1)
    nb = spec.nb
    g = np.random.default_rng(5)
    cls = np.where(g.random((1, 2, nb, nb)) < 0.3, osla.CRITICAL, osla.SKIP).astype(np.uint8)
    cls[0, 0, 0] = osla.CRITICAL     # everything kept
    cls[0, 0, 1] = osla.SKIP         # nothing kept
    idx, cnt = osla.index_lists(cls, osla.CRITICAL, nb)
    q, k = to_dev(data["q"]), to_dev(data["k"])
    r = sla.sla_mask_recall(q, k, block, torch.from_numpy(idx).cuda(), torch.from_numpy(cnt).cuda())
    torch.cuda.synchronize()
    want = osla.mask_recall(osla.bf16_to_f64(data["q"]), osla.bf16_to_f64(data["k"]), cls, block)
    _check(r.cpu().numpy().astype(np.float64), want, f"recall d={d} block={block}")


def test_recall_workload_head():
    from synth import CONFIGS
    spec = CONFIGS["wan1p3b"]
    say(f"[recall] {spec.name}: one head checked in full")
    data = generate(spec)
    q, k = to_dev(data["q"]), to_dev(data["k"])
    kc, km = osla.selection_counts("sla3", spec.nb, spec.keep, spec.marg)
    cls = sla.sla_pool_classify(q, k, spec.block, "sla3", kc, km)
    ci, cc, _, _ = sla.sla_block_mask(cls, kc)
    r = sla.sla_mask_recall(q, k, spec.block, ci, cc)
    torch.cuda.synchronize()
    h = 5
    want = osla.mask_recall(osla.bf16_to_f64(data["q"][:, h:h + 1]),
                            osla.bf16_to_f64(data["k"][:, h:h + 1]),
                            cls.cpu().numpy()[:, h:h + 1], spec.block)
    _check(r[:, h:h + 1].cpu().numpy().astype(np.float64), want, f"recall head {h}")
