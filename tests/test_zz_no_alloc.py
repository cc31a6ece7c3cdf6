"""The allocation-free pool/classify entry point against the workspace one.

sla_pool_classify_noalloc runs the same kernels as sla_pool_classify with the
library's static device scratch in place of the caller's workspace, a chunk of
heads at a time.  Both are called through the C ABI on the same seeded inputs;
the class maps and the pooled Q/K must be identical bit for bit.  Two calls in
a row share the scratch, the second on a smaller input; the first spans two
head chunks (one head at 4096 key blocks fills most of the scratch).
"""

from fractions import Fraction as F

import numpy as np
import pytest
import torch

import block_sparse_attention_meanpool_amd as sla
from gpu_util import say, to_dev
from synth.generate import f32_to_bf16_bits

pytestmark = pytest.mark.gpu


def _inputs(B, H, N, d, seed):
    g = np.random.default_rng(seed)
    q = f32_to_bf16_bits(g.standard_normal((B, H, N, d), dtype=np.float32))
    k = f32_to_bf16_bits(g.standard_normal((B, H, N, d), dtype=np.float32))
    return to_dev(q), to_dev(k)


def _compare(B, H, N, d, block, mode, keep, marg, thr, seed, pooled_out):
    q, k = _inputs(B, H, N, d, seed)
    nb = sla.num_blocks(N, block)
    kc, km = sla.counts_for(mode, nb, keep, marg)
    dev = q.device
    pooled = lambda: (torch.empty((B, H, nb, d), dtype=torch.float32, device=dev) for _ in range(2))
    qp0, kp0 = pooled() if pooled_out else (None, None)
    qp1, kp1 = pooled() if pooled_out else (None, None)
    cls_ref = sla.sla_pool_classify(q, k, block, mode, kc, km, thr, q_pool=qp0, k_pool=kp0)
    cls = torch.full((B, H, nb, nb), 7, dtype=torch.uint8, device=dev)
    sla.sla_pool_classify_noalloc(q, k, block, mode, kc, km, thr, q_pool=qp1, k_pool=kp1, cls=cls)
    torch.cuda.synchronize()
    assert torch.equal(cls, cls_ref), f"class maps differ at {(cls != cls_ref).sum().item()} pairs"
    if pooled_out:
        assert torch.equal(qp0.view(torch.int32), qp1.view(torch.int32))
        assert torch.equal(kp0.view(torch.int32), kp1.view(torch.int32))
    counts = torch.bincount(cls.flatten().long(), minlength=3).tolist()
    say(f"  B={B} H={H} N={N} d={d} block={block} {mode}: class maps identical "
        f"(skip/marginal/critical = {counts}){', pooled Q/K identical' if pooled_out else ''}")


def test_noalloc_matches_workspace_entry_point():
    per_head = 4096 * 4096 * 4 + 2 * 4096 * 64 * 4
    scratch = sla.lib().sla_pool_classify_noalloc_scratch_bytes()
    say(f"[no-alloc] static scratch {scratch} B; one head at nb = 4096, d = 64 needs {per_head} B")
    assert scratch // per_head == 1  # the first call below runs as two head chunks
    # 1) two heads of 4096 key blocks: two chunks, three-way split
    _compare(1, 2, 4096 * 64, 64, 64, "sla3", F(1, 50), F(1, 20), 0.0, seed=1, pooled_out=False)
    # 2) a smaller input right after: top-k with the pooled outputs written by the caller
    _compare(2, 3, 1000, 128, 128, "topk", F(1, 4), None, 0.0, seed=2, pooled_out=True)
    # 3) and a CDF cut with a ragged last block, sharing the same scratch again
    _compare(1, 4, 8000, 64, 64, "cdf", None, None, 0.1, seed=3, pooled_out=False)


def test_noalloc_rejects_bad_arguments_before_launch():
    lib = sla.lib()
    P = lambda x: None if x is None else __import__("ctypes").c_void_p(x)
    good, odd = 0x10000, 0x10008
    call = lambda q=good, d=64, kc=4, mode=0: lib.sla_pool_classify_noalloc(
        P(q), P(good), 1, 2, 1024, d, 64, mode, kc, 0, 0.0, 0.125, None, None, P(good), None)
    assert call(q=None) == -1
    assert call(d=96) == -2
    assert call(q=odd) == -3
    assert call(kc=0) == -1
    assert call(mode=9) == -1
