"""The shader-clock probe (a measurement aid of the benchmark), through the C ABI:
alone it waits the requested span of the fixed-rate counter and reports a clock
within the chip's range; beside a long kernel on another stream it still ends
and reports a clock in that range (the clock the chip runs that kernel at)."""

import pytest
import torch

import block_sparse_attention_meanpool_amd as sla
from gpu_util import say

pytestmark = pytest.mark.gpu


def test_clock_probe_alone():
    span = 3000
    out, hz = sla.sla_clock_probe(span)
    torch.cuda.synchronize()
    c0, c1, r0, r1 = out.cpu().tolist()
    waited = (r1 - r0) / hz
    ghz = sla.probe_clock_hz(out, hz) / 1e9
    say(f"[clock] fixed rate {hz / 1e6:.1f} MHz, waited {waited * 1e3:.3f} ms, clock {ghz:.3f} GHz")
    assert hz > 0
    assert 0.9 * span * 1e-6 <= waited <= 2.0 * span * 1e-6
    assert c1 > c0
    assert 0.3 <= ghz <= 3.0


def test_clock_probe_beside_a_kernel():
    B, H, N, d, b = 1, 8, 8192, 128, 128
    g = torch.Generator().manual_seed(1)
    q, k, v = (torch.randn((B, H, N, d), generator=g).to(torch.bfloat16).cuda() for _ in range(3))
    o = torch.empty((B, H, N, d), dtype=torch.bfloat16, device="cuda")
    sla.sla_dense_attn_fwd(q, k, v, b, o=o)
    torch.cuda.synchronize()
    side = torch.cuda.Stream()
    out, hz = sla.sla_clock_probe(2000, stream=side)
    for _ in range(8):
        sla.sla_dense_attn_fwd(q, k, v, b, o=o)
    torch.cuda.synchronize()
    ghz = sla.probe_clock_hz(out, hz) / 1e9
    say(f"[clock] beside the dense kernel: {ghz:.3f} GHz")
    assert 0.3 <= ghz <= 3.0
