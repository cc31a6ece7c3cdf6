"""The path captured in a HIP graph (torch.cuda.CUDAGraph): every replay, with
eager work and synchronisation between replays, must reproduce the eager
results bit for bit.  The library clears memory with a fill kernel (no
hipMemsetAsync) and allocates nothing, so its calls can be captured."""

from fractions import Fraction as F

import numpy as np
import pytest
import torch

import block_sparse_attention_meanpool_amd as sla
from gpu_util import to_dev
from synth import generate
from synth.configs import Spec

pytestmark = pytest.mark.gpu

SPEC = Spec(601, "graph", B=1, H=3, N=2000, d=128, block=128, kind="fourier", grid=(5, 20, 20),
            mode="sla3", keep=F(2, 16), marg=F(3, 16))


def _bits(t):
    return t.view(torch.int16) if t.dtype == torch.bfloat16 else t.view(torch.int32)


def test_forward_and_backward_in_a_graph():
    data = generate(SPEC, repairs=None, threads=1)
    q, k, v = (to_dev(data[t]) for t in "qkv")
    g = torch.Generator(device="cuda").manual_seed(3)
    d_o = torch.randn(q.shape, generator=g, device="cuda").to(torch.bfloat16)
    B, H, N, d, b, nb = SPEC.B, SPEC.H, SPEC.N, SPEC.d, SPEC.block, SPEC.nb
    kc, km = sla.counts_for("sla3", nb, SPEC.keep, SPEC.marg)
    lib = sla.lib()
    bufs = {
        "cls": torch.empty((B, H, nb, nb), dtype=torch.uint8, device="cuda"),
        "ws": torch.empty(lib.sla_pool_classify_ws_bytes(B, H, N, d, b, 0), dtype=torch.uint8,
                          device="cuda"),
        "ci": torch.empty((B, H, nb, kc), dtype=torch.int32, device="cuda"),
        "cc": torch.empty((B, H, nb), dtype=torch.int32, device="cuda"),
        "mi": torch.empty((B, H, nb, km), dtype=torch.int32, device="cuda"),
        "mc": torch.empty((B, H, nb), dtype=torch.int32, device="cuda"),
        "lin": torch.empty(lib.sla_linear_branch_ws_bytes(B, H, N, d, b), dtype=torch.uint8,
                           device="cuda"),
        "o": torch.empty(q.shape, dtype=torch.bfloat16, device="cuda"),
        "o_s": torch.empty(q.shape, dtype=torch.float32, device="cuda"),
        "lse": torch.empty((B, H, N), dtype=torch.float32, device="cuda"),
        "bws": torch.empty(lib.sla_sparse_attn_bwd_ws_bytes(B, H, N, d, b), dtype=torch.uint8,
                           device="cuda"),
        "lbws": torch.empty(lib.sla_linear_branch_bwd_ws_bytes(B, H, N, d, b), dtype=torch.uint8,
                            device="cuda"),
        "dq": torch.empty(q.shape, dtype=torch.float32, device="cuda"),
        "dk": torch.empty(q.shape, dtype=torch.float32, device="cuda"),
        "dv": torch.empty(q.shape, dtype=torch.float32, device="cuda"),
    }
    x = bufs

    def layer():
        sla.sla_pool_classify(q, k, b, "sla3", kc, km, cls=x["cls"], ws=x["ws"])
        sla.sla_block_mask(x["cls"], kc, km, x["ci"], x["cc"], x["mi"], x["mc"])
        sla.sla_linear_branch_prepare(k, v, b, x["mi"], x["mc"], ws=x["lin"])
        sla.sla_sparse_linear_attn_fwd(q, k, v, b, x["ci"], x["cc"], x["lin"], o=x["o"])
        sla.sla_sparse_attn_fwd(q, k, v, b, x["ci"], x["cc"], o_s=x["o_s"], lse=x["lse"])
        sla.sla_sparse_attn_bwd(q, k, v, b, x["ci"], x["cc"], x["o_s"], x["lse"], d_o, dq=x["dq"],
                                dk=x["dk"], dv=x["dv"], ws=x["bws"])
        sla.sla_linear_branch_bwd(q, k, v, b, x["mi"], x["mc"], d_o, x["lin"], x["dq"], x["dk"],
                                  x["dv"], ws=x["lbws"])

    outs = ("cls", "ci", "cc", "mi", "mc", "o", "lse", "dq", "dk", "dv")
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        layer()                                 # eager, on the capture stream
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    eager = {n: x[n].clone() for n in outs}

    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        layer()
    for rep in range(3):
        for n in outs:                          # clobber every output between replays
            x[n].zero_()
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for n in outs:
            assert torch.equal(_bits(x[n]) if x[n].dtype in (torch.bfloat16, torch.float32) else x[n],
                               _bits(eager[n]) if eager[n].dtype in (torch.bfloat16, torch.float32)
                               else eager[n]), (rep, n)
