"""Thin Python binding of libsla.so: argument marshalling only.

Each function carries the name of the C entry point it calls and takes torch
tensors as device memory (plus the current HIP stream).  Every step of the
computation runs in the library's kernels; nothing here computes on tensor
data, and there is no fallback: if the library is not built or no GPU is
visible, the calls raise.
"""

import ctypes
import math
import os
from fractions import Fraction

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libsla.so")

SEL_TOPK, SEL_CDF, SEL_SLA3 = 0, 1, 2
MODES = {"topk": SEL_TOPK, "cdf": SEL_CDF, "sla3": SEL_SLA3}
CLS_SKIP, CLS_MARGINAL, CLS_CRITICAL = 0, 1, 2
FLAG_BAD_CLASS, FLAG_OVERFLOW = 1, 2

_lib = None

_P = ctypes.c_void_p
_I64 = ctypes.c_int64
_I32 = ctypes.c_int32
_F = ctypes.c_float
_SZ = ctypes.c_size_t

_SIGS = {
    "sla_pool_classify": (_I32, [_P, _P, _I64, _I64, _I64, _I64, _I32, _I32, _I32, _I32, _F, _F,
                                 _P, _P, _P, _P, _SZ, _P]),
    "sla_pool_classify_ws_bytes": (_SZ, [_I64, _I64, _I64, _I64, _I32, _I32]),
    "sla_pool_classify_noalloc": (_I32, [_P, _P, _I64, _I64, _I64, _I64, _I32, _I32, _I32, _I32,
                                         _F, _F, _P, _P, _P, _P]),
    "sla_pool_classify_noalloc_scratch_bytes": (_SZ, []),
    "sla_block_mask": (_I32, [_P, _I64, _I64, _I64, _I64, _P, _P, _I32, _P, _P, _I32, _P, _P]),
    "sla_sparse_attn_fwd": (_I32, [_P, _P, _P, _I64, _I64, _I64, _I64, _I32, _P, _P, _I32, _F,
                                   _P, _I32, _P, _P]),
    "sla_linear_branch_fwd": (_I32, [_P, _P, _P, _I64, _I64, _I64, _I64, _I32, _P, _P, _I32, _P,
                                     _P, _SZ, _P]),
    "sla_linear_branch_ws_bytes": (_SZ, [_I64, _I64, _I64, _I64, _I32]),
    "sla_linear_branch_prepare": (_I32, [_P, _P, _I64, _I64, _I64, _I64, _I32, _P, _P, _I32, _P,
                                         _SZ, _P]),
    "sla_sparse_linear_attn_fwd": (_I32, [_P, _P, _P, _I64, _I64, _I64, _I64, _I32, _P, _P, _I32,
                                          _F, _P, _SZ, _P, _I32, _P, _P]),
    "sla_combine": (_I32, [_P, _I32, _P, _P, _I64, _P]),
    "sla_sparse_attn_bwd": (_I32, [_P, _P, _P, _I64, _I64, _I64, _I64, _I32, _P, _P, _I32, _F, _P,
                                   _I32, _P, _P, _P, _P, _P, _P, _SZ, _P]),
    "sla_sparse_attn_bwd_ws_bytes": (_SZ, [_I64, _I64, _I64, _I64, _I32]),
    "sla_linear_branch_bwd": (_I32, [_P, _P, _P, _I64, _I64, _I64, _I64, _I32, _P, _P, _I32, _P, _P,
                                     _SZ, _P, _P, _P, _P, _SZ, _P]),
    "sla_linear_branch_bwd_ws_bytes": (_SZ, [_I64, _I64, _I64, _I64, _I32]),
    "sla_mask_recall": (_I32, [_P, _P, _I64, _I64, _I64, _I64, _I32, _P, _P, _I32, _F, _P, _P, _SZ,
                               _P]),
    "sla_mask_recall_ws_bytes": (_SZ, [_I64, _I64, _I64, _I64, _I32]),
    "sla_tile_permute": (_I32, [_P, _P, _I64, _I64, _I64, _I64, _I64, _I64, _I32, _P, _I32, _P]),
    "sla_dense_attn_fwd": (_I32, [_P, _P, _P, _I64, _I64, _I64, _I64, _I32, _F, _P, _I32, _P, _P]),
    "sla_status_string": (ctypes.c_char_p, [_I32]),
    "sla_version": (_I32, []),
}
EXPORTS = tuple(_SIGS)


class SlaError(RuntimeError):
    def __init__(self, name, status):
        super().__init__(f"{name} failed: {sla_status_string(status)} (status {status})")
        self.status = status


def lib():
    """Load libsla.so once; raise if it is missing."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is not built; run "
                               "`python -m block_sparse_attention_meanpool_amd.build`")
        h = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in _SIGS.items():
            fn = getattr(h, name)
            fn.restype = res
            fn.argtypes = args
        _lib = h
    return _lib


def sla_status_string(status):
    return lib().sla_status_string(int(status)).decode()


def sla_version():
    return lib().sla_version()


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream):
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


def _call(name, *args):
    st = getattr(lib(), name)(*args)
    if st != 0:
        raise SlaError(name, st)


def _dev(t, dtype, name):
    if not isinstance(t, torch.Tensor) or not t.is_cuda:
        raise ValueError(f"{name} must be a GPU tensor")
    if t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype}, got {t.dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    return t


def num_blocks(N, block):
    return -(-N // block)


def count_from_fraction(frac, nkb):
    """A keep fraction of nkb key blocks as a block count: ceil, at least one."""
    return max(1, math.ceil(Fraction(frac) * nkb))


def counts_for(mode, nkb, keep=None, marg=None):
    """(k_crit, k_marg) for a selection rule given as fractions of the key blocks."""
    if mode == "cdf":
        return 0, 0
    kc = count_from_fraction(keep, nkb)
    if mode == "topk" or marg is None or Fraction(marg) == 0:
        return kc, 0
    total = min(nkb, math.ceil((Fraction(keep) + Fraction(marg)) * nkb))
    return kc, max(0, total - kc)


# ---------------------------------------------------------------------------
# one wrapper per C entry point
# ---------------------------------------------------------------------------

def sla_pool_classify(q, k, block, mode, k_crit=0, k_marg=0, thr=0.0, scale=None, q_pool=None,
                      k_pool=None, cls=None, ws=None, stream=None):
    _dev(q, torch.bfloat16, "q")
    _dev(k, torch.bfloat16, "k")
    B, H, N, d = q.shape
    nb = num_blocks(N, block)
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    if cls is None:
        cls = torch.empty((B, H, nb, nb), dtype=torch.uint8, device=q.device)
    need = lib().sla_pool_classify_ws_bytes(B, H, N, d, block, int(q_pool is not None))
    if ws is None:
        ws = torch.empty(max(need, 1), dtype=torch.uint8, device=q.device)
    _call("sla_pool_classify", _ptr(q), _ptr(k), B, H, N, d, block, MODES.get(mode, mode),
          int(k_crit), int(k_marg), float(thr), float(scale), _ptr(q_pool), _ptr(k_pool),
          _ptr(cls), _ptr(ws), ws.numel() * ws.element_size(), _stream(stream))
    return cls


def sla_pool_classify_noalloc(q, k, block, mode, k_crit=0, k_marg=0, thr=0.0, scale=None,
                              q_pool=None, k_pool=None, cls=None, stream=None):
    """sla_pool_classify without a workspace (the library's static device
    scratch instead): for callers that cannot allocate.  Pass `cls` (and the
    pooled outputs, if wanted) to make the whole call allocation-free."""
    _dev(q, torch.bfloat16, "q")
    _dev(k, torch.bfloat16, "k")
    B, H, N, d = q.shape
    nb = num_blocks(N, block)
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    if cls is None:
        cls = torch.empty((B, H, nb, nb), dtype=torch.uint8, device=q.device)
    _call("sla_pool_classify_noalloc", _ptr(q), _ptr(k), B, H, N, d, block, MODES.get(mode, mode),
          int(k_crit), int(k_marg), float(thr), float(scale), _ptr(q_pool), _ptr(k_pool),
          _ptr(cls), _stream(stream))
    return cls


def sla_block_mask(cls, kc_max, km_max=0, crit_idx=None, crit_cnt=None, marg_idx=None,
                   marg_cnt=None, err_flag=None, stream=None):
    _dev(cls, torch.uint8, "cls")
    B, H, nqb, nkb = cls.shape
    dev = cls.device
    if crit_idx is None:
        crit_idx = torch.empty((B, H, nqb, kc_max), dtype=torch.int32, device=dev)
        crit_cnt = torch.empty((B, H, nqb), dtype=torch.int32, device=dev)
    if km_max and marg_idx is None:
        marg_idx = torch.empty((B, H, nqb, km_max), dtype=torch.int32, device=dev)
        marg_cnt = torch.empty((B, H, nqb), dtype=torch.int32, device=dev)
    _call("sla_block_mask", _ptr(cls), B, H, nqb, nkb, _ptr(crit_idx), _ptr(crit_cnt), int(kc_max),
          _ptr(marg_idx), _ptr(marg_cnt), int(km_max), _ptr(err_flag), _stream(stream))
    return crit_idx, crit_cnt, marg_idx, marg_cnt


def sla_sparse_attn_fwd(q, k, v, block, crit_idx, crit_cnt, scale=None, o_s=None, o_fp32=True,
                        lse=None, want_lse=False, stream=None):
    for t, n in ((q, "q"), (k, "k"), (v, "v")):
        _dev(t, torch.bfloat16, n)
    _dev(crit_idx, torch.int32, "crit_idx")
    _dev(crit_cnt, torch.int32, "crit_cnt")
    B, H, N, d = q.shape
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    if o_s is None:
        o_s = torch.empty(q.shape, dtype=torch.float32 if o_fp32 else torch.bfloat16, device=q.device)
    if want_lse and lse is None:
        lse = torch.empty((B, H, N), dtype=torch.float32, device=q.device)
    _call("sla_sparse_attn_fwd", _ptr(q), _ptr(k), _ptr(v), B, H, N, d, block, _ptr(crit_idx),
          _ptr(crit_cnt), crit_idx.shape[-1], float(scale), _ptr(o_s),
          int(o_s.dtype == torch.float32), _ptr(lse), _stream(stream))
    return o_s, lse


def sla_dense_attn_fwd(q, k, v, block, scale=None, o=None, o_fp32=False, lse=None, want_lse=False,
                       stream=None):
    for t, n in ((q, "q"), (k, "k"), (v, "v")):
        _dev(t, torch.bfloat16, n)
    B, H, N, d = q.shape
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    if o is None:
        o = torch.empty(q.shape, dtype=torch.float32 if o_fp32 else torch.bfloat16, device=q.device)
    if want_lse and lse is None:
        lse = torch.empty((B, H, N), dtype=torch.float32, device=q.device)
    _call("sla_dense_attn_fwd", _ptr(q), _ptr(k), _ptr(v), B, H, N, d, block, float(scale), _ptr(o),
          int(o.dtype == torch.float32), _ptr(lse), _stream(stream))
    return o, lse


def sla_linear_branch_fwd(q, k, v, block, marg_idx, marg_cnt, o_lin=None, ws=None, stream=None):
    for t, n in ((q, "q"), (k, "k"), (v, "v")):
        _dev(t, torch.bfloat16, n)
    _dev(marg_idx, torch.int32, "marg_idx")
    _dev(marg_cnt, torch.int32, "marg_cnt")
    B, H, N, d = q.shape
    if o_lin is None:
        o_lin = torch.empty(q.shape, dtype=torch.float32, device=q.device)
    need = lib().sla_linear_branch_ws_bytes(B, H, N, d, block)
    if ws is None:
        ws = torch.empty(max(need, 1), dtype=torch.uint8, device=q.device)
    _call("sla_linear_branch_fwd", _ptr(q), _ptr(k), _ptr(v), B, H, N, d, block, _ptr(marg_idx),
          _ptr(marg_cnt), marg_idx.shape[-1], _ptr(o_lin), _ptr(ws), ws.numel() * ws.element_size(),
          _stream(stream))
    return o_lin


def sla_linear_branch_prepare(k, v, block, marg_idx, marg_cnt, ws=None, stream=None):
    for t, n in ((k, "k"), (v, "v")):
        _dev(t, torch.bfloat16, n)
    _dev(marg_idx, torch.int32, "marg_idx")
    _dev(marg_cnt, torch.int32, "marg_cnt")
    B, H, N, d = k.shape
    need = lib().sla_linear_branch_ws_bytes(B, H, N, d, block)
    if ws is None:
        ws = torch.empty(max(need, 1), dtype=torch.uint8, device=k.device)
    _call("sla_linear_branch_prepare", _ptr(k), _ptr(v), B, H, N, d, block, _ptr(marg_idx),
          _ptr(marg_cnt), marg_idx.shape[-1], _ptr(ws), ws.numel() * ws.element_size(),
          _stream(stream))
    return ws


def sla_sparse_linear_attn_fwd(q, k, v, block, crit_idx, crit_cnt, lin_ws, scale=None, o=None,
                               o_fp32=False, lse=None, want_lse=False, stream=None):
    for t, n in ((q, "q"), (k, "k"), (v, "v")):
        _dev(t, torch.bfloat16, n)
    _dev(crit_idx, torch.int32, "crit_idx")
    _dev(crit_cnt, torch.int32, "crit_cnt")
    _dev(lin_ws, torch.uint8, "lin_ws")
    B, H, N, d = q.shape
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    if o is None:
        o = torch.empty(q.shape, dtype=torch.float32 if o_fp32 else torch.bfloat16, device=q.device)
    if want_lse and lse is None:
        lse = torch.empty((B, H, N), dtype=torch.float32, device=q.device)
    _call("sla_sparse_linear_attn_fwd", _ptr(q), _ptr(k), _ptr(v), B, H, N, d, block,
          _ptr(crit_idx), _ptr(crit_cnt), crit_idx.shape[-1], float(scale), _ptr(lin_ws),
          lin_ws.numel(), _ptr(o), int(o.dtype == torch.float32), _ptr(lse), _stream(stream))
    return o, lse


def sla_sparse_attn_bwd(q, k, v, block, crit_idx, crit_cnt, o_s, lse, d_o, scale=None, dq=None,
                        dk=None, dv=None, ws=None, stream=None):
    for t, n in ((q, "q"), (k, "k"), (v, "v"), (d_o, "d_o")):
        _dev(t, torch.bfloat16, n)
    _dev(crit_idx, torch.int32, "crit_idx")
    _dev(crit_cnt, torch.int32, "crit_cnt")
    _dev(lse, torch.float32, "lse")
    B, H, N, d = q.shape
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    dq, dk, dv = (torch.empty(q.shape, dtype=torch.float32, device=q.device) if t is None else t
                  for t in (dq, dk, dv))
    need = lib().sla_sparse_attn_bwd_ws_bytes(B, H, N, d, block)
    if ws is None:
        ws = torch.empty(max(need, 1), dtype=torch.uint8, device=q.device)
    _call("sla_sparse_attn_bwd", _ptr(q), _ptr(k), _ptr(v), B, H, N, d, block, _ptr(crit_idx),
          _ptr(crit_cnt), crit_idx.shape[-1], float(scale), _ptr(o_s),
          int(o_s.dtype == torch.float32), _ptr(lse), _ptr(d_o), _ptr(dq), _ptr(dk), _ptr(dv),
          _ptr(ws), ws.numel() * ws.element_size(), _stream(stream))
    return dq, dk, dv


def sla_linear_branch_bwd(q, k, v, block, marg_idx, marg_cnt, d_o, lin_ws, dq, dk, dv, ws=None,
                          stream=None):
    """Adds the linear branch's gradients into dq, dk, dv (fp32)."""
    for t, n in ((q, "q"), (k, "k"), (v, "v"), (d_o, "d_o")):
        _dev(t, torch.bfloat16, n)
    _dev(marg_idx, torch.int32, "marg_idx")
    _dev(marg_cnt, torch.int32, "marg_cnt")
    _dev(lin_ws, torch.uint8, "lin_ws")
    for t, n in ((dq, "dq"), (dk, "dk"), (dv, "dv")):
        _dev(t, torch.float32, n)
    B, H, N, d = q.shape
    need = lib().sla_linear_branch_bwd_ws_bytes(B, H, N, d, block)
    if ws is None:
        ws = torch.empty(max(need, 1), dtype=torch.uint8, device=q.device)
    _call("sla_linear_branch_bwd", _ptr(q), _ptr(k), _ptr(v), B, H, N, d, block, _ptr(marg_idx),
          _ptr(marg_cnt), marg_idx.shape[-1], _ptr(d_o), _ptr(lin_ws), lin_ws.numel(), _ptr(dq),
          _ptr(dk), _ptr(dv), _ptr(ws), ws.numel() * ws.element_size(), _stream(stream))
    return dq, dk, dv


def sla_mask_recall(q, k, block, crit_idx, crit_cnt, scale=None, recall=None, ws=None,
                    stream=None):
    """Share of each query's dense softmax mass held by its kept tiles, fp32 [B, H, N]."""
    _dev(q, torch.bfloat16, "q")
    _dev(k, torch.bfloat16, "k")
    _dev(crit_idx, torch.int32, "crit_idx")
    _dev(crit_cnt, torch.int32, "crit_cnt")
    B, H, N, d = q.shape
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    if recall is None:
        recall = torch.empty((B, H, N), dtype=torch.float32, device=q.device)
    need = lib().sla_mask_recall_ws_bytes(B, H, N, d, block)
    if ws is None:
        ws = torch.empty(max(need, 1), dtype=torch.uint8, device=q.device)
    _call("sla_mask_recall", _ptr(q), _ptr(k), B, H, N, d, block, _ptr(crit_idx), _ptr(crit_cnt),
          crit_idx.shape[-1], float(scale), _ptr(recall), _ptr(ws), ws.numel() * ws.element_size(),
          _stream(stream))
    return recall


def sla_tile_permute(x, grid, tiles, block, inverse=False, y=None, stream=None):
    """Rows of x [B, H, T*Y*X, d] into per-head 3D tile order (or back, inverse=True).

    grid = (T, Y, X); tiles = one (bt, by, bx) per head (host ints)."""
    _dev(x, torch.bfloat16, "x")
    B, H, N, d = x.shape
    T, Y, X = (int(g) for g in grid)
    if len(tiles) != H:
        raise ValueError(f"need one tile shape per head ({H}), got {len(tiles)}")
    arr = (ctypes.c_int32 * (3 * H))(*[int(t) for shape in tiles for t in shape])
    if y is None:
        y = torch.empty_like(x)
    _call("sla_tile_permute", _ptr(x), _ptr(y), B, H, T, Y, X, d, int(block),
          ctypes.cast(arr, ctypes.c_void_p), int(bool(inverse)), _stream(stream))
    return y


def sla_combine(o_s, o_lin=None, o=None, stream=None):
    if o is None:
        o = torch.empty(o_s.shape, dtype=torch.bfloat16, device=o_s.device)
    _call("sla_combine", _ptr(o_s), int(o_s.dtype == torch.float32), _ptr(o_lin), _ptr(o),
          o_s.numel(), _stream(stream))
    return o


# ---------------------------------------------------------------------------
# the whole path
# ---------------------------------------------------------------------------

def _select(q, k, block, mode, keep, marg, thr, cls, stream):
    """Class map (pooled and classified, unless given) and its compacted lists;
    the marginal lists are None when the selection has no marginal tiles."""
    B, H, N, d = q.shape
    nb = num_blocks(N, block)
    if cls is None:
        kc, km = counts_for(mode, nb, keep, marg)
        cls = sla_pool_classify(q, k, block, mode, kc, km, thr or 0.0, stream=stream)
        kc_max = nb if mode == "cdf" else kc
        km_max = km
    else:
        # a given map: the fractions, when given, only size the lists
        kc_max = count_from_fraction(keep, nb) if keep is not None else nb
        km_max = (counts_for("sla3", nb, keep, marg)[1] if keep is not None and marg is not None
                  else nb)
    crit_idx, crit_cnt, marg_idx, marg_cnt = sla_block_mask(cls, kc_max, km_max, stream=stream)
    return cls, crit_idx, crit_cnt, marg_idx, marg_cnt


def forward(q, k, v, block, mode="topk", keep=None, marg=None, thr=None, cls=None, o_fp32=False,
            fused=False, stream=None):
    """Pool and classify (unless `cls` is given: mask-in), compact the lists,
    run the sparse and linear branches and combine.  With fused=True and a
    linear branch, the two branches run as sla_linear_branch_prepare plus
    sla_sparse_linear_attn_fwd (no O_s / O_lin intermediates).

    mode "topk" (keep), "cdf" (thr), "sla3" (keep, marg).  With a given cls,
    `keep`/`marg` only size the lists (default: the whole row).
    Returns a dict with o (bf16 [B, H, N, d]) and every intermediate.
    """
    cls, crit_idx, crit_cnt, marg_idx, marg_cnt = _select(q, k, block, mode, keep, marg, thr, cls,
                                                          stream)
    km_max = 0 if marg_idx is None else marg_idx.shape[-1]
    out = {"cls": cls, "crit_idx": crit_idx, "crit_cnt": crit_cnt, "marg_idx": marg_idx,
           "marg_cnt": marg_cnt}
    if km_max and fused:
        lin_ws = sla_linear_branch_prepare(k, v, block, marg_idx, marg_cnt, stream=stream)
        o, _ = sla_sparse_linear_attn_fwd(q, k, v, block, crit_idx, crit_cnt, lin_ws, stream=stream)
        out.update(o=o)
    elif km_max:
        o_s, _ = sla_sparse_attn_fwd(q, k, v, block, crit_idx, crit_cnt, o_fp32=True, stream=stream)
        o_lin = sla_linear_branch_fwd(q, k, v, block, marg_idx, marg_cnt, stream=stream)
        o = sla_combine(o_s, o_lin, stream=stream)
        out.update(o_s=o_s, o_lin=o_lin, o=o)
    elif o_fp32:
        o_s, _ = sla_sparse_attn_fwd(q, k, v, block, crit_idx, crit_cnt, o_fp32=True, stream=stream)
        out.update(o_s=o_s, o=sla_combine(o_s, None, stream=stream))
    else:
        o, _ = sla_sparse_attn_fwd(q, k, v, block, crit_idx, crit_cnt, o_fp32=False, stream=stream)
        out.update(o=o)
    return out


# ---------------------------------------------------------------------------
# training: the path as a torch.autograd.Function
# ---------------------------------------------------------------------------

class SlaAttention(torch.autograd.Function):
    """O = sparse softmax attention over the critical tiles plus linear
    attention over the marginal tiles (bf16), differentiable in q, k and v
    with the lists held fixed.  Forward: sla_sparse_attn_fwd (fp32 O_s and
    LSE kept for the backward), sla_linear_branch_fwd, sla_combine.  Backward:
    sla_sparse_attn_bwd, then sla_linear_branch_bwd adds the linear branch's
    gradients; they are fp32, and autograd rounds them to the inputs' bf16.
    marg_idx / marg_cnt may be None (no linear branch)."""

    @staticmethod
    def forward(ctx, q, k, v, block, crit_idx, crit_cnt, marg_idx=None, marg_cnt=None):
        o_s, lse = sla_sparse_attn_fwd(q, k, v, block, crit_idx, crit_cnt, o_fp32=True,
                                       want_lse=True)
        lin_ws = None
        o_lin = None
        if marg_idx is not None:
            B, H, N, d = q.shape
            lin_ws = torch.empty(max(lib().sla_linear_branch_ws_bytes(B, H, N, d, block), 1),
                                 dtype=torch.uint8, device=q.device)
            o_lin = sla_linear_branch_fwd(q, k, v, block, marg_idx, marg_cnt, ws=lin_ws)
        o = sla_combine(o_s, o_lin)
        ctx.block = block
        ctx.save_for_backward(q, k, v, crit_idx, crit_cnt, marg_idx, marg_cnt, o_s, lse, lin_ws)
        return o

    @staticmethod
    def backward(ctx, d_o):
        q, k, v, crit_idx, crit_cnt, marg_idx, marg_cnt, o_s, lse, lin_ws = ctx.saved_tensors
        if d_o.dtype != torch.bfloat16:
            raise ValueError(f"the output gradient must be bf16, got {d_o.dtype}")
        d_o = d_o.contiguous()
        dq, dk, dv = sla_sparse_attn_bwd(q, k, v, ctx.block, crit_idx, crit_cnt, o_s, lse, d_o)
        if marg_idx is not None:
            sla_linear_branch_bwd(q, k, v, ctx.block, marg_idx, marg_cnt, d_o, lin_ws, dq, dk, dv)
        return dq, dk, dv, None, None, None, None, None


def sla_attention(q, k, v, block, mode="topk", keep=None, marg=None, thr=None, cls=None):
    """Selection (no gradient) followed by SlaAttention: the differentiable
    form of forward().  Everything runs on the current stream, as autograd's
    own backward does.  Returns (o, lists) with lists = (cls, crit_idx,
    crit_cnt, marg_idx, marg_cnt)."""
    with torch.no_grad():
        lists = _select(q.detach(), k.detach(), block, mode, keep, marg, thr, cls, None)
    _, crit_idx, crit_cnt, marg_idx, marg_cnt = lists
    return SlaAttention.apply(q, k, v, block, crit_idx, crit_cnt, marg_idx, marg_cnt), lists
