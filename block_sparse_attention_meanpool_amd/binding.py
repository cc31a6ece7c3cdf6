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
# SLA_LIBRARY selects another build of the same library (the debug-checks or
# host-sanitized variants); the default is the in-tree release build.
LIB_PATH = os.environ.get("SLA_LIBRARY") or os.path.join(_HERE, "libsla.so")

SEL_TOPK, SEL_CDF, SEL_SLA3 = 0, 1, 2
MODES = {"topk": SEL_TOPK, "cdf": SEL_CDF, "sla3": SEL_SLA3}
CLS_SKIP, CLS_MARGINAL, CLS_CRITICAL = 0, 1, 2
FLAG_BAD_CLASS, FLAG_OVERFLOW = 1, 2
FLAG_LIST_RANGE, FLAG_LIST_REPEAT, FLAG_LIST_ORDER, FLAG_LIST_COUNT = 4, 8, 16, 32
FLAG_ORDER_PERM = 64

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
    "sla_sparse_attn_fwd": (_I32, [_P, _P, _P, _I64, _I64, _I64, _I64, _I32, _P, _P, _I32, _P,
                                   _F, _P, _I32, _P, _P]),
    "sla_linear_branch_fwd": (_I32, [_P, _P, _P, _I64, _I64, _I64, _I64, _I32, _P, _P, _I32, _P,
                                     _P, _SZ, _P]),
    "sla_linear_branch_ws_bytes": (_SZ, [_I64, _I64, _I64, _I64, _I32]),
    "sla_linear_branch_prepare": (_I32, [_P, _P, _I64, _I64, _I64, _I64, _I32, _P, _P, _I32, _P,
                                         _SZ, _P]),
    "sla_sparse_linear_attn_fwd": (_I32, [_P, _P, _P, _I64, _I64, _I64, _I64, _I32, _P, _P, _I32,
                                          _P, _F, _P, _SZ, _P, _I32, _P, _P]),
    "sla_combine": (_I32, [_P, _I32, _P, _P, _I64, _P]),
    "sla_sparse_attn_bwd": (_I32, [_P, _P, _P, _I64, _I64, _I64, _I64, _I32, _P, _P, _I32, _P, _F,
                                   _P, _I32, _P, _P, _P, _P, _P, _P, _SZ, _P]),
    "sla_sparse_attn_bwd_ws_bytes": (_SZ, [_I64, _I64, _I64, _I64, _I32]),
    "sla_linear_branch_bwd": (_I32, [_P, _P, _P, _I64, _I64, _I64, _I64, _I32, _P, _P, _I32, _P, _P,
                                     _SZ, _P, _P, _P, _P, _SZ, _P]),
    "sla_linear_branch_bwd_ws_bytes": (_SZ, [_I64, _I64, _I64, _I64, _I32]),
    "sla_mask_recall": (_I32, [_P, _P, _I64, _I64, _I64, _I64, _I32, _P, _P, _I32, _F, _P, _P, _SZ,
                               _P]),
    "sla_mask_recall_ws_bytes": (_SZ, [_I64, _I64, _I64, _I64, _I32]),
    "sla_tile_permute": (_I32, [_P, _P, _I64, _I64, _I64, _I64, _I64, _I64, _I32, _P, _I32, _P]),
    "sla_dense_attn_fwd": (_I32, [_P, _P, _P, _I64, _I64, _I64, _I64, _I32, _F, _P, _I32, _P, _P]),
    "sla_check_lists": (_I32, [_P, _P, _I64, _I32, _I64, _P, _P]),
    "sla_check_row_order": (_I32, [_P, _I64, _I64, _I64, _P, _P]),
    "sla_clock_probe": (_I32, [_P, _I32, _P, _P]),
    "sla_row_order": (_I32, [_P, _P, _I64, _I64, _I64, _I32, _P, _P]),
    "sla_debug_flag": (_P, []),
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


def _dev(t, dtype, name, device=None):
    """A contiguous GPU tensor of `dtype` (or one of a tuple of dtypes), on
    `device` when given."""
    if not isinstance(t, torch.Tensor) or not t.is_cuda:
        raise ValueError(f"{name} must be a GPU tensor")
    if t.dtype not in (dtype if isinstance(dtype, tuple) else (dtype,)):
        raise ValueError(f"{name} must be {dtype}, got {t.dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if device is not None and t.device != device:
        raise ValueError(f"{name} is on {t.device}, the inputs on {device}")
    return t


def _shape(t, shape, name):
    """Raise unless tensor t (skipped when None) has exactly `shape`: every
    buffer the library writes or reads is sized from q's shape, so a mismatch
    would be an out-of-bounds device access."""
    if t is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")


def _qshape(q, name="q"):
    if not isinstance(q, torch.Tensor) or q.dim() != 4:
        raise ValueError(f"{name} must be a 4-D tensor [B, H, N, d]")
    return tuple(q.shape)


def _lists(idx, cnt, B, H, nb, name):
    """A [B, H, nb, width] list and its [B, H, nb] counts."""
    if idx is None or cnt is None:
        raise ValueError(f"{name}_idx and {name}_cnt are both required")
    if idx.dim() != 4 or tuple(idx.shape[:3]) != (B, H, nb) or idx.shape[3] < 1:
        raise ValueError(f"{name}_idx must have shape ({B}, {H}, {nb}, width), got {tuple(idx.shape)}")
    _shape(cnt, (B, H, nb), f"{name}_cnt")


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

def _pool_classify_args(q, k, block, q_pool, k_pool, cls):
    B, H, N, d = _qshape(q)
    nb = num_blocks(N, block)
    _shape(k, q.shape, "k")
    _shape(q_pool, (B, H, nb, d), "q_pool")
    _shape(k_pool, (B, H, nb, d), "k_pool")
    _shape(cls, (B, H, nb, nb), "cls")
    _dev(q, torch.bfloat16, "q")
    _dev(k, torch.bfloat16, "k", q.device)
    for t, n in ((q_pool, "q_pool"), (k_pool, "k_pool")):
        if t is not None:
            _dev(t, torch.float32, n, q.device)
    if cls is not None:
        _dev(cls, torch.uint8, "cls", q.device)
    return B, H, N, d, nb


def sla_pool_classify(q, k, block, mode, k_crit=0, k_marg=0, thr=0.0, scale=None, q_pool=None,
                      k_pool=None, cls=None, ws=None, stream=None):
    B, H, N, d, nb = _pool_classify_args(q, k, block, q_pool, k_pool, cls)
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    if cls is None:
        cls = torch.empty((B, H, nb, nb), dtype=torch.uint8, device=q.device)
    need = lib().sla_pool_classify_ws_bytes(B, H, N, d, block, int(q_pool is not None))
    if ws is not None:
        _dev(ws, torch.uint8, "ws", q.device)
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
    B, H, N, d, nb = _pool_classify_args(q, k, block, q_pool, k_pool, cls)
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
    B, H, nqb, nkb = _qshape(cls, "cls")
    if (crit_idx is None) != (crit_cnt is None) or (marg_idx is None) != (marg_cnt is None):
        raise ValueError("give each list with its counts, or neither")
    _shape(crit_idx, (B, H, nqb, kc_max), "crit_idx")
    _shape(crit_cnt, (B, H, nqb), "crit_cnt")
    if km_max:
        _shape(marg_idx, (B, H, nqb, km_max), "marg_idx")
        _shape(marg_cnt, (B, H, nqb), "marg_cnt")
    if err_flag is not None and err_flag.numel() < 1:
        raise ValueError("err_flag must hold one int32")
    _dev(cls, torch.uint8, "cls")
    dev = cls.device
    for t, n in ((crit_idx, "crit_idx"), (crit_cnt, "crit_cnt"), (marg_idx, "marg_idx"),
                 (marg_cnt, "marg_cnt"), (err_flag, "err_flag")):
        if t is not None:
            _dev(t, torch.int32, n, dev)
    if crit_idx is None:
        crit_idx = torch.empty((B, H, nqb, kc_max), dtype=torch.int32, device=dev)
        crit_cnt = torch.empty((B, H, nqb), dtype=torch.int32, device=dev)
    if km_max and marg_idx is None:
        marg_idx = torch.empty((B, H, nqb, km_max), dtype=torch.int32, device=dev)
        marg_cnt = torch.empty((B, H, nqb), dtype=torch.int32, device=dev)
    _call("sla_block_mask", _ptr(cls), B, H, nqb, nkb, _ptr(crit_idx), _ptr(crit_cnt), int(kc_max),
          _ptr(marg_idx), _ptr(marg_cnt), int(km_max), _ptr(err_flag), _stream(stream))
    return crit_idx, crit_cnt, marg_idx, marg_cnt


def _attn_args(q, k, v, block, lists=(), outs=(), lse=None, row_order=None):
    """Shape and device checks shared by the attention wrappers: k and v (and
    any extra [B, H, N, d] buffers in outs, given as (tensor, name, dtypes))
    like q; each (idx, cnt, name) list of lists; lse [B, H, N]; a row order
    [B, H, nb]."""
    B, H, N, d = _qshape(q)
    nb = num_blocks(N, block)
    _shape(row_order, (B, H, nb), "row_order")
    for t, n in ((k, "k"), (v, "v")):
        if t is not None:
            _shape(t, q.shape, n)
    for idx, cnt, n in lists:
        _lists(idx, cnt, B, H, nb, n)
    for t, n, _ in outs:
        _shape(t, q.shape, n)
    _shape(lse, (B, H, N), "lse")
    _dev(q, torch.bfloat16, "q")
    for t, n in ((k, "k"), (v, "v")):
        if t is not None:
            _dev(t, torch.bfloat16, n, q.device)
    for idx, cnt, n in lists:
        _dev(idx, torch.int32, f"{n}_idx", q.device)
        _dev(cnt, torch.int32, f"{n}_cnt", q.device)
    for t, n, dt in outs:
        if t is not None:
            _dev(t, dt, n, q.device)
    if lse is not None:
        _dev(lse, torch.float32, "lse", q.device)
    if row_order is not None:
        _dev(row_order, torch.int32, "row_order", q.device)
    return B, H, N, d, nb


_O_TYPES = (torch.float32, torch.bfloat16)


def sla_sparse_attn_fwd(q, k, v, block, crit_idx, crit_cnt, scale=None, o_s=None, o_fp32=True,
                        lse=None, want_lse=False, row_order=None, stream=None):
    B, H, N, d, _ = _attn_args(q, k, v, block, [(crit_idx, crit_cnt, "crit")],
                               [(o_s, "o_s", _O_TYPES)], lse, row_order)
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    if o_s is None:
        o_s = torch.empty(q.shape, dtype=torch.float32 if o_fp32 else torch.bfloat16, device=q.device)
    if want_lse and lse is None:
        lse = torch.empty((B, H, N), dtype=torch.float32, device=q.device)
    _call("sla_sparse_attn_fwd", _ptr(q), _ptr(k), _ptr(v), B, H, N, d, block, _ptr(crit_idx),
          _ptr(crit_cnt), crit_idx.shape[-1], _ptr(row_order), float(scale), _ptr(o_s),
          int(o_s.dtype == torch.float32), _ptr(lse), _stream(stream))
    return o_s, lse


def sla_dense_attn_fwd(q, k, v, block, scale=None, o=None, o_fp32=False, lse=None, want_lse=False,
                       stream=None):
    B, H, N, d, _ = _attn_args(q, k, v, block, [], [(o, "o", _O_TYPES)], lse)
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
    B, H, N, d, _ = _attn_args(q, k, v, block, [(marg_idx, marg_cnt, "marg")],
                               [(o_lin, "o_lin", torch.float32)])
    if ws is not None:
        _dev(ws, torch.uint8, "ws", q.device)
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
    B, H, N, d, _ = _attn_args(k, v, None, block, [(marg_idx, marg_cnt, "marg")])
    if ws is not None:
        _dev(ws, torch.uint8, "ws", k.device)
    need = lib().sla_linear_branch_ws_bytes(B, H, N, d, block)
    if ws is None:
        ws = torch.empty(max(need, 1), dtype=torch.uint8, device=k.device)
    _call("sla_linear_branch_prepare", _ptr(k), _ptr(v), B, H, N, d, block, _ptr(marg_idx),
          _ptr(marg_cnt), marg_idx.shape[-1], _ptr(ws), ws.numel() * ws.element_size(),
          _stream(stream))
    return ws


def sla_sparse_linear_attn_fwd(q, k, v, block, crit_idx, crit_cnt, lin_ws, scale=None, o=None,
                               o_fp32=False, lse=None, want_lse=False, row_order=None, stream=None):
    B, H, N, d, _ = _attn_args(q, k, v, block, [(crit_idx, crit_cnt, "crit")],
                               [(o, "o", _O_TYPES)], lse, row_order)
    _dev(lin_ws, torch.uint8, "lin_ws", q.device)
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    if o is None:
        o = torch.empty(q.shape, dtype=torch.float32 if o_fp32 else torch.bfloat16, device=q.device)
    if want_lse and lse is None:
        lse = torch.empty((B, H, N), dtype=torch.float32, device=q.device)
    _call("sla_sparse_linear_attn_fwd", _ptr(q), _ptr(k), _ptr(v), B, H, N, d, block,
          _ptr(crit_idx), _ptr(crit_cnt), crit_idx.shape[-1], _ptr(row_order), float(scale),
          _ptr(lin_ws),
          lin_ws.numel(), _ptr(o), int(o.dtype == torch.float32), _ptr(lse), _stream(stream))
    return o, lse


def sla_sparse_attn_bwd(q, k, v, block, crit_idx, crit_cnt, o_s, lse, d_o, scale=None, dq=None,
                        dk=None, dv=None, ws=None, row_order=None, stream=None):
    if o_s is None or lse is None or d_o is None:
        raise ValueError("o_s, lse and d_o are required")
    B, H, N, d, _ = _attn_args(q, k, v, block, [(crit_idx, crit_cnt, "crit")],
                               [(o_s, "o_s", _O_TYPES), (d_o, "d_o", torch.bfloat16),
                                (dq, "dq", torch.float32), (dk, "dk", torch.float32),
                                (dv, "dv", torch.float32)], lse, row_order)
    if ws is not None:
        _dev(ws, torch.uint8, "ws", q.device)
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    dq, dk, dv = (torch.empty(q.shape, dtype=torch.float32, device=q.device) if t is None else t
                  for t in (dq, dk, dv))
    need = lib().sla_sparse_attn_bwd_ws_bytes(B, H, N, d, block)
    if ws is None:
        ws = torch.empty(max(need, 1), dtype=torch.uint8, device=q.device)
    _call("sla_sparse_attn_bwd", _ptr(q), _ptr(k), _ptr(v), B, H, N, d, block, _ptr(crit_idx),
          _ptr(crit_cnt), crit_idx.shape[-1], _ptr(row_order), float(scale), _ptr(o_s),
          int(o_s.dtype == torch.float32), _ptr(lse), _ptr(d_o), _ptr(dq), _ptr(dk), _ptr(dv),
          _ptr(ws), ws.numel() * ws.element_size(), _stream(stream))
    return dq, dk, dv


def sla_linear_branch_bwd(q, k, v, block, marg_idx, marg_cnt, d_o, lin_ws, dq, dk, dv, ws=None,
                          stream=None):
    """Adds the linear branch's gradients into dq, dk, dv (fp32)."""
    if d_o is None or dq is None or dk is None or dv is None:
        raise ValueError("d_o, dq, dk and dv are required")
    B, H, N, d, _ = _attn_args(q, k, v, block, [(marg_idx, marg_cnt, "marg")],
                               [(d_o, "d_o", torch.bfloat16), (dq, "dq", torch.float32),
                                (dk, "dk", torch.float32), (dv, "dv", torch.float32)])
    _dev(lin_ws, torch.uint8, "lin_ws", q.device)
    if ws is not None:
        _dev(ws, torch.uint8, "ws", q.device)
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
    B, H, N, d, _ = _attn_args(q, k, None, block, [(crit_idx, crit_cnt, "crit")], [], recall)
    if ws is not None:
        _dev(ws, torch.uint8, "ws", q.device)
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
    B, H, N, d = _qshape(x, "x")
    _shape(y, x.shape, "y")
    _dev(x, torch.bfloat16, "x")
    if y is not None:
        _dev(y, torch.bfloat16, "y", x.device)
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
    if not isinstance(o_s, torch.Tensor):
        raise ValueError("o_s must be a tensor")
    _shape(o_lin, o_s.shape, "o_lin")
    _shape(o, o_s.shape, "o")
    _dev(o_s, _O_TYPES, "o_s")
    if o_lin is not None:
        _dev(o_lin, torch.float32, "o_lin", o_s.device)
    if o is not None:
        _dev(o, torch.bfloat16, "o", o_s.device)
    if o is None:
        o = torch.empty(o_s.shape, dtype=torch.bfloat16, device=o_s.device)
    _call("sla_combine", _ptr(o_s), int(o_s.dtype == torch.float32), _ptr(o_lin), _ptr(o),
          o_s.numel(), _stream(stream))
    return o


def sla_check_lists(idx, cnt, nkb, err_flag=None, stream=None):
    """OR the FLAG_LIST_* bits of every violation of the list form (entries in
    [0, nkb), strictly ascending, counts in [0, width]) into err_flag (device
    int32 [1], zeroed here when not given); returns err_flag."""
    if not isinstance(idx, torch.Tensor) or idx.dim() < 1:
        raise ValueError("idx must be a tensor [..., width]")
    _shape(cnt, idx.shape[:-1], "cnt")
    _dev(idx, torch.int32, "idx")
    _dev(cnt, torch.int32, "cnt", idx.device)
    if err_flag is None:
        err_flag = torch.zeros(1, dtype=torch.int32, device=idx.device)
    _dev(err_flag, torch.int32, "err_flag", idx.device)
    rows = idx.numel() // idx.shape[-1]
    _call("sla_check_lists", _ptr(idx), _ptr(cnt), rows, idx.shape[-1], int(nkb), _ptr(err_flag),
          _stream(stream))
    return err_flag


def sla_check_row_order(order, err_flag=None, stream=None):
    """OR FLAG_ORDER_PERM into err_flag (device int32 [1], zeroed here when not
    given) when some head's row order (int32 [B, H, nqb]) is not a permutation
    of its query blocks; returns err_flag."""
    if not isinstance(order, torch.Tensor) or order.dim() != 3:
        got = tuple(order.shape) if isinstance(order, torch.Tensor) else type(order).__name__
        raise ValueError(f"order must have shape [B, H, nqb], got {got}")
    B, H, nqb = tuple(order.shape)
    _dev(order, torch.int32, "order")
    if err_flag is None:
        err_flag = torch.zeros(1, dtype=torch.int32, device=order.device)
    _dev(err_flag, torch.int32, "err_flag", order.device)
    _call("sla_check_row_order", _ptr(order), B, H, nqb, _ptr(err_flag), _stream(stream))
    return err_flag


def sla_row_order(idx, cnt, order=None, stream=None):
    """Per head, the query blocks sorted by the median tile of their lists
    (int32 [B, H, nqb], a permutation per head): the run order to pass as
    row_order.  Scheduling only; results do not depend on it."""
    B, H, nqb, width = _qshape(idx, "idx")
    _shape(cnt, (B, H, nqb), "cnt")
    _shape(order, (B, H, nqb), "order")
    _dev(idx, torch.int32, "idx")
    _dev(cnt, torch.int32, "cnt", idx.device)
    if order is None:
        order = torch.empty((B, H, nqb), dtype=torch.int32, device=idx.device)
    _dev(order, torch.int32, "order", idx.device)
    _call("sla_row_order", _ptr(idx), _ptr(cnt), B, H, nqb, width, _ptr(order), _stream(stream))
    return order


def sla_clock_probe(span_us, out=None, stream=None):
    """Launch the shader-clock probe on `stream` (a second stream beside the work to
    measure): it waits span_us microseconds of the fixed-rate counter.  Returns
    (out, fixed_hz); after a synchronize, probe_clock_hz(out, fixed_hz) is the
    clock the chip ran at meanwhile."""
    if out is None:
        out = torch.zeros(4, dtype=torch.int64, device="cuda")
    _shape(out, (4,), "out")
    _dev(out, torch.int64, "out")
    hz = ctypes.c_int64(0)
    _call("sla_clock_probe", _ptr(out), int(span_us),
          ctypes.cast(ctypes.pointer(hz), ctypes.c_void_p), _stream(stream))
    return out, hz.value


def probe_clock_hz(out, fixed_hz):
    """Shader clock (Hz) from the probe's readings: counter differences times the
    fixed rate."""
    c0, c1, r0, r1 = (int(x) for x in out.cpu().tolist())
    return (c1 - c0) / max(r1 - r0, 1) * fixed_hz


def debug_flag_address():
    """Device address of the debug flag word (library built with
    SLA_DEBUG_CHECKS), or None for the release build."""
    return lib().sla_debug_flag()


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
        crit_idx, crit_cnt, marg_idx, marg_cnt = sla_block_mask(cls, kc_max, km_max, stream=stream)
        return cls, crit_idx, crit_cnt, marg_idx, marg_cnt
    # a given map: the fractions, when given, only size the lists, and a row
    # with more tiles than that width (which sla_block_mask would cut) raises
    kc_max = count_from_fraction(keep, nb) if keep is not None else nb
    km_max = (counts_for("sla3", nb, keep, marg)[1] if keep is not None and marg is not None
              else nb)
    flag = torch.zeros(1, dtype=torch.int32, device=q.device)
    crit_idx, crit_cnt, marg_idx, marg_cnt = sla_block_mask(cls, kc_max, km_max, err_flag=flag,
                                                            stream=stream)
    bits = int(flag.item())
    if bits & FLAG_OVERFLOW:
        raise ValueError(f"the given class map has a row with more critical or marginal tiles "
                         f"than the list widths ({kc_max}, {km_max}) that keep/marg imply")
    if bits & FLAG_BAD_CLASS:
        raise ValueError("the given class map holds a class value above 2")
    return cls, crit_idx, crit_cnt, marg_idx, marg_cnt


def forward(q, k, v, block, mode="topk", keep=None, marg=None, thr=None, cls=None, o_fp32=False,
            fused=False, stream=None):
    """Pool and classify (unless `cls` is given: mask-in), compact the lists,
    order the query blocks for L2 locality (sla_row_order), run the sparse and
    linear branches and combine.  With fused=True and a linear branch, the two
    branches run as sla_linear_branch_prepare plus sla_sparse_linear_attn_fwd
    (no O_s / O_lin intermediates).

    mode "topk" (keep), "cdf" (thr), "sla3" (keep, marg).  With a given cls,
    `keep`/`marg` only size the lists (default: the whole row).
    Returns a dict with o (bf16 [B, H, N, d]) and every intermediate.
    """
    cls, crit_idx, crit_cnt, marg_idx, marg_cnt = _select(q, k, block, mode, keep, marg, thr, cls,
                                                          stream)
    order = sla_row_order(crit_idx, crit_cnt, stream=stream)
    km_max = 0 if marg_idx is None else marg_idx.shape[-1]
    out = {"cls": cls, "crit_idx": crit_idx, "crit_cnt": crit_cnt, "marg_idx": marg_idx,
           "marg_cnt": marg_cnt, "row_order": order}
    attn = dict(row_order=order, stream=stream)
    if km_max and fused:
        lin_ws = sla_linear_branch_prepare(k, v, block, marg_idx, marg_cnt, stream=stream)
        o, _ = sla_sparse_linear_attn_fwd(q, k, v, block, crit_idx, crit_cnt, lin_ws, **attn)
        out.update(o=o)
    elif km_max:
        o_s, _ = sla_sparse_attn_fwd(q, k, v, block, crit_idx, crit_cnt, o_fp32=True, **attn)
        o_lin = sla_linear_branch_fwd(q, k, v, block, marg_idx, marg_cnt, stream=stream)
        o = sla_combine(o_s, o_lin, stream=stream)
        out.update(o_s=o_s, o_lin=o_lin, o=o)
    elif o_fp32:
        o_s, _ = sla_sparse_attn_fwd(q, k, v, block, crit_idx, crit_cnt, o_fp32=True, **attn)
        out.update(o_s=o_s, o=sla_combine(o_s, None, stream=stream))
    else:
        o, _ = sla_sparse_attn_fwd(q, k, v, block, crit_idx, crit_cnt, o_fp32=False, **attn)
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
    marg_idx / marg_cnt may be None (no linear branch); row_order (from
    sla_row_order) may be None and only sets the kernels' schedule."""

    @staticmethod
    def forward(ctx, q, k, v, block, crit_idx, crit_cnt, marg_idx=None, marg_cnt=None,
                row_order=None):
        o_s, lse = sla_sparse_attn_fwd(q, k, v, block, crit_idx, crit_cnt, o_fp32=True,
                                       want_lse=True, row_order=row_order)
        lin_ws = None
        o_lin = None
        if marg_idx is not None:
            B, H, N, d = q.shape
            lin_ws = torch.empty(max(lib().sla_linear_branch_ws_bytes(B, H, N, d, block), 1),
                                 dtype=torch.uint8, device=q.device)
            o_lin = sla_linear_branch_fwd(q, k, v, block, marg_idx, marg_cnt, ws=lin_ws)
        o = sla_combine(o_s, o_lin)
        ctx.block = block
        ctx.save_for_backward(q, k, v, crit_idx, crit_cnt, marg_idx, marg_cnt, o_s, lse, lin_ws,
                              row_order)
        return o

    @staticmethod
    def backward(ctx, d_o):
        q, k, v, crit_idx, crit_cnt, marg_idx, marg_cnt, o_s, lse, lin_ws, order = ctx.saved_tensors
        if d_o.dtype != torch.bfloat16:
            raise ValueError(f"the output gradient must be bf16, got {d_o.dtype}")
        d_o = d_o.contiguous()
        dq, dk, dv = sla_sparse_attn_bwd(q, k, v, ctx.block, crit_idx, crit_cnt, o_s, lse, d_o,
                                         row_order=order)
        if marg_idx is not None:
            sla_linear_branch_bwd(q, k, v, ctx.block, marg_idx, marg_cnt, d_o, lin_ws, dq, dk, dv)
        return dq, dk, dv, None, None, None, None, None, None


def sla_attention(q, k, v, block, mode="topk", keep=None, marg=None, thr=None, cls=None):
    """Selection (no gradient) followed by SlaAttention: the differentiable
    form of forward().  Everything runs on the current stream, as autograd's
    own backward does.  Returns (o, lists) with lists = (cls, crit_idx,
    crit_cnt, marg_idx, marg_cnt)."""
    with torch.no_grad():
        lists = _select(q.detach(), k.detach(), block, mode, keep, marg, thr, cls, None)
        _, crit_idx, crit_cnt, marg_idx, marg_cnt = lists
        order = sla_row_order(crit_idx, crit_cnt)
    return SlaAttention.apply(q, k, v, block, crit_idx, crit_cnt, marg_idx, marg_cnt, order), lists
