"""The oracle proper: fp64 numpy, plain definitions, no blocking beyond the method's.

Readings taken where the pages are silent or loose (each one is also stated
in the design notes):

R1  pooled scores are scaled like attention logits: s_ij = (qbar_i . kbar_j) / sqrt(d).
R2  "mean pooling" pools Q and K first and then takes one dot product per block pair.
R3  block j covers tokens [j*b, min((j+1)*b, N)); a partial last block is pooled
    over its valid tokens only; tokens past N never enter any sum.
R4  a keep fraction f becomes the count max(1, ceil(f * nkb)), in exact rationals;
    "the next g" marginal fraction becomes ceil((f + g) * nkb) - (critical count).
R5  score order is descending and stable: equal scores keep the lower key-block
    index first.
R6  the NABLA cut keeps the smallest prefix of that order whose softmax mass is
    >= 1 - thr (at least one block).
R7  selection is per (batch, head, query block) row, over that row's key blocks.
R8  the three-way split takes the first k_c blocks of the order as critical,
    the next k_m as marginal and the rest as skipped.
R9  the linear branch uses phi(x) = elu(x) + 1 elementwise on raw q and k, with no
    1/sqrt(d), and normalises by phi(q) . sum phi(k).
R10 the two branches are summed without weights.
R11 the softmax of the critical branch is renormalised over the kept keys only.
R12 a query block with no critical tile gets O_s = 0 and LSE = -inf; one with no
    marginal tile gets O_lin = 0.
R14 attention is non-causal.
R15 query blocks and key blocks have the same size b.

Class codes in a class map: 0 skipped, 1 marginal, 2 critical.
"""

import math
from fractions import Fraction

import numpy as np

SKIP, MARGINAL, CRITICAL = 0, 1, 2


# ----------------------------------------------------------------------------
# input decoding and blocks
# ----------------------------------------------------------------------------

def bf16_to_f64(bits):
    """Exact decode of bf16 bit patterns (uint16) to float64.

    A bf16 number is the upper half of an IEEE float32, so its value is that
    float32 with the low 16 mantissa bits zero; float32 -> float64 is exact.
    """
    bits = np.asarray(bits, dtype=np.uint16)
    return (bits.astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)


def num_blocks(N, b):
    return -(-N // b)


def block_bounds(N, b, j):
    """Token range [lo, hi) of block j (R3)."""
    lo = j * b
    return lo, min(lo + b, N)


# ----------------------------------------------------------------------------
# step 1: mean pooling (SLA post: a fast mean-pooling step marks blocks;
#         NABLA post point 2: Query and Key are compressed)
# ----------------------------------------------------------------------------

def pool(x, b):
    """Mean of each block of b consecutive tokens, over valid tokens only (R3).

    x: float64 [..., N, d]  ->  float64 [..., nb, d]
    """
    N = x.shape[-2]
    nb = num_blocks(N, b)
    out = np.empty(x.shape[:-2] + (nb, x.shape[-1]), dtype=np.float64)
    for j in range(nb):
        lo, hi = block_bounds(N, b, j)
        out[..., j, :] = x[..., lo:hi, :].sum(axis=-2) / (hi - lo)
    return out


def pooled_scores(q_pool, k_pool, scale):
    """s_ij = scale * (qbar_i . kbar_j)  (R1, R2).  [..., nqb, d] x [..., nkb, d] -> [..., nqb, nkb]."""
    return scale * np.matmul(q_pool, np.swapaxes(k_pool, -1, -2))


# ----------------------------------------------------------------------------
# step 2: classification of block pairs
# ----------------------------------------------------------------------------

def count_from_fraction(frac, nkb):
    """R4: a fraction of the key blocks as a count, rounded up, at least 1."""
    frac = Fraction(frac)
    return max(1, math.ceil(frac * nkb))


def split_counts(keep, marg, nkb):
    """(k_c, k_m) for a critical fraction and a following marginal fraction (R4)."""
    kc = count_from_fraction(keep, nkb)
    if marg is None or Fraction(marg) == 0:
        return kc, 0
    total = min(nkb, math.ceil((Fraction(keep) + Fraction(marg)) * nkb))
    return kc, max(0, total - kc)


def descending_order(s_row):
    """Key-block indices by descending score, ties to the lower index (R5)."""
    # A stable sort of the negated scores keeps equal scores in index order.
    return np.argsort(-np.asarray(s_row, dtype=np.float64), kind="stable")


def softmax(s_row):
    s = np.asarray(s_row, dtype=np.float64)
    e = np.exp(s - s.max())
    return e / e.sum()


def cdf_count(s_row, thr):
    """NABLA cut (R6): smallest m >= 1 whose top-m softmax mass is >= 1 - thr."""
    order = descending_order(s_row)
    p = softmax(s_row)
    target = 1.0 - thr
    mass = 0.0
    for m, j in enumerate(order, start=1):
        mass += p[j]
        if mass >= target:
            return m
    return len(order)


def classify_row(s_row, mode, kc=0, km=0, thr=None):
    """Class codes of one row of key blocks (R7, R8)."""
    order = descending_order(s_row)
    cls = np.full(len(order), SKIP, dtype=np.uint8)
    if mode == "topk":
        cls[order[:kc]] = CRITICAL
    elif mode == "sla3":
        cls[order[:kc]] = CRITICAL
        cls[order[kc:kc + km]] = MARGINAL
    elif mode == "cdf":
        cls[order[:cdf_count(s_row, thr)]] = CRITICAL
    else:
        raise ValueError(f"unknown selection mode {mode!r}")
    return cls


def classify(scores, mode, kc=0, km=0, thr=None):
    """Class map [..., nqb, nkb] from pooled scores [..., nqb, nkb]."""
    cls = np.empty(scores.shape, dtype=np.uint8)
    flat_s = scores.reshape(-1, scores.shape[-1])
    flat_c = cls.reshape(-1, scores.shape[-1])
    for r in range(flat_s.shape[0]):
        flat_c[r] = classify_row(flat_s[r], mode, kc, km, thr)
    return cls


def index_lists(cls, value, width):
    """Ascending key-block lists of one class, padded with -1, plus counts.

    cls [..., nqb, nkb] -> idx int32 [..., nqb, width], cnt int32 [..., nqb]
    """
    lead = cls.shape[:-1]
    idx = np.full(lead + (width,), -1, dtype=np.int32)
    cnt = np.zeros(lead, dtype=np.int32)
    flat_c = cls.reshape(-1, cls.shape[-1])
    flat_i = idx.reshape(-1, width)
    flat_n = cnt.reshape(-1)
    for r in range(flat_c.shape[0]):
        js = np.nonzero(flat_c[r] == value)[0]
        if len(js) > width:
            raise ValueError(f"row {r}: {len(js)} blocks of class {value} exceed width {width}")
        flat_i[r, :len(js)] = js
        flat_n[r] = len(js)
    return idx, cnt


# ----------------------------------------------------------------------------
# step 3: softmax attention over the critical blocks (SLA: critical blocks via
#         FlashAttention; Veda: attention only in the selected tiles)
# ----------------------------------------------------------------------------

def _tokens_of(blocks, N, b):
    parts = [np.arange(*block_bounds(N, b, int(j))) for j in blocks]
    return np.concatenate(parts) if parts else np.zeros(0, dtype=np.int64)


def attend_block(q_rows, k, v, kept_blocks, b, scale, return_p=False):
    """Masked softmax attention of one query block (R11, R12, R14).

    q_rows [r, d]; k, v [N, d]; kept_blocks: key-block indices.
    Returns O [r, d], LSE [r] (and P [r, |T|] when asked).
    """
    N = k.shape[0]
    toks = _tokens_of(kept_blocks, N, b)
    r = q_rows.shape[0]
    if len(toks) == 0:
        o = np.zeros((r, v.shape[1]))
        lse = np.full(r, -np.inf)
        return (o, lse, np.zeros((r, 0))) if return_p else (o, lse)
    logits = scale * (q_rows @ k[toks].T)                  # [r, |T|]
    mx = logits.max(axis=1, keepdims=True)
    e = np.exp(logits - mx)
    z = e.sum(axis=1, keepdims=True)
    p = e / z
    o = p @ v[toks]
    lse = mx[:, 0] + np.log(z[:, 0])
    return (o, lse, p) if return_p else (o, lse)


# ----------------------------------------------------------------------------
# step 4: linear attention over the marginal blocks (SLA: intermediate blocks
#         via linear attention), phi = elu + 1 (R9)
# ----------------------------------------------------------------------------

def phi(x):
    """elu(x) + 1 with alpha = 1: x + 1 for x > 0, exp(x) otherwise."""
    x = np.asarray(x, dtype=np.float64)
    return np.where(x > 0, x + 1.0, np.exp(np.minimum(x, 0.0)))


def linear_block(q_rows, k, v, marg_blocks, b):
    """Linear attention of one query block over its marginal key blocks (R9, R12).

    S = sum_m phi(k_m) v_m^T, zeta = sum_m phi(k_m) over the marginal tokens;
    O_lin[n] = phi(q_n)^T S / (phi(q_n) . zeta).
    """
    N = k.shape[0]
    toks = _tokens_of(marg_blocks, N, b)
    if len(toks) == 0:
        return np.zeros((q_rows.shape[0], v.shape[1]))
    pk = phi(k[toks])                                      # [|M|, d]
    state = pk.T @ v[toks]                                 # [d, d]
    zeta = pk.sum(axis=0)                                  # [d]
    pq = phi(q_rows)                                       # [r, d]
    return (pq @ state) / (pq @ zeta)[:, None]


# ----------------------------------------------------------------------------
# whole forward
# ----------------------------------------------------------------------------

def selection_counts(mode, nkb, keep=None, marg=None):
    """(k_c, k_m) for the count-based modes; (0, 0) for the NABLA cut."""
    if mode == "cdf":
        return 0, 0
    if mode == "topk":
        return count_from_fraction(keep, nkb), 0
    return split_counts(keep, marg, nkb)


def class_map(q, k, b, mode, keep=None, marg=None, thr=None, scale=None):
    """Pool, score and classify: q, k float64 [B, H, N, d] -> (cls, scores, q_pool, k_pool).

    mode "maskin" draws its mask by the same per-head top-k (with the following
    marginal fraction) as "sla3"; a caller may also pass its own map to forward().
    """
    d = q.shape[-1]
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    qp, kp = pool(q, b), pool(k, b)
    s = pooled_scores(qp, kp, scale)
    nkb = s.shape[-1]
    sel = "sla3" if mode == "maskin" else mode
    kc, km = selection_counts(sel, nkb, keep, marg)
    cls = classify(s, sel, kc, km, thr)
    return cls, s, qp, kp


def forward_rows(q, k, v, cls, b, rows, scale=None):
    """Outputs of selected query blocks.

    q, k, v float64 [B, H, N, d]; cls [B, H, nqb, nkb]; rows: iterable of
    (batch, head, query block).  Returns {row: (O_s, LSE, O_lin, O)} with
    O = O_s + O_lin (R10), all float64 over the block's valid query tokens.
    """
    N, d = q.shape[-2], q.shape[-1]
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    out = {}
    for (bi, h, i) in rows:
        lo, hi = block_bounds(N, b, i)
        qr = q[bi, h, lo:hi]
        crit = np.nonzero(cls[bi, h, i] == CRITICAL)[0]
        marg = np.nonzero(cls[bi, h, i] == MARGINAL)[0]
        o_s, lse = attend_block(qr, k[bi, h], v[bi, h], crit, b, scale)
        o_lin = linear_block(qr, k[bi, h], v[bi, h], marg, b)
        out[(bi, h, i)] = (o_s, lse, o_lin, o_s + o_lin)
    return out


def forward(q, k, v, cls, b, scale=None):
    """Dense outputs for every query block: (O_s, LSE, O_lin, O), float64 [B, H, N, d] / [B, H, N]."""
    B, H, N, d = q.shape
    nqb = num_blocks(N, b)
    o_s = np.zeros((B, H, N, d))
    o_lin = np.zeros((B, H, N, d))
    lse = np.zeros((B, H, N))
    rows = [(bi, h, i) for bi in range(B) for h in range(H) for i in range(nqb)]
    for (bi, h, i), (a, l, c, _) in forward_rows(q, k, v, cls, b, rows, scale).items():
        lo, hi = block_bounds(N, b, i)
        o_s[bi, h, lo:hi] = a
        lse[bi, h, lo:hi] = l
        o_lin[bi, h, lo:hi] = c
    return o_s, lse, o_lin, o_s + o_lin


# ----------------------------------------------------------------------------
# mask quality: attention-mass recall (Veda article: fidelity to the structure
# of dense attention, reported as recall)
# ----------------------------------------------------------------------------

def mask_recall(q, k, cls, b, scale=None, kept=(CRITICAL,)):
    """Per query token, the share of its dense softmax attention mass that falls
    on the keys of the tiles the class map keeps for its query block.

    q, k float64 [B, H, N, d]; cls [B, H, nqb, nkb]; `kept` lists the class
    codes counted as kept.  Returns float64 [B, H, N] in [0, 1]: the softmax is
    taken over all N keys (the dense distribution), its entries summed over the
    kept tokens only.
    """
    B, H, N, d = q.shape
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    nqb = num_blocks(N, b)
    out = np.zeros((B, H, N))
    for bi in range(B):
        for h in range(H):
            for i in range(nqb):
                lo, hi = block_bounds(N, b, i)
                logits = scale * (q[bi, h, lo:hi] @ k[bi, h].T)        # [r, N]
                blocks = [j for j in range(cls.shape[-1]) if cls[bi, h, i, j] in kept]
                toks = _tokens_of(blocks, N, b)
                for r in range(hi - lo):
                    p = softmax(logits[r])
                    out[bi, h, lo + r] = p[toks].sum() if len(toks) else 0.0
    return out
