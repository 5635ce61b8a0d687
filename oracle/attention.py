"""CPU oracle for the attention forward pass -- TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this module.  It shares nothing with the GPU library.

What it computes ("Two Waves, One Stage Apart: Warp-Pipelining Triton GEMMs
on AMD Instinct", section "Beyond GEMM: FlashAttention", names the loop: a
score product, an online softmax, then the product with V; the function is
the usual scaled dot-product attention, which an online softmax reaches up to
rounding order).  For every batch b, head h and query row i:

    s_ij   = scale * sum_d Q[b,h,i,d] K[b,h,j,d]          (keys j allowed for i)
    lse_i  = log(sum_j exp(s_ij))
    O[i,:] = sum_j exp(s_ij - lse_i) V[b,h,j,:]

Keys allowed: all of them, or with ``causal`` the keys j <= i + (Sk - Sq)
(the last query row sees every key: causal masks aligned at the bottom
right).  A query row with no allowed key has O = 0 and lse = -inf.

Every operand bit pattern is widened exactly to float64 (``oracle.decode``);
the scores, the softmax and the weighted sum are float64: numpy matmuls for
the two products (library steps), the softmax written out.  Results are
float64, not rounded to the output type; the acceptance bound below adds the
output's rounding.

Pins (tests/test_oracle_attention.py): a pure-Python loop brute force with
math.fsum on tiny shapes; torch's scaled_dot_product_attention in float64;
closed forms (one key: O = V; identical keys: O = the mean of the allowed V
rows; a dominant key); key-permutation invariance; causal rows not depending
on masked keys; rows of P summing to one; and planted mistakes that each fail
one of these.
"""
from __future__ import annotations

import numpy as np

from . import decode


def _values(bits, elem: str) -> np.ndarray:
    return decode(np.ascontiguousarray(bits), elem)


def allowed_keys(Sq: int, Sk: int, causal: bool) -> np.ndarray:
    """Sq x Sk boolean mask of the keys each query row attends to."""
    if not causal:
        return np.ones((Sq, Sk), dtype=bool)
    i = np.arange(Sq)[:, None]
    j = np.arange(Sk)[None, :]
    return j <= i + (Sk - Sq)


def _head(q, k, v, scale, mask, rows):
    """One (batch, head): O rows, lse, P|V| rows and max_j scale*|q_i|.|k_j| for
    the query rows ``rows`` (float64 inputs)."""
    qr = q[rows]
    s = scale * (qr @ k.T)                                  # scores
    m = mask[rows]
    s = np.where(m, s, -np.inf)
    smax = s.max(axis=1, keepdims=True)
    live = np.isfinite(smax[:, 0])
    shift = np.where(np.isfinite(smax), smax, 0.0)
    e = np.where(m, np.exp(s - shift), 0.0)
    tot = e.sum(axis=1, keepdims=True)
    p = np.divide(e, tot, out=np.zeros_like(e), where=tot > 0)  # softmax over the allowed keys
    o = p @ v
    a = p @ np.abs(v)                                       # sum_j P_ij |V_jd|
    lse = np.where(live, shift[:, 0] + np.log(np.where(live, tot[:, 0], 1.0)), -np.inf)
    sabs = scale * np.where(m, np.abs(qr) @ np.abs(k).T, 0.0).max(axis=1)
    return o, lse, a, sabs


def attention(Q, K, V, elem: str, scale: float, causal: bool = False, rows=None):
    """O (B,H,R,D), lse (B,H,R), A = sum_j P_ij |V_jd| (B,H,R,D) and Sabs (B,H,R)
    = max_j scale * sum_d |Q_id K_jd| for query rows ``rows`` (all rows by
    default) of Q (B,H,Sq,D), K, V (B,H,Sk,D) given as FP16/BF16 bit patterns."""
    Q, K, V = (np.asarray(x) for x in (Q, K, V))
    if Q.ndim != 4 or K.shape != V.shape or Q.shape[:2] != K.shape[:2] or Q.shape[3] != K.shape[3]:
        raise ValueError("Q (B,H,Sq,D), K and V (B,H,Sk,D) expected")
    B, H, Sq, D = Q.shape
    Sk = K.shape[2]
    rows = np.arange(Sq) if rows is None else np.asarray(rows, dtype=np.int64)
    mask = allowed_keys(Sq, Sk, causal)
    O = np.empty((B, H, rows.size, D))
    A = np.empty((B, H, rows.size, D))
    L = np.empty((B, H, rows.size))
    S = np.empty((B, H, rows.size))
    for b in range(B):
        for h in range(H):
            q = _values(Q[b, h], elem)
            k = _values(K[b, h], elem)
            v = _values(V[b, h], elem)
            O[b, h], L[b, h], A[b, h], S[b, h] = _head(q, k, v, scale, mask, rows)
    return O, L, A, S


def probabilities(Q, K, elem: str, scale: float, causal: bool = False) -> np.ndarray:
    """The softmax matrix P (B,H,Sq,Sk) the oracle weights V with."""
    B, H, Sq, D = Q.shape
    Sk = K.shape[2]
    mask = allowed_keys(Sq, Sk, causal)
    P = np.zeros((B, H, Sq, Sk))
    eye = np.eye(Sk)
    for b in range(B):
        for h in range(H):
            q = _values(Q[b, h], elem)
            k = _values(K[b, h], elem)
            P[b, h] = _head(q, k, eye, scale, mask, np.arange(Sq))[0]
    return P


# Rounding unit of the probabilities the kernel feeds to its second product
# (it rounds P to the operand type) and of the output type.
UNIT = {"f16": 2.0 ** -11, "bf16": 2.0 ** -8}
F32 = 2.0 ** -24


def within_tolerance(o, oref, a, sabs, D: int, Sk: int, elem: str) -> np.ndarray:
    """Per-element acceptance of an attention output of type ``elem``:

        |o - Oref| <= (u + e) A + u |Oref|
        e = 2 D 2^-24 Sabs + 2 (Sk + 64) 2^-24 + 2^-20

    with A = sum_j P_ij |V_jd|, u = 2^-11 (FP16) or 2^-8 (BF16).  Each
    probability reaches the second product off by a relative u (rounded to
    the operand type) plus e: its score and the row's shift are FP32 sums of
    D products (each off by at most D 2^-24 Sabs), the row sum and the
    weighted sum are FP32 sums of at most Sk + 64 terms, and the exponential
    and scaling add a few FP32 roundings.  u |Oref| is the output's own
    rounding (half a spacing is at most u |O|)."""
    u = UNIT[elem]
    o = np.asarray(o, dtype=np.float64)
    e = 2 * D * F32 * np.asarray(sabs)[..., None] + 2 * (Sk + 64) * F32 + 2.0 ** -20
    with np.errstate(invalid="ignore"):
        ok = np.abs(o - oref) <= (u + e) * a + u * np.abs(oref)
    return ok & np.isfinite(o)


def lse_within_tolerance(lse, lref, sabs, D: int, Sk: int) -> np.ndarray:
    """|lse - lse_ref| <= 2 D 2^-24 Sabs + (Sk + 64) 2^-24 + 2^-20 (1 + |lse_ref|):
    FP32 scores, the FP32 row sum, and FP32 exp/log rounding.  Rows with no
    allowed key must give -inf on both sides."""
    lse = np.asarray(lse, dtype=np.float64)
    both_inf = np.isneginf(lse) & np.isneginf(lref)
    bound = 2 * D * F32 * sabs + (Sk + 64) * F32 + 2.0 ** -20 * (1 + np.abs(np.where(np.isfinite(lref), lref, 0)))
    with np.errstate(invalid="ignore"):
        ok = np.abs(lse - lref) <= bound
    return both_inf | ok
