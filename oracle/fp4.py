"""FP4 inference forward in MXFP4 form (test infrastructure only).

The SageAttention3 summary ("Approach" and the table of measured effects)
describes an inference-only attention with both matmuls on FP4 microscaling
operands: NVFP4 (E2M1 elements, one E4M3 scale per 1x16 block) with a
two-level scaling of the softmax matrix P, whose first level renormalizes
each row to [0, 448 x 6] so that the E4M3 block scales use their full range.
It also reports MXFP4 (one E8M0 scale per 1x32 block) as less accurate than
NVFP4 (CosSim 98.37 % against 99.52 %), and direct quantization of P as far
worse than the two-level scaling (93.32 % against 99.52 %).

MI355X multiplies FP4 operands with one E8M0 scale per 32 values of the
contraction index inside its scaled matrix instruction, so this module
defines the forward in that form, step by step:

  Y1  QK-norm, smoothing means and centring exactly as the INT8 steps F0-F2.
  Y2  block quantizer  per block of 32 values along the contraction index:
                         a = max|x|;  e = the least integer with 6 * 2^e >= a,
                         clamped to [-126, 127] (an all-zero block gets -126),
                         code = E2M1_rne(x * 2^-e)
                       (6 is the largest E2M1 value, so codes never overflow).
                       Q and K: blocks of 32 consecutive channels of a token.
                       V: for each channel, the 32 keys of one key class of a
                       64-key tile, class h = (key mod 8) div 4 (keys
                       8j + 4h + i, j = 0..7, i = 0..3, of the tile).
  Y3  Q-smoothing bias b_j = mu_q . K~_j with K~ the centred K before
                       quantization (float32 values, exact float64 sum).
                       The 8-bit modes use the dequantized K (F4); with
                       E2M1 codes that term would carry K's 4-bit rounding
                       error times |mu_q|, which is large exactly when
                       Q-smoothing matters (Q channels with large means), and
                       the float K costs the same one product per key.
  Y4  scores           S = (Q^ K^^T + b_j) / 8, masked entries -inf.
  Y5  P~ codes         online over the 64-key tiles with the running row
                       maximum M_t (as the MXFP8 step X5): P~ = exp(S - M_t)
                       in (0, 1]; for each query, tile and key class, Y2 on
                       the 32 values of P~ (the block of the P~V product).
  Y6  combine          l = sum_t exp(M_t - M) sum_j P^ (the row sum of the
                       dequantized P~), O = sum_t exp(M_t - M) P^_t V^_t / l,
                       LSE = M + ln l + (q_raw . mu_k) / 8.

The key classes make a block of P~ or V the 32 keys one half of a 64-lane
wave holds in the accumulator layout of the score product; any fixed
partition of a tile's keys into two sets of 32 is a block of "32 values along
the contraction index", and this one needs no data movement.

The first level of the two-level P scaling has no counterpart here: a row
factor that is a power of two changes no code (the block exponents absorb
it), and E8M0 scales cover 2^+-127, so there is no scale range to fill.
``p_blocks=False`` replaces the Y5 block exponents by the fixed exponent -2
of a block whose maximum is 1 (direct quantization of P~ with one scale).

With ``rounding=False`` the E2M1 rounding and the fp32 roundings are removed
(the power-of-two scales stay), so the result must equal exact attention.
"""
from __future__ import annotations

from dataclasses import dataclass

import numpy as np

from . import faithful as _F

BLK = 64                 # tile side (keys per online step, tokens per code block)
MB = 32                  # values per quantization block
D = 64
SCALE = 1.0 / 8.0
E2M1_MAX = 6.0


# ---------------------------------------------------------------- Y2

def _e2m1_table() -> np.ndarray:
    """Values of the 16 E2M1 codes: sign bit 3, exponent bits 2..1 (bias 1),
    mantissa bit 0; exponent 0 is subnormal (m * 0.5)."""
    vals = np.zeros(16)
    for c in range(16):
        s = -1.0 if c & 8 else 1.0
        e = (c >> 1) & 3
        m = c & 1
        vals[c] = s * (m * 0.5 if e == 0 else (1.0 + m / 2.0) * 2.0 ** (e - 1))
    return vals


E2M1_VALUES = _e2m1_table()


def e2m1_encode(y) -> np.ndarray:
    """Code of the nearest E2M1 value (ties to the even code) for |y| <= 6,
    given exactly in float64: below 2 the grid has step 0.5, in [2, 4) step
    1 and in [4, 6] step 2, so the code is the rounded position on that grid."""
    y = np.asarray(y, np.float64)
    a = np.abs(y)
    if np.any(~np.isfinite(a)) or np.any(a > E2M1_MAX):
        raise ValueError("E2M1 input out of range")
    code = np.empty(a.shape, np.int64)
    lo = a < 2.0
    code[lo] = np.rint(a[lo] * 2.0).astype(np.int64)            # 0, 0.5, ..., 2.0 -> codes 0..4
    mid = (a >= 2.0) & (a < 4.0)
    code[mid] = 4 + np.rint(a[mid] - 2.0).astype(np.int64)        # 2, 3, 4 -> codes 4, 5, 6
    hi = a >= 4.0
    code[hi] = 6 + np.rint((a[hi] - 4.0) / 2.0).astype(np.int64)  # 4, 6 -> codes 6, 7
    return (code | np.where(np.signbit(y), 8, 0)).astype(np.uint8)


def e2m1_round(y) -> np.ndarray:
    """Nearest E2M1 value (ties to the even code) of each finite |y| <= 6."""
    y = np.asarray(y, np.float64)
    v = E2M1_VALUES[e2m1_encode(y)]
    return np.where(y == 0, y, v)


def fp4_exponent(a) -> np.ndarray:
    """Y2 scale exponent: the least integer e with 6 2^e >= a (a > 0), clamped
    to [-126, 127]; -126 for a = 0."""
    a = np.asarray(a, np.float64)
    e = np.zeros(a.shape, np.int64)
    pos = a > 0
    g = np.ceil(np.log2(a[pos] / E2M1_MAX)).astype(np.int64)
    g = np.where(np.ldexp(E2M1_MAX, g) < a[pos], g + 1, g)          # exact comparisons fix the log2
    g = np.where(np.ldexp(E2M1_MAX, g - 1) >= a[pos], g - 1, g)
    e[pos] = g
    e[~pos] = -126
    return np.clip(e, -126, 127)


def quantize_groups(x, rounding: bool = True):
    """Y2 over the last axis of ``x`` (its length 32 is one block).  Returns
    (dequantized values, exponents x.shape[:-1], codes = value / 2^e)."""
    x = np.asarray(x, np.float64)
    e = fp4_exponent(np.max(np.abs(x), axis=-1))
    scaled = x * np.ldexp(1.0, -e)[..., None]
    codes = e2m1_round(scaled) if rounding else scaled
    return codes * np.ldexp(1.0, e)[..., None], e, codes


def key_class_order(partition: str = "class") -> np.ndarray:
    """[2, 32]: the keys of key class h of a 64-key tile, in increasing order.
    partition "class": class h = (key mod 8) div 4 (the blocks the GPU forms
    in its score accumulators); "contiguous": keys 32h .. 32h + 31, kept as a
    reference partition for the accuracy comparison of the two."""
    k = np.arange(BLK)
    if partition == "contiguous":
        return np.stack([k[k // 32 == h] for h in (0, 1)])
    if partition != "class":
        raise ValueError(partition)
    return np.stack([k[(k % 8) // 4 == h] for h in (0, 1)])


def quantize_rows(x, nrows: int, rounding: bool = True):
    """Q or K [Np, 64]: blocks of 32 consecutive channels of each token; rows
    >= nrows are padding (zero).  Returns (dequantized [Np, 64], exponents
    [Np, 2])."""
    x = np.array(x, np.float64)
    x[nrows:] = 0.0
    deq, e, _ = quantize_groups(x.reshape(-1, 2, MB), rounding)
    return deq.reshape(x.shape), e


def quantize_v(v, nrows: int, rounding: bool = True, partition: str = "class"):
    """V [Np, 64]: for each channel, the 32 keys of each key class of each
    64-key tile.  Returns (dequantized [Np, 64], exponents [T, 2, 64] as
    (tile, class, channel))."""
    v = np.array(v, np.float64)
    v[nrows:] = 0.0
    T = v.shape[0] // BLK
    cls = key_class_order(partition)
    g = v.reshape(T, BLK, D)[:, cls, :]                        # [T, 2, 32, 64]
    deq, e, _ = quantize_groups(np.swapaxes(g, 2, 3), rounding)  # blocks along the 32 keys
    out = np.zeros((T, BLK, D))
    out[:, cls, :] = np.swapaxes(deq, 2, 3)
    return out.reshape(v.shape), e


# ---------------------------------------------------------------- Y1-Y4

@dataclass
class Prepared:
    N: int
    T: int
    mu_q: np.ndarray
    mu_k: np.ndarray
    qh: np.ndarray       # [Np, 64] dequantized smoothed Q
    kh: np.ndarray
    vh: np.ndarray
    eq: np.ndarray       # [Np, 2] exponents (token, channel half)
    ek: np.ndarray
    ev: np.ndarray       # [T, 2, 64] exponents (tile, key class, channel)
    b: np.ndarray        # [Np] Q-smoothing bias
    corr: np.ndarray     # [Np]
    rounding: bool
    partition: str = "class"   # the key partition of the P~ and V blocks (key_class_order)


def prepare(q, k, v, smooth_q: bool, smooth_k: bool, rounding: bool = True, qk_norm: bool = False,
            partition: str = "class") -> Prepared:
    """Y1-Y3 for one head (q, k, v: [N, 64] arrays of bf16 values)."""
    fp = _F.prepare(q, k, v, smooth_q, smooth_k, rounding, qk_norm)    # F0-F2 and the means
    N, T = fp.N, fp.T
    Np = T * BLK
    dt = np.float32 if rounding else np.float64

    def centre(x, mu):
        out = np.zeros((Np, D), dt)
        if rounding:
            out[:N] = np.asarray(x, np.float32) - np.float32(mu)
        else:
            out[:N] = np.asarray(x, np.float64) - np.asarray(mu, np.float64)
        return out

    qh, eq = quantize_rows(centre(fp.q_raw, fp.mu_q), N, rounding)
    kt = centre(fp.k_in, fp.mu_k)
    kh, ek = quantize_rows(kt, N, rounding)
    vh, ev = quantize_v(centre(v, np.zeros(D, dt)), N, rounding, partition)
    b = np.asarray(kt, np.float64) @ np.asarray(fp.mu_q, np.float64)
    return Prepared(N, T, fp.mu_q, fp.mu_k, qh, kh, vh, eq, ek, ev, b, fp.corr, rounding, partition)


# ---------------------------------------------------------------- Y5-Y6

def fwd_head(pp: Prepared, causal: bool, qblocks=None, chunk_blocks: int = 4, p_blocks: bool = True,
             return_codes: bool = False):
    """Y4-Y6 for the query blocks ``qblocks`` (default all).  Returns (O, LSE)
    for their padded rows, plus (the dequantized P^ [R, Np], the P~ block
    exponents [R, T, 2], the running maxima [R, T]) if return_codes."""
    T = pp.T
    qblocks = list(range(T)) if qblocks is None else list(qblocks)
    cols = np.arange(T * BLK)
    cls = key_class_order(pp.partition)
    vb = pp.vh.reshape(T, BLK, D)
    oo, ll, pq, ee, mm = [], [], [], [], []
    for c0 in range(0, len(qblocks), chunk_blocks):
        rows = np.concatenate([np.arange(i * BLK, (i + 1) * BLK) for i in qblocks[c0:c0 + chunk_blocks]])
        R = rows.size
        S = (pp.qh[rows] @ pp.kh.T + pp.b[None, :]) * SCALE
        keep = (cols[None, :] < pp.N) & (rows[:, None] < pp.N)
        if causal:
            keep &= cols[None, :] <= rows[:, None]
        S = np.where(keep, S, -np.inf).reshape(R, T, BLK)
        kt = keep.reshape(R, T, BLK)
        Mt = np.maximum.accumulate(np.max(S, axis=2), axis=1)              # [R, T] running max
        Mf = np.where(np.isfinite(Mt), Mt, 0.0)
        with np.errstate(invalid="ignore"):
            pt = np.where(kt, np.exp(S - Mf[:, :, None]), 0.0)              # [R, T, 64]
        g = pt[:, :, cls]                                                   # [R, T, 2, 32]
        if p_blocks:
            ph, e, _ = quantize_groups(g, pp.rounding)
        else:
            e = np.full(g.shape[:3], -2)
            scaled = g * 4.0
            ph = (e2m1_round(scaled) if pp.rounding else scaled) / 4.0
        P = np.zeros((R, T, BLK))
        P[:, :, cls] = ph
        M = Mt[:, -1]
        with np.errstate(invalid="ignore"):
            w = np.where(np.isfinite(Mt), np.exp(Mf - M[:, None]), 0.0)    # [R, T]
        l = np.sum(w * np.sum(P, axis=2), axis=1)
        acc = np.einsum("rt,trc->rc", w, np.matmul(P.transpose(1, 0, 2), vb))
        with np.errstate(invalid="ignore", divide="ignore"):
            oo.append(acc / l[:, None])
            ll.append(M + np.log(l) + pp.corr[rows])
        if return_codes:
            pq.append(P.reshape(R, T * BLK))
            ee.append(e)
            mm.append(Mt)
    o, lse = np.concatenate(oo), np.concatenate(ll)
    if return_codes:
        return o, lse, np.concatenate(pq), np.concatenate(ee), np.concatenate(mm)
    return o, lse


def fwd(q, k, v, causal: bool, smooth_q: bool, smooth_k: bool, rounding: bool = True, qk_norm: bool = False,
        p_blocks: bool = True):
    """FP4 forward over [B, H, N, 64] arrays of bf16 values."""
    B, H, N, _ = q.shape
    o = np.zeros((B, H, N, D))
    lse = np.zeros((B, H, N))
    for b in range(B):
        for h in range(H):
            pp = prepare(q[b, h], k[b, h], v[b, h], smooth_q, smooth_k, rounding, qk_norm)
            ob, lb = fwd_head(pp, causal, p_blocks=p_blocks)
            o[b, h], lse[b, h] = ob[:N], lb[:N]
    return o, lse
