"""Quantization-faithful SageBwd forward and backward (test infrastructure only).

The method (SageBwd page, abstract; SageAttention3 summary, "Approach" and the
ablation table) runs six of the seven attention matmuls on INT8 operands with
integer accumulation and keeps dO.V^T in 16-bit float.  The pages fix neither
the quantization granularity nor the arithmetic of the quantizers, so this
module writes out one precise reading of every step (each reading is listed,
with its reason, in the design notes that ship with the library):

  F0  QK-norm (option; SageBwd abstract, insight (i): necessary for stable
      training at many tokens per step): per token row of Q and of K,
      r = fp32(1 / sqrt(S / 64 + 1e-6)) (float64 steps) with S the float64
      sum of the exact squares (here the correctly rounded one; another
      summation order moves S by a few float64 ulps, which changes the
      float32 r only if r lies within ~1e-16 of a float32 rounding boundary),
      and the normalized row x_n = bf16(fp32(x r)), the tensor a separate norm
      would hand to attention; every later step reads x_n in place of x.
  F1  smoothing means  mu = fp32( exact_sum(x over the N valid tokens) / N )
      per (batch, head, channel), for K when smooth_k and for Q when smooth_q
      (SageBwd abstract, insight (iv): K-smoothing, optional Q-smoothing).
  F2  centring         x~ = fp32(x - mu)                (IEEE float32)
  F3  block quantizer  per block of 64 tokens x 64 channels, valid rows only:
                         a = max|x~|;  a < 2^-100 -> s = 0, all codes 0;
                         else s = fp32(a / 127), inv = fp32(127 / a) (both
                         correctly rounded quotients),
                         code = round_half_even(x~ * inv)  (exact product)
      giving codes in [-127, 127] and one float32 scale per block.
  F4  Q-smoothing bias b_j = mu_q . (s_K,t K_code_j): with it the score is the
      product of the dequantized operands (Q^ + mu_q) . K^_j; K's mean only
      shifts every score row by a constant, which softmax ignores.
  F5  score tile       A = Q_code_i K_code_t^T (exact integers);
                       S = (s_Q,i s_K,t A + b_j) / 8, masked entries -inf.
  F6  P~ codes         per row and 64-key tile: m = max of the tile row;
                       P^ = exp(S - m); code = round_half_even(127 P^) in [0,127]
                       (fixed scale 1/127 on P~ in [0,1]).
  F7  PV tile          B = P~_code V_code_t (exact integers).
  F8  combine          M = max_t m_t, w_t = exp(m_t - M),
                       l = sum_t w_t sum_j P~_code / 127   (the row sum of the
                       quantized probabilities, so O is exactly the normalized
                       product of the dequantized P~ and V),
                       O = sum_t w_t (s_V,t / 127) B_t / l,
                       LSE = M + ln l + (q_raw . mu_k) / 8   (true-score frame).
  B1  backward prep    same codes as the forward; dO quantized with F3 (no
                       centring); Delta = rowsum(dO * O) with the O passed in.
  B2  P = exp(S - (LSE - corr)), masked -> 0.
  B3  P codes          per 64x64 tile, F3 on fp32(P) (codes in [0,127]).
  B4  dV_t += s_P s_dO,i (P_code^T dO_code_i).
  B5  dP = fp16(dO) fp16(V)^T, accumulated exactly (the one 16-bit matmul).
      With int8_dp (the all-INT8 ablation in the SageAttention3 summary's
      table of measured effects, which keeps this product in FP16 because
      quantizing it costs dQ accuracy): dP = s_dO,i s_V,t (dO_code_i
      V_code_t^T) with the F3 codes of dO and V (exact integers).
  B6  dS = P * (dP - Delta) with the unquantized P.
  B7  dS codes         per 64x64 tile, F3 on fp32(dS).
  B8  dQ_i += s_dS s_K,t (dS_code K_code_t)      (smoothed K codes, no mu_k)
  B9  dK_t += s_dS s_Q,i (dS_code^T Q_code_i) + [smooth_q] s_dS colsum(dS_code) mu_q
  B10 dQ, dK scaled by 1/8 = 1/sqrt(64).
  B11 with F0: the gradient through the norm, dx = r (dx_n - x_n mean_c(dx_n x_n))
      with the x_n and r of F0.

With ``rounding=False`` every rounding step is removed (codes are x~/s
unrounded, no float32 or float16 rounding, P~/P/dS unquantized); the result
must then equal the exact attention of ``oracle.exact`` up to float64
rounding, which pins every scale, bias, correction and mask above.

Integer tile products are formed with float64 matmuls; every partial sum is an
integer of magnitude <= 64 * 127^2 < 2^53, hence exact in any order.
"""
from __future__ import annotations

import math
from dataclasses import dataclass

import numpy as np

BLK = 64                 # tokens per quantization block (and per tile side)
D = 64                   # head dimension
SCALE = 1.0 / 8.0        # 1/sqrt(64), exact
A_MIN = 2.0 ** -100      # absmax below this -> an all-zero block
_F127 = np.float32(127.0)


# ---------------------------------------------------------------- F0

QK_NORM_EPS = 1e-6


def bf16_rne(x) -> np.ndarray:
    """Round float32 values to bfloat16 (round half to even); float32 result."""
    u = np.asarray(x, np.float32).view(np.uint32).astype(np.uint64)
    u = ((u + 0x7FFF + ((u >> 16) & 1)) >> 16) << 16
    return u.astype(np.uint32).view(np.float32)


def qk_norm_rows(x, rounding: bool = True):
    """F0 for one head: (x_n, r).  The sum of squares is the correctly rounded
    float64 sum (fsum) of the exact float64 squares of the bf16 inputs;
    r = 1/sqrt(sum/64 + 1e-6) in float64 rounded once to float32;
    x_n = bf16(fp32(x * r)).  Without rounding: x_n = x r in float64."""
    x64 = np.asarray(x, np.float64)
    ss = np.array([math.fsum((row * row).tolist()) for row in x64])
    r64 = 1.0 / np.sqrt(ss / 64.0 + QK_NORM_EPS)
    if not rounding:
        return x64 * r64[:, None], r64
    r = r64.astype(np.float32)
    return bf16_rne(np.asarray(x, np.float32) * r[:, None]), r


def qk_norm_grad(dxn, xn, r) -> np.ndarray:
    """B11: dx = r (dx_n - x_n mean_c(dx_n x_n)), rows of one head."""
    dxn = np.asarray(dxn, np.float64)
    xn = np.asarray(xn, np.float64)
    return np.asarray(r, np.float64)[:, None] * (dxn - xn * np.mean(dxn * xn, axis=1, keepdims=True))


# ---------------------------------------------------------------- F1, F3

def exact_mean_f32(x: np.ndarray, n: int) -> np.ndarray:
    """F1: per-column mean of the first n rows of x (float32 values), formed as
    the correctly rounded float64 sum (math.fsum) divided by n in float64 and
    rounded to float32."""
    x = np.asarray(x, np.float64)[:n]
    s = np.array([math.fsum(x[:, c].tolist()) for c in range(x.shape[1])])
    return (s / np.float64(n)).astype(np.float32)


def sum_order_free(x: np.ndarray) -> bool:
    """True if a float64 sum of these values is exact in every order: with u
    the smallest power of two that divides every value, each partial sum is a
    multiple of u, and all of them fit when sum|x| < 2^53 u."""
    x = np.asarray(x, np.float64).ravel()
    nz = x[x != 0]
    if nz.size == 0:
        return True
    f, e = np.frexp(np.abs(nz))                  # |x| = f 2^e, f in [0.5, 1)
    m = (f * 2.0 ** 53).astype(np.int64)         # exact 53-bit integer mantissas
    low = m & -m                                 # lowest set bit of each mantissa
    u = np.min(np.ldexp(low.astype(np.float64), e - 53))
    return float(np.sum(np.abs(nz))) < 2.0 ** 53 * u


def block_scale(a, rounding: bool = True):
    """F3 scale and inverse for one block absmax a (float32 if rounding)."""
    if rounding:
        a = np.float32(a)
        if not (a >= A_MIN):
            return np.float32(0.0), np.float32(0.0)
        # IEEE float32 divisions: the correctly rounded a/127 and 127/a
        return np.float32(a / _F127), np.float32(_F127 / a)
    a = float(a)
    if a == 0.0:
        return 0.0, 0.0
    return a / 127.0, 127.0 / a


def block_codes(x, inv, rounding: bool = True) -> np.ndarray:
    """F3 codes: round-half-even of the exact product x * inv (x, inv float32)."""
    prod = np.asarray(x, np.float64) * np.float64(inv)
    if not rounding:
        return prod
    return np.clip(np.rint(prod), -127.0, 127.0)


def quantize_rows(x: np.ndarray, n: int, rounding: bool = True):
    """F3 over a [Np, 64] array in blocks of 64 rows; rows >= n are padding
    (code 0, excluded from the absmax).  Returns (codes [Np,64] float64,
    scales [T])."""
    np_rows = x.shape[0]
    T = np_rows // BLK
    codes = np.zeros(x.shape, np.float64)
    scales = np.zeros(T, np.float32 if rounding else np.float64)
    for t in range(T):
        r0, r1 = t * BLK, min(n, (t + 1) * BLK)
        if r1 <= r0:
            continue
        blk = x[r0:r1]
        a = np.max(np.abs(blk))
        s, inv = block_scale(a, rounding)
        scales[t] = s
        codes[r0:r1] = block_codes(blk, inv, rounding)
    return codes, scales


def quantize_tiles(x: np.ndarray, rounding: bool = True):
    """F3 applied per 64x64 tile of a [R, C] array (R, C multiples of 64) of
    values already masked to 0 where excluded (B3, B7).  Returns (codes,
    scales [R/64, C/64])."""
    R, C = x.shape
    I, J = R // BLK, C // BLK
    xt = x.reshape(I, BLK, J, BLK)
    if rounding:
        xt = xt.astype(np.float32)
    a = np.max(np.abs(xt), axis=(1, 3))
    scales = np.zeros((I, J), np.float32 if rounding else np.float64)
    invs = np.zeros((I, J), np.float32 if rounding else np.float64)
    for i in range(I):
        for j in range(J):
            scales[i, j], invs[i, j] = block_scale(a[i, j], rounding)
    prod = xt.astype(np.float64) * invs.astype(np.float64)[:, None, :, None]
    codes = np.clip(np.rint(prod), -127.0, 127.0) if rounding else prod
    return codes.reshape(R, C), scales


# ---------------------------------------------------------------- F1-F4

@dataclass
class Prepared:
    """Per-head quantized operands (F1-F4)."""
    N: int
    T: int
    mu_q: np.ndarray     # [64] (zeros unless smooth_q)
    mu_k: np.ndarray     # [64] (zeros unless smooth_k)
    qc: np.ndarray       # [Np, 64] codes (float64 integers)
    kc: np.ndarray
    vc: np.ndarray
    sq: np.ndarray       # [T]
    sk: np.ndarray
    sv: np.ndarray
    b: np.ndarray        # [Np] per-key bias (F4), 0 for padded keys
    corr: np.ndarray     # [Np] (q_raw . mu_k) / 8, 0 for padded rows
    q_raw: np.ndarray    # [N, 64] float64 query values the scores use (x_n with F0)
    rounding: bool
    k_in: np.ndarray = None   # [N, 64] float64 key values the scores use (x_n with F0)
    rq: np.ndarray = None     # [N] F0 factors (None without QK-norm)
    rk: np.ndarray = None


def prepare(q, k, v, smooth_q: bool, smooth_k: bool, rounding: bool = True, qk_norm: bool = False) -> Prepared:
    """F0-F4 for one head.  q, k, v: [N, 64] arrays holding bf16 values."""
    dt = np.float32 if rounding else np.float64
    rq = rk = None
    if qk_norm:
        q, rq = qk_norm_rows(q, rounding)
        k, rk = qk_norm_rows(k, rounding)
    q = np.asarray(q, dt)
    k = np.asarray(k, dt)
    v = np.asarray(v, dt)
    N = q.shape[0]
    T = (N + BLK - 1) // BLK
    Np = T * BLK

    def mean(x):
        if rounding:
            return exact_mean_f32(x, N)
        return np.mean(np.asarray(x, np.float64), axis=0)

    zero = np.zeros(D, np.float32 if rounding else np.float64)
    mu_q = mean(q) if smooth_q else zero
    mu_k = mean(k) if smooth_k else zero

    def centre(x, mu):
        out = np.zeros((Np, D), np.float32 if rounding else np.float64)
        if rounding:
            out[:N] = np.float32(x) - np.float32(mu)       # IEEE float32 subtract
        else:
            out[:N] = np.asarray(x, np.float64) - np.asarray(mu, np.float64)
        return out

    qc, sq = quantize_rows(centre(q, mu_q), N, rounding)
    kc, sk = quantize_rows(centre(k, mu_k), N, rounding)
    vc, sv = quantize_rows(centre(v, zero), N, rounding)
    khat = kc * np.repeat(np.asarray(sk, np.float64), BLK)[:, None]
    b = khat @ np.asarray(mu_q, np.float64)
    corr = np.zeros(Np)
    corr[:N] = (np.asarray(q, np.float64) @ np.asarray(mu_k, np.float64)) * SCALE
    return Prepared(N, T, mu_q, mu_k, qc, kc, vc, sq, sk, sv, b, corr,
                    np.asarray(q, np.float64), rounding, np.asarray(k, np.float64), rq, rk)


def _score_block(pp: Prepared, rows: np.ndarray, cols: np.ndarray, causal: bool):
    """F5 for padded row indices ``rows`` x padded key indices ``cols``.
    Returns (A exact integers, S with -inf where masked, keep mask)."""
    A = pp.qc[rows] @ pp.kc[cols].T
    sq = np.asarray(pp.sq, np.float64)[rows // BLK]
    sk = np.asarray(pp.sk, np.float64)[cols // BLK]
    S = (sq[:, None] * sk[None, :] * A + pp.b[cols][None, :]) * SCALE
    keep = (cols[None, :] < pp.N) & (rows[:, None] < pp.N)
    if causal:
        keep &= cols[None, :] <= rows[:, None]
    return A, np.where(keep, S, -np.inf), keep


def _blocks_rows(blocks) -> np.ndarray:
    return np.concatenate([np.arange(i * BLK, (i + 1) * BLK) for i in blocks])


# ---------------------------------------------------------------- forward

def fwd_head(pp: Prepared, causal: bool, qblocks=None, reading: str = "B",
             chunk_blocks: int = 4, return_codes: bool = False):
    """F5-F8 for the query blocks ``qblocks`` (default all).  Returns
    (O [R,64] float64, LSE [R]) for the padded rows of those blocks (rows
    >= N are meaningless), plus (codes, m) if return_codes.

    reading "B": the P~ reference max is the tile-row max (codes do not depend
    on the kv order).  reading "A": the running max over tiles 0..t, i.e. the
    plain FlashAttention-2 online max (an alternative kept for comparison)."""
    T = pp.T
    if qblocks is None:
        qblocks = list(range(T))
    outs_o, outs_l, outs_c, outs_m = [], [], [], []
    cols = np.arange(T * BLK)
    vcb = pp.vc.reshape(T, BLK, D)
    svt = np.asarray(pp.sv, np.float64)
    for c0 in range(0, len(qblocks), chunk_blocks):
        rows = _blocks_rows(qblocks[c0:c0 + chunk_blocks])
        R = rows.size
        _, S, keep = _score_block(pp, rows, cols, causal)
        St = S.reshape(R, T, BLK)
        kt = keep.reshape(R, T, BLK)
        m = np.max(St, axis=2)                                   # [R, T]
        if reading == "A":
            m = np.maximum.accumulate(m, axis=1)
        elif reading != "B":
            raise ValueError(reading)
        mf = np.where(np.isfinite(m), m, 0.0)
        with np.errstate(invalid="ignore"):
            phat = np.where(kt, np.exp(St - mf[:, :, None]), 0.0)
        if pp.rounding:
            codes = np.rint(127.0 * phat)
        else:
            codes = 127.0 * phat
        Bt = np.matmul(codes.transpose(1, 0, 2), vcb)            # [T, R, 64] exact ints
        M = np.max(m, axis=1)                                    # [R]
        with np.errstate(invalid="ignore"):
            w = np.where(np.isfinite(m), np.exp(mf - M[:, None]), 0.0)   # [R, T]
        l = np.sum(w * np.sum(codes, axis=2), axis=1) / 127.0    # [R]
        acc = np.einsum("rt,trc->rc", w * (svt / 127.0)[None, :], Bt)
        with np.errstate(invalid="ignore", divide="ignore"):
            o = acc / l[:, None]
            lse = M + np.log(l) + pp.corr[rows]
        outs_o.append(o)
        outs_l.append(lse)
        if return_codes:
            outs_c.append(codes.reshape(R, T * BLK))
            outs_m.append(m)
    o = np.concatenate(outs_o)
    lse = np.concatenate(outs_l)
    if return_codes:
        return o, lse, np.concatenate(outs_c), np.concatenate(outs_m)
    return o, lse


def fwd_head_loop(pp: Prepared, causal: bool, reading: str = "B"):
    """F5-F8 written as the tile-by-tile online loop a flash kernel runs
    (running max M, running sum l, rescale factor alpha = exp(M_old - M_new)),
    one row block at a time.  A second formulation of ``fwd_head`` used only to
    pin it: same codes, same O and LSE up to float64 rounding."""
    T = pp.T
    o = np.zeros((T * BLK, D))
    lse = np.zeros(T * BLK)
    codes_all = np.zeros((T * BLK, T * BLK))
    for i in range(T):
        rows = np.arange(i * BLK, (i + 1) * BLK)
        M = np.full(BLK, -np.inf)
        l = np.zeros(BLK)
        acc = np.zeros((BLK, D))
        m_run = np.full(BLK, -np.inf)
        for t in range(T):
            cols = np.arange(t * BLK, (t + 1) * BLK)
            _, S, keep = _score_block(pp, rows, cols, causal)
            if not keep.any():
                continue
            m_tile = np.max(S, axis=1)
            m_run = np.maximum(m_run, m_tile)
            m_ref = m_tile if reading == "B" else m_run
            live = np.isfinite(m_ref)
            mr = np.where(live, m_ref, 0.0)
            with np.errstate(invalid="ignore"):
                phat = np.where(keep, np.exp(S - mr[:, None]), 0.0)
            c = np.rint(127.0 * phat) if pp.rounding else 127.0 * phat
            codes_all[rows[:, None], cols[None, :]] = c
            Bt = c @ pp.vc[cols]
            M_new = np.where(live, np.maximum(M, mr), M)
            with np.errstate(invalid="ignore"):
                alpha = np.where(np.isfinite(M), np.exp(M - M_new), 0.0)
                w = np.where(live, np.exp(mr - M_new), 0.0)
            l = l * alpha + w * np.sum(c, axis=1) / 127.0
            acc = acc * alpha[:, None] + (w * float(pp.sv[t]) / 127.0)[:, None] * Bt
            M = M_new
        with np.errstate(invalid="ignore", divide="ignore"):
            o[rows] = acc / l[:, None]
            lse[rows] = M + np.log(l) + pp.corr[rows]
    return o, lse, codes_all


def fwd(q, k, v, causal: bool, smooth_q: bool, smooth_k: bool, rounding: bool = True,
        reading: str = "B", qk_norm: bool = False):
    """Faithful forward over [B, H, N, 64] arrays of bf16 values.
    Returns (O float64 [B,H,N,64], LSE float64 [B,H,N])."""
    B, H, N, _ = q.shape
    o = np.zeros((B, H, N, D))
    lse = np.zeros((B, H, N))
    for b in range(B):
        for h in range(H):
            pp = prepare(q[b, h], k[b, h], v[b, h], smooth_q, smooth_k, rounding, qk_norm)
            ob, lb = fwd_head(pp, causal, reading=reading)
            o[b, h], lse[b, h] = ob[:N], lb[:N]
    return o, lse


# ---------------------------------------------------------------- backward

@dataclass
class BwdPrepared:
    pp: Prepared
    doc: np.ndarray      # [Np, 64] dO codes
    sdo: np.ndarray      # [T]
    do16: np.ndarray     # [Np, 64] float64 of fp16(dO) (or dO if not rounding)
    v16: np.ndarray      # [Np, 64]
    delta: np.ndarray    # [Np]
    lsep: np.ndarray     # [Np] LSE - corr (+inf on padded rows)
    int8_dp: bool = False


def prepare_bwd(pp: Prepared, v, o, lse, do, int8_dp: bool = False) -> BwdPrepared:
    """B1 for one head.  o: forward output values (e.g. bf16), lse: float32
    natural-log LSE in the true-score frame, do: bf16 values.  int8_dp selects
    the all-INT8 form of B5."""
    N, T = pp.N, pp.T
    Np = T * BLK
    r = pp.rounding
    do32 = np.zeros((Np, D), np.float32 if r else np.float64)
    do32[:N] = np.asarray(do, np.float32 if r else np.float64)
    doc, sdo = quantize_rows(do32, N, r)
    do16 = np.zeros((Np, D))
    v16 = np.zeros((Np, D))
    if r:
        do16[:N] = np.asarray(do, np.float32).astype(np.float16).astype(np.float64)
        v16[:N] = np.asarray(v, np.float32).astype(np.float16).astype(np.float64)
    else:
        do16[:N] = np.asarray(do, np.float64)
        v16[:N] = np.asarray(v, np.float64)
    delta = np.zeros(Np)
    delta[:N] = np.sum(np.asarray(do, np.float64) * np.asarray(o, np.float64), axis=1)
    lsep = np.full(Np, np.inf)
    lsep[:N] = np.asarray(lse, np.float64) - pp.corr[:N]
    return BwdPrepared(pp, doc, sdo, do16, v16, delta, lsep, int8_dp)


def bwd_tiles(bp: BwdPrepared, iblocks, tblocks, causal: bool):
    """B2-B7 on the tile grid iblocks x tblocks.  Returns a dict with P, dS
    (float64), their codes and per-tile scales, and the score integers A."""
    pp = bp.pp
    r = pp.rounding
    rows = _blocks_rows(iblocks)
    cols = _blocks_rows(tblocks)
    A, S, keep = _score_block(pp, rows, cols, causal)
    with np.errstate(invalid="ignore", over="ignore"):
        P = np.where(keep, np.exp(S - bp.lsep[rows][:, None]), 0.0)
    Pq = P.astype(np.float32) if r else P
    cP, sP = quantize_tiles(Pq, r)
    if bp.int8_dp:
        w = np.asarray(bp.sdo, np.float64)[rows // BLK][:, None] * np.asarray(pp.sv, np.float64)[cols // BLK][None, :]
        dP = w * (bp.doc[rows] @ pp.vc[cols].T)
    else:
        dP = bp.do16[rows] @ bp.v16[cols].T
    dS = np.where(keep, P * (dP - bp.delta[rows][:, None]), 0.0)
    dSq = dS.astype(np.float32) if r else dS
    cdS, sdS = quantize_tiles(dSq, r)
    return {"rows": rows, "cols": cols, "A": A, "P": P, "dP": dP, "dS": dS,
            "cP": cP, "sP": sP, "cdS": cdS, "sdS": sdS}


def _tile_products(c: np.ndarray, x_codes: np.ndarray, I: int, J: int, transpose: bool):
    """Exact per-tile integer products.  c: [I*64, J*64] codes.
    transpose=False: out[i, j] = c_ij @ x_codes[j-block]  -> [I, J, 64, 64]
    transpose=True : out[i, j] = c_ij^T @ x_codes[i-block] -> [I, J, 64, 64]"""
    ct = c.reshape(I, BLK, J, BLK).transpose(0, 2, 1, 3)        # [I, J, 64r, 64c]
    if transpose:
        xb = x_codes.reshape(I, BLK, D)[:, None]                 # [I, 1, 64, 64]
        return np.matmul(ct.transpose(0, 1, 3, 2), xb)
    xb = x_codes.reshape(J, BLK, D)[None]                        # [1, J, 64, 64]
    return np.matmul(ct, xb)


def bwd_head(bp: BwdPrepared, causal: bool, qblocks=None, kblocks=None, chunk: int = 4):
    """B2-B10 for one head.  dQ is returned for the rows of ``qblocks``
    (default all), dK and dV for the keys of ``kblocks`` (default all).
    Returns (dQ [len(qblocks)*64, 64], dK [len(kblocks)*64, 64], dV [...])."""
    pp = bp.pp
    T = pp.T
    allb = list(range(T))
    qblocks = allb if qblocks is None else list(qblocks)
    kblocks = allb if kblocks is None else list(kblocks)
    sq = np.asarray(pp.sq, np.float64)
    sk = np.asarray(pp.sk, np.float64)
    sdo = np.asarray(bp.sdo, np.float64)
    mu_q = np.asarray(pp.mu_q, np.float64)

    # dQ: rows of qblocks against every key block (B8)
    dq = np.zeros((len(qblocks) * BLK, D))
    for c0 in range(0, len(qblocks), chunk):
        ib = qblocks[c0:c0 + chunk]
        tl = bwd_tiles(bp, ib, allb, causal)
        I = len(ib)
        prod = _tile_products(tl["cdS"], pp.kc, I, T, transpose=False)     # [I, T, 64, 64]
        w = np.asarray(tl["sdS"], np.float64) * sk[None, :]
        dq[c0 * BLK:(c0 + I) * BLK] = np.einsum("it,itrc->irc", w, prod).reshape(I * BLK, D) * SCALE

    # dK, dV: keys of kblocks against every query block (B4, B9)
    dk = np.zeros((len(kblocks) * BLK, D))
    dv = np.zeros((len(kblocks) * BLK, D))
    for c0 in range(0, len(kblocks), chunk):
        tb = kblocks[c0:c0 + chunk]
        J = len(tb)
        for i0 in range(0, T, max(1, 16 // J)):
            ib = allb[i0:i0 + max(1, 16 // J)]
            I = len(ib)
            tl = bwd_tiles(bp, ib, tb, causal)
            iidx = np.asarray(ib)
            pv = _tile_products(tl["cP"], bp.doc[_blocks_rows(ib)], I, J, transpose=True)
            wv = np.asarray(tl["sP"], np.float64) * sdo[iidx][:, None]
            dv[c0 * BLK:(c0 + J) * BLK] += np.einsum("ij,ijrc->jrc", wv, pv).reshape(J * BLK, D)
            pk = _tile_products(tl["cdS"], pp.qc[_blocks_rows(ib)], I, J, transpose=True)
            wk = np.asarray(tl["sdS"], np.float64) * sq[iidx][:, None]
            dkc = np.einsum("ij,ijrc->jrc", wk, pk)
            if np.any(mu_q != 0):
                colsum = tl["cdS"].reshape(I, BLK, J, BLK).sum(axis=1)             # [I, J, 64]
                g = np.einsum("ij,ijr->jr", np.asarray(tl["sdS"], np.float64), colsum)
                dkc = dkc + g[:, :, None] * mu_q[None, None, :]
            dk[c0 * BLK:(c0 + J) * BLK] += dkc.reshape(J * BLK, D) * SCALE
    return dq, dk, dv


def norm_grads(pp: Prepared, dq, dk, qrows=None, krows=None):
    """B11 applied to dQ rows ``qrows`` and dK rows ``krows`` (default: the
    first len(dq) / len(dk) tokens); identity without F0."""
    if pp.rq is None:
        return dq, dk
    qrows = np.arange(len(dq)) if qrows is None else np.asarray(qrows)
    krows = np.arange(len(dk)) if krows is None else np.asarray(krows)
    return (qk_norm_grad(dq, pp.q_raw[qrows], pp.rq[qrows]), qk_norm_grad(dk, pp.k_in[krows], pp.rk[krows]))


def bwd(q, k, v, o, lse, do, causal: bool, smooth_q: bool, smooth_k: bool,
        rounding: bool = True, int8_dp: bool = False, qk_norm: bool = False):
    """Faithful backward over [B, H, N, 64] arrays.  ``o``/``lse`` are the
    forward outputs handed to the backward (O as bf16 values, LSE float32).
    Returns (dQ, dK, dV) float64 [B,H,N,64], the gradients of the raw Q, K
    (through the norm with qk_norm) and V."""
    B, H, N, _ = q.shape
    out = [np.zeros((B, H, N, D)) for _ in range(3)]
    for b in range(B):
        for h in range(H):
            pp = prepare(q[b, h], k[b, h], v[b, h], smooth_q, smooth_k, rounding, qk_norm)
            bp = prepare_bwd(pp, v[b, h], o[b, h], lse[b, h], do[b, h], int8_dp)
            dq, dk, dv = bwd_head(bp, causal)
            dq, dk = norm_grads(pp, dq[:N], dk[:N])
            out[0][b, h], out[1][b, h], out[2][b, h] = dq, dk, dv[:N]
    return tuple(out)
