"""Pins for oracle.faithful against things other than itself: brute-force
integer products, an exact-rational re-derivation of the quantizer, hand-derived
quantizer cases, the rounding-free reduction to exact attention, a literal
online tile loop, and the exactness of the smoothing-mean sums."""
import math
from fractions import Fraction

import numpy as np
import pytest

import workloads as W
from oracle import exact, faithful as F, metrics as M


def _f32(bits):
    return W.bf16_bits_to_f32(bits)


# ------------------------------------------------------------ integer products

def _brute(a, b):
    n, kk = a.shape
    m = b.shape[1]
    out = np.zeros((n, m), dtype=np.int64)
    for i in range(n):
        for j in range(m):
            s = 0
            for t in range(kk):
                s += int(a[i, t]) * int(b[t, j])
            out[i, j] = s
    return out


@pytest.mark.parametrize("kind", ["random", "extreme"])
def test_int_matmul_exact(kind):
    r = np.random.default_rng(1)
    if kind == "random":
        a = r.integers(-127, 128, (64, 64))
        b = r.integers(-127, 128, (64, 64))
    else:
        a = np.where(r.random((64, 64)) < 0.5, -127, 127)
        b = np.where(r.random((64, 64)) < 0.5, -127, 127)
        a[0, :] = 127
        b[:, 0] = 127            # one entry hits 64 * 127^2
    ref = _brute(a, b)
    got = a.astype(np.float64) @ b.astype(np.float64)
    assert np.array_equal(got.astype(np.int64), ref)
    assert ref.max() == 64 * 127 * 127 or kind == "random"
    # the oracle's per-tile product helper on a 2x2 tile grid
    c = r.integers(-127, 128, (128, 128)).astype(np.float64)
    x = r.integers(-127, 128, (128, 64)).astype(np.float64)
    p = F._tile_products(c, x, 2, 2, transpose=False)
    pt = F._tile_products(c, x, 2, 2, transpose=True)
    for i in range(2):
        for j in range(2):
            tile = c[64 * i:64 * i + 64, 64 * j:64 * j + 64].astype(np.int64)
            assert np.array_equal(p[i, j].astype(np.int64), _brute(tile, x[64 * j:64 * j + 64].astype(np.int64)))
            assert np.array_equal(pt[i, j].astype(np.int64), _brute(tile.T, x[64 * i:64 * i + 64].astype(np.int64)))


# ------------------------------------------------------------ quantizer

def _rne(fr: Fraction) -> int:
    fl = fr.numerator // fr.denominator
    rem = fr - fl
    if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and fl % 2 == 1):
        fl += 1
    return fl


def _f32_round(fr: Fraction) -> Fraction:
    """Round an exact rational to the nearest float32 (ties to even), normal range."""
    if fr == 0:
        return Fraction(0)
    sign = -1 if fr < 0 else 1
    x = abs(fr)
    e = x.numerator.bit_length() - x.denominator.bit_length()
    if Fraction(2) ** e > x:
        e -= 1
    ulp = Fraction(2) ** (e - 23)
    return sign * _rne(x / ulp) * ulp


def test_quantizer_matches_exact_rationals():
    """Scale, inverse and codes re-derived with exact rationals, with float32
    rounding done by hand, agree bit for bit with the float32 route: the scale
    is the correctly rounded absmax/127 and the inverse the correctly rounded
    127/absmax (the SageBwd reading of "absmax/127 scales")."""
    r = np.random.default_rng(7)
    n_checked = 0
    n_shortcut_differs = 0
    r127 = _f32_round(Fraction(1, 127))
    for trial in range(2000):
        scale = float(np.exp(r.uniform(-12, 6)))
        x = (r.standard_normal(512) * scale).astype(np.float32)
        a = np.max(np.abs(x))
        s, inv = F.block_scale(a)
        fa = Fraction(float(a))
        s_ref = _f32_round(fa / 127)
        inv_ref = _f32_round(Fraction(127) / fa)
        assert Fraction(float(s)) == s_ref
        assert Fraction(float(inv)) == inv_ref
        # a planted mistake, the one-multiply a * fp32(1/127), differs from the
        # quotient on some of these blocks, so this check would catch it
        n_shortcut_differs += _f32_round(fa * r127) != s_ref
        codes = F.block_codes(x, inv)
        for xi, ci in zip(x.tolist(), codes.tolist()):
            assert ci == max(-127, min(127, _rne(Fraction(xi) * inv_ref)))
            n_checked += 1
    assert n_checked == 2000 * 512        # 1 024 000 values
    assert n_shortcut_differs > 20


def test_block_scale_quotient_exhaustive_binade():
    """s = fp32(a/127) for every float32 a in [1, 2) (all 2^23 mantissas),
    against the quotient rounded by hand from an exact integer division: with
    a = m 2^-23, a/127 = m / (127 2^23); its float32 rounding is read off the
    integer quotient and remainder of m 2^k / 127.  Division by 127 commutes
    with scaling by powers of two, so this covers every normal a."""
    m = np.arange(2 ** 23, dtype=np.int64) + 2 ** 23          # a = m 2^-23 in [1, 2)
    a = m.astype(np.float32) * np.float32(2.0 ** -23)
    s = np.array([F.block_scale(v)[0] for v in a[:: 4099]])  # the oracle's route on a sample
    # exact: a/127 lies in [2^-7, 2^-6) (float32 ulp 2^-30, quotient m 2^7 / 127
    # in ulps) for m < 127 2^17, else in [2^-6, 2^-5) (ulp 2^-29, m 2^6 / 127)
    hi = m >= 127 * 2 ** 17
    sh = np.where(hi, 6, 7)
    num = m << sh
    q, rem = num // 127, num % 127
    up = (2 * rem > 127) | ((2 * rem == 127) & (q % 2 == 1))
    ref = ((q + up).astype(np.float64) * np.where(hi, 2.0 ** -29, 2.0 ** -30)).astype(np.float32)
    assert np.array_equal(s, ref[:: 4099])
    got = (a / np.float32(127.0)).astype(np.float32)          # the oracle's float32 division, all of them
    assert np.array_equal(got, ref)


def _tile_loop(x, rounding=True):
    """B3/B7 written as a loop over 64x64 tiles of the pinned block_scale and
    block_codes (a second formulation of quantize_tiles)."""
    I, J = x.shape[0] // 64, x.shape[1] // 64
    codes = np.zeros(x.shape)
    scales = np.zeros((I, J), np.float32)
    for i in range(I):
        for j in range(J):
            t = np.asarray(x[64 * i:64 * i + 64, 64 * j:64 * j + 64], np.float32)
            s, inv = F.block_scale(np.max(np.abs(t)))
            scales[i, j] = s
            codes[64 * i:64 * i + 64, 64 * j:64 * j + 64] = F.block_codes(t, inv)
    return codes, scales


def _planted_per_row(x):
    """A plausible mistake: one absmax per row of each tile instead of per tile."""
    codes = np.zeros(x.shape)
    for r0 in range(0, x.shape[0]):
        for j in range(x.shape[1] // 64):
            t = np.asarray(x[r0, 64 * j:64 * j + 64], np.float32)
            _, inv = F.block_scale(np.max(np.abs(t)))
            codes[r0, 64 * j:64 * j + 64] = F.block_codes(t, inv)
    return codes


def test_quantize_tiles_against_tile_loop():
    """quantize_tiles (B3, B7, with rounding) equals the per-tile loop over the
    pinned scalar quantizer, on signed dS-like and non-negative P-like tiles
    with exact ties and zero tiles; a per-row absmax would not."""
    r = np.random.default_rng(11)
    x = (r.standard_normal((192, 128)) * np.exp(r.uniform(-6, 3, (192, 1)))).astype(np.float32)
    x[64:128, 64:128] = 0.0                                   # an all-zero tile
    x[0:64, 0:64] = np.abs(x[0:64, 0:64])                     # a P-like tile
    x[5, 3] = np.max(np.abs(x[0:64, 0:64])) * 2.5 / 127       # exact-ish ties near 2.5 codes
    c, s = F.quantize_tiles(x)
    c_ref, s_ref = _tile_loop(x)
    assert np.array_equal(s, s_ref)
    assert np.array_equal(c, c_ref)
    assert np.max(np.abs(c)) == 127 and np.all(np.abs(c) <= 127)
    assert not np.array_equal(_planted_per_row(x), c_ref)


def test_quantizer_hand_cases():
    # absmax 1 -> s = fp32(1/127), inv = 127; x * 127 exactly
    x = np.array([1.0, -0.5, 0.25, 2.5 / 127, 3.5 / 127, -1.0, 0.0], np.float32)
    s, inv = F.block_scale(np.max(np.abs(x)))
    assert inv == np.float32(127.0)
    assert s == np.float32(1.0) / np.float32(127.0)
    c = F.block_codes(x, inv)
    # 127, -63.5 -> -64 (tie to even), 31.75 -> 32, ~2.5 and ~3.5 depend on the
    # float32 value of 2.5/127 (not exactly representable) -> check exactly:
    assert c[0] == 127 and c[1] == -64 and c[2] == 32 and c[5] == -127 and c[6] == 0
    assert c[3] == np.rint(np.float64(x[3]) * 127.0) and c[4] == np.rint(np.float64(x[4]) * 127.0)
    # exact ties: with absmax 127, inv = 1 and codes are round-half-even of x
    y = np.array([127.0, 2.5, 3.5, -2.5, -0.5, 0.5, 1.5, 126.5], np.float32)
    s, inv = F.block_scale(127.0)
    assert inv == 1.0 and s == 1.0
    assert F.block_codes(y, inv).tolist() == [127, 2, 4, -2, -0, 0, 2, 126]
    # all-zero and tiny blocks
    assert F.block_scale(0.0) == (0.0, 0.0)
    assert F.block_scale(2.0 ** -101) == (0.0, 0.0)
    assert F.block_scale(2.0 ** -99)[0] > 0


def test_quantizer_error_bound():
    r = np.random.default_rng(3)
    for _ in range(50):
        x = (r.standard_normal((64, 64)) * r.uniform(0.01, 30)).astype(np.float32)
        codes, s = F.quantize_rows(x, 64)
        a = np.max(np.abs(x))
        assert np.max(np.abs(codes)) == 127
        assert np.abs(codes[np.unravel_index(np.argmax(np.abs(x)), x.shape)]) == 127
        err = np.abs(x.astype(np.float64) - float(s[0]) * codes)
        assert np.max(err) <= float(s[0]) * 0.5 * (1 + 1e-6) + a * 1e-7


def test_quantize_rows_ragged_padding():
    r = np.random.default_rng(4)
    x = np.zeros((128, 64), np.float32)
    x[:100] = r.standard_normal((100, 64))
    x[100:] = 1000.0                   # padding content must be ignored
    codes, s = F.quantize_rows(x, 100)
    assert np.all(codes[100:] == 0)
    assert np.isclose(float(s[1]), np.max(np.abs(x[64:100])) / 127, rtol=1e-6)


# ------------------------------------------------------------ smoothing means

def test_exact_mean_and_order_free():
    r = np.random.default_rng(11)
    x = W.bf16_bits_to_f32(W.f32_to_bf16_bits(r.standard_normal((1000, 64)).astype(np.float32) * 3 + 1))
    mu = F.exact_mean_f32(x, 1000)
    for c in range(64):
        ref = sum(Fraction(float(v)) for v in x[:, c]) / 1000
        # fp32(fp64(exact sum) / n): reproduce by hand
        s64 = float(sum(Fraction(float(v)) for v in x[:, c]))   # exact sum fits: order-free below
        assert np.float32(s64 / 1000.0) == mu[c]
        assert abs(float(mu[c]) - float(ref)) <= abs(float(ref)) * 2 ** -23 + 1e-30
    assert F.sum_order_free(x[:, 0])
    # a value far below the others breaks order-freedom
    y = np.array([1.0, 2.0 ** -60, 3.0])
    assert not F.sum_order_free(np.concatenate([y, np.full(10, 2.0 ** 40)]))
    assert F.sum_order_free(np.array([0.5, 0.25, 1.5]))


@pytest.mark.parametrize("name", ["tiny", "pretrain", "llama8k", "video"])
def test_workload_means_order_free(name):
    """The GPU sums K (and Q) in float64 in its own order; the result equals
    the correctly rounded sum whenever the sum is order-free, which holds for
    the sampled heads of these seeded inputs (the GPU tests re-check the heads
    they compare)."""
    w = W.WORKLOADS[name]
    heads = [(b, h) for b in range(w.B) for h in range(w.H)][:4]
    for b, h in heads:
        x = W.make_head(w, b, h)
        for key in ("k", "q"):
            v = _f32(x[key])
            for c in range(64):
                assert F.sum_order_free(v[:, c]), (name, key, b, h, c)


# ------------------------------------------------------------ reduction to exact

CASES = [
    dict(N=128, causal=False, sq=False, sk=True, dist="normal"),
    dict(N=100, causal=True, sq=True, sk=True, dist="kbias"),
    dict(N=129, causal=False, sq=True, sk=False, dist="outlier"),
    dict(N=64, causal=True, sq=False, sk=False, dist="qknorm"),
    dict(N=1, causal=True, sq=True, sk=True, dist="normal"),
]


@pytest.mark.parametrize("int8_dp", [False, True], ids=["fp16dp", "int8dp"])
@pytest.mark.parametrize("case", CASES, ids=lambda c: f"N{c['N']}c{int(c['causal'])}q{int(c['sq'])}k{int(c['sk'])}")
def test_rounding_free_reduces_to_exact(case, int8_dp):
    w = W.custom(1, 2, case["N"], case["causal"], case["sk"], case["sq"], case["dist"], seed_family=31)
    x = {k: _f32(v).astype(np.float64) for k, v in W.make_inputs(w).items()}
    o, lse = F.fwd(x["q"], x["k"], x["v"], w.causal, w.smooth_q, w.smooth_k, rounding=False)
    oe, le = exact.fwd_bh(x["q"], x["k"], x["v"], w.causal)
    assert np.max(np.abs(o - oe)) < 1e-12
    assert np.max(np.abs(lse - le)) < 1e-11
    g = F.bwd(x["q"], x["k"], x["v"], oe, le, x["do"], w.causal, w.smooth_q, w.smooth_k, rounding=False,
              int8_dp=int8_dp)
    ge = exact.bwd_bh(x["q"], x["k"], x["v"], x["do"], w.causal)
    for a, b in zip(g, ge):
        assert np.max(np.abs(a - b)) < 1e-11 * max(1.0, np.max(np.abs(b)))


def test_planted_mistakes_are_caught(monkeypatch):
    """Sanity of the reduction pin: a dropped Q-smoothing bias, a dropped dK
    colsum term or a wrong softmax scale in the oracle each break it."""
    w = W.custom(1, 1, 96, True, True, True, "outlier", seed_family=32)
    x = {k: _f32(v).astype(np.float64) for k, v in W.make_inputs(w).items()}
    oe, le = exact.fwd_bh(x["q"], x["k"], x["v"], True)
    ge = exact.bwd_bh(x["q"], x["k"], x["v"], x["do"], True)

    def err():
        o, _ = F.fwd(x["q"], x["k"], x["v"], True, True, True, rounding=False)
        g = F.bwd(x["q"], x["k"], x["v"], oe, le, x["do"], True, True, True, rounding=False)
        return max(np.max(np.abs(o - oe)), max(np.max(np.abs(a - b)) for a, b in zip(g, ge)))

    assert err() < 1e-10
    real_prepare = F.prepare

    def no_bias(*a, **k):
        pp = real_prepare(*a, **k)
        pp.b = np.zeros_like(pp.b)
        return pp
    monkeypatch.setattr(F, "prepare", no_bias)
    assert err() > 1e-3
    monkeypatch.setattr(F, "prepare", real_prepare)
    monkeypatch.setattr(F, "SCALE", 1.0 / 7.0)
    assert err() > 1e-3
    monkeypatch.setattr(F, "SCALE", 1.0 / 8.0)
    real_mu = F.Prepared

    def no_colsum(*a, **k):
        pp = real_prepare(*a, **k)
        return pp
    # dK without the colsum(dS) mu_q term: zero mu_q only after the bias is formed
    def drop_mu_q(*a, **k):
        pp = real_prepare(*a, **k)
        pp.mu_q = np.zeros_like(pp.mu_q)
        return pp
    monkeypatch.setattr(F, "prepare", drop_mu_q)
    g = F.bwd(x["q"], x["k"], x["v"], oe, le, x["do"], True, True, True, rounding=False)
    assert np.max(np.abs(g[1] - ge[1])) > 1e-3
    assert real_mu is F.Prepared


# ------------------------------------------------------------ online loop

@pytest.mark.parametrize("reading", ["A", "B"])
@pytest.mark.parametrize("causal,N", [(False, 128), (True, 200)])
def test_online_loop_matches_vectorized(reading, causal, N):
    w = W.custom(1, 1, N, causal, True, True, "kbias", seed_family=33)
    x = {k: _f32(v)[0, 0] for k, v in W.make_inputs(w).items()}
    pp = F.prepare(x["q"], x["k"], x["v"], True, True)
    o1, l1, c1, _ = F.fwd_head(pp, causal, reading=reading, return_codes=True)
    o2, l2, c2 = F.fwd_head_loop(pp, causal, reading=reading)
    assert np.array_equal(c1, c2)
    assert np.max(np.abs(o1[:N] - o2[:N])) < 1e-12
    assert np.max(np.abs(l1[:N] - l2[:N])) < 1e-12


# ------------------------------------------------------------ accuracy study

def _study(name, qblocks, kblocks, heads, smooth_q=None):
    """Faithful vs exact on sampled blocks of a workload (one head at a time)."""
    w = W.WORKLOADS[name]
    sq = w.smooth_q if smooth_q is None else smooth_q
    N = w.N
    res = []
    for b, h in heads:
        x = W.make_head(w, b, h)
        q, k, v, do = (_f32(x[n]) for n in ("q", "k", "v", "do"))
        pp = F.prepare(q, k, v, sq, w.smooth_k)
        o, lse = F.fwd_head(pp, w.causal)
        o_bf = _f32(W.f32_to_bf16_bits(o[:N].astype(np.float32)))
        bp = F.prepare_bwd(pp, v, o_bf, lse[:N].astype(np.float32), do)
        dq, dk, dv = F.bwd_head(bp, w.causal, qblocks, kblocks)
        qr = np.concatenate([np.arange(i * 64, min(N, i * 64 + 64)) for i in qblocks])
        kr = np.concatenate([np.arange(t * 64, min(N, t * 64 + 64)) for t in kblocks])
        qi = np.concatenate([np.arange(j * 64, j * 64 + min(64, N - i * 64)) for j, i in enumerate(qblocks)])
        ki = np.concatenate([np.arange(j * 64, j * 64 + min(64, N - t * 64)) for j, t in enumerate(kblocks)])
        oe, le, dqe, dke, dve = exact.sampled(q, k, v, do, w.causal, np.arange(N), kr)
        res.append((M.cos_sim(o[:N], oe), M.cos_sim(dq[qi], dqe[qr]), M.cos_sim(dk[ki], dke),
                    M.cos_sim(dv[ki], dve)))
    return np.array(res)


@pytest.mark.slow
@pytest.mark.parametrize("name,qb,kb", [
    ("tiny", [0, 1], [0, 1]),
    ("pretrain", [0, 5, 31], [0, 16, 31]),
    ("llama8k", [0, 64, 127], [0, 64, 127]),
    ("video", [0, 150, 277], [0, 150, 277]),
])
def test_accuracy_bars(name, qb, kb):
    """The specified scheme meets the stated accuracy bars against exact
    attention: cos >= 0.999 for O, >= 0.99 for dQ, dK, dV (sampled blocks)."""
    r = _study(name, qb, kb, [(0, 0), (0, 1)])
    assert np.all(r[:, 0] >= 0.999), r
    assert np.all(r[:, 1:] >= 0.99), r


# ------------------------------------------------------------ all-INT8 ablation

def test_int8_dp_planted_scale_mistake(monkeypatch):
    """The all-INT8 dP uses the dO scale of the query block: reversing the dO
    block scales after quantization breaks dQ in that mode only (the FP16 dP
    never reads them; dQ does not depend on them otherwise)."""
    w = W.custom(1, 1, 200, True, True, True, "kbias", seed_family=33)
    x = {k: _f32(v).astype(np.float64) for k, v in W.make_inputs(w).items()}
    oe, le = exact.fwd_bh(x["q"], x["k"], x["v"], True)
    ge = exact.bwd_bh(x["q"], x["k"], x["v"], x["do"], True)
    real = F.prepare_bwd

    def reversed_sdo(*a, **k):
        bp = real(*a, **k)
        bp.sdo = bp.sdo[::-1].copy()
        return bp

    def dq_err(int8_dp):
        g = F.bwd(x["q"], x["k"], x["v"], oe, le, x["do"], True, True, True, rounding=False, int8_dp=int8_dp)
        return np.max(np.abs(g[0] - ge[0]))

    assert dq_err(True) < 1e-10 and dq_err(False) < 1e-10
    monkeypatch.setattr(F, "prepare_bwd", reversed_sdo)
    assert dq_err(True) > 1e-3
    assert dq_err(False) < 1e-10


@pytest.mark.parametrize("dist,causal,sq", [("qknorm", True, False), ("kbias", True, True), ("outlier", False, True),
                                             ("normal", False, False)])
def test_int8_dp_ablation_ordering(dist, causal, sq):
    """The pages' ablation (SageAttention3 summary, table of measured effects
    and "Surprising findings"): keeping dO V^T in FP16 gives a more accurate dQ
    than quantizing it to INT8.  On these synthetic heads the same ordering
    holds for dQ and dK against exact attention, and dV (which does not use
    dP) is identical in both modes."""
    w = W.custom(1, 2, 384, causal, True, sq, dist, seed_family=77)
    x = {k: W.bf16_bits_to_f32(v) for k, v in W.make_inputs(w).items()}
    o, lse = F.fwd(x["q"], x["k"], x["v"], causal, sq, True)
    ob = W.bf16_bits_to_f32(W.f32_to_bf16_bits(o.astype(np.float32)))
    g16 = F.bwd(x["q"], x["k"], x["v"], ob, lse.astype(np.float32), x["do"], causal, sq, True)
    g8 = F.bwd(x["q"], x["k"], x["v"], ob, lse.astype(np.float32), x["do"], causal, sq, True, int8_dp=True)
    ge = exact.bwd_bh(*(x[n].astype(np.float64) for n in ("q", "k", "v", "do")), causal)
    for i in (0, 1):
        c16, c8 = M.cos_sim(g16[i], ge[i]), M.cos_sim(g8[i], ge[i])
        print(f"  {dist} {'dQ' if i == 0 else 'dK'} cos fp16 dP {c16:.6f}  int8 dP {c8:.6f}")
        assert c16 > c8
    assert np.array_equal(g16[2], g8[2])


# ------------------------------------------------------------ QK-norm (F0, B11)

def _qk_rows(n, seed, scale_lo=0.05, scale_hi=20.0):
    """bf16 rows of very different sizes, so the norm is far from a no-op."""
    r = np.random.default_rng(seed)
    x = r.standard_normal((n, 64)) * np.exp(r.uniform(np.log(scale_lo), np.log(scale_hi), n))[:, None]
    return F.bf16_rne(x.astype(np.float32))


@pytest.mark.parametrize("causal,sq,sk", [(True, True, True), (False, False, True), (True, False, False)])
def test_rounding_free_reduces_to_exact_qk_norm(causal, sq, sk):
    """F0 and B11 without rounding: faithful = exact attention on QK-normalized
    inputs, gradients carried back through the norm."""
    n = 150
    q, k = _qk_rows(n, 61)[None, None], _qk_rows(n, 62)[None, None]
    r = np.random.default_rng(63)
    v, do = (F.bf16_rne(r.standard_normal((1, 1, n, 64)).astype(np.float32)) for _ in range(2))
    x = {"q": q.astype(np.float64), "k": k.astype(np.float64), "v": v.astype(np.float64), "do": do.astype(np.float64)}
    o, lse = F.fwd(x["q"], x["k"], x["v"], causal, sq, sk, rounding=False, qk_norm=True)
    oe, le = exact.fwd_bh(x["q"], x["k"], x["v"], causal, qk_norm=True)
    assert np.max(np.abs(o - oe)) < 1e-12 and np.max(np.abs(lse - le)) < 1e-11
    g = F.bwd(x["q"], x["k"], x["v"], oe, le, x["do"], causal, sq, sk, rounding=False, qk_norm=True)
    ge = exact.bwd_bh(x["q"], x["k"], x["v"], x["do"], causal, qk_norm=True)
    for a, b in zip(g, ge):
        assert np.max(np.abs(a - b)) < 1e-11 * max(1.0, np.max(np.abs(b)))


def test_qk_norm_step_against_high_precision():
    """F0 with rounding: r is within one float32 ulp of 1/sqrt(mean x^2 + 1e-6)
    computed with 50 significant digits; x_n is within half a bf16 ulp (plus
    the float32 product's error) of x r; normalized rows have mean square 1 to
    bf16 precision; and r does not change when the float64 sum of squares is
    formed in another order (the GPU's), even on rows whose exact sum does not
    fit a float64."""
    from decimal import Decimal, getcontext
    getcontext().prec = 50
    x = _qk_rows(500, 64, 1e-3, 1e3)
    xn, r = F.qk_norm_rows(x)
    for i in range(x.shape[0]):
        row = [Decimal(float(t)) for t in x[i]]
        ref = 1 / (sum(t * t for t in row) / 64 + Decimal("0.000001")).sqrt()
        rf = float(ref)
        assert abs(float(r[i]) - rf) <= np.spacing(np.float32(rf))
    sq = x.astype(np.float64) ** 2
    for s_other in (np.sum(sq, axis=1), np.sum(sq[:, ::-1], axis=1), np.sum(sq.reshape(-1, 4, 16), axis=2).sum(axis=1)):
        r_other = (1.0 / np.sqrt(s_other / 64.0 + 1e-6)).astype(np.float32)
        assert np.array_equal(r_other.view(np.uint32), r.view(np.uint32))
    exact_xn = x.astype(np.float64) * r.astype(np.float64)[:, None]
    ulp = 2.0 ** (np.floor(np.log2(np.maximum(np.abs(exact_xn), 1e-30))) - 7)
    assert np.all(np.abs(xn - exact_xn) <= 0.5 * ulp * (1 + 2 ** -16))
    ms = np.mean(xn.astype(np.float64) ** 2, axis=1)
    m = np.mean(x.astype(np.float64) ** 2, axis=1)
    assert np.all(np.abs(ms - m / (m + 1e-6)) < 2 ** -6)      # 1 unless the row is as small as eps


def test_qk_norm_planted_mistakes(monkeypatch):
    """A wrong epsilon in F0 or a sign slip in B11 breaks the rounding-free
    reduction."""
    n = 96
    q, k = _qk_rows(n, 65, 1e-3, 1e-1)[None, None], _qk_rows(n, 66)[None, None]   # tiny rows: eps matters
    r = np.random.default_rng(67)
    v, do = (r.standard_normal((1, 1, n, 64)) for _ in range(2))
    x = {"q": q.astype(np.float64), "k": k.astype(np.float64), "v": v, "do": do}
    oe, le = exact.fwd_bh(x["q"], x["k"], x["v"], True, qk_norm=True)
    ge = exact.bwd_bh(x["q"], x["k"], x["v"], x["do"], True, qk_norm=True)

    def err():
        o, _ = F.fwd(x["q"], x["k"], x["v"], True, True, True, rounding=False, qk_norm=True)
        g = F.bwd(x["q"], x["k"], x["v"], oe, le, x["do"], True, True, True, rounding=False, qk_norm=True)
        return max(np.max(np.abs(o - oe)), max(np.max(np.abs(a - b)) / np.max(np.abs(b)) for a, b in zip(g, ge)))

    assert err() < 1e-10
    monkeypatch.setattr(F, "QK_NORM_EPS", 1e-5)
    assert err() > 1e-6
    monkeypatch.setattr(F, "QK_NORM_EPS", 1e-6)
    monkeypatch.setattr(F, "qk_norm_grad", lambda dxn, xn, rr: np.asarray(rr, np.float64)[:, None] * (
        dxn + xn * np.mean(dxn * xn, axis=1, keepdims=True)))      # + where the gradient has -
    assert err() > 1e-3
