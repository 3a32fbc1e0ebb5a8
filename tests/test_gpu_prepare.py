"""Bit-exact checks of the preparation kernels against the oracle: smoothing
means, INT8 codes of Q, K, V, dO in both operand layouts, and block scales.
Side outputs (correction, bias, Delta, log2 LSE) are float32 reductions whose
order differs from the oracle's, so they are compared within float32
rounding; the FP16 copies are compared bit for bit with IEEE conversion."""
import math

import numpy as np
import pytest
import torch

import bit_trainable_attention_amd as sb
import workloads as W
from oracle import faithful as F
from tests import gpu_util as G

pytestmark = pytest.mark.gpu

CASES = [
    ("tiny", None, None),
    ("ragged_causal_q", W.custom(1, 2, 200, True, True, True, "kbias", 41), None),
    ("ragged_outlier", W.custom(2, 1, 129, False, True, True, "outlier", 42), None),
    ("one_token", W.custom(1, 1, 1, True, True, True, "normal", 43), None),
    ("no_smoothing", W.custom(1, 2, 65, False, False, False, "normal", 44), None),
    ("pretrain", None, [(0, 0), (7, 15)]),
    ("llama8k", None, [(0, 31)]),
    ("video", None, [(1, 29)]),
]


def _run(w, heads, int8_dp=False, qk_norm=False, x=None):
    print(f"[prepare] {w.name} B{w.B} H{w.H} N{w.N} causal={w.causal} sq={w.smooth_q} sk={w.smooth_k} "
          f"int8_dp={int8_dp} qk_norm={qk_norm}", flush=True)
    x = W.make_inputs(w) if x is None else x
    r = np.random.default_rng(5)
    o_bits = W.f32_to_bf16_bits(r.standard_normal(x["q"].shape).astype(np.float32))
    lse = (r.standard_normal(x["q"].shape[:3]) * 3 + 5).astype(np.float32)
    tq, tk, tv, tdo = (G.dev(x[n]) for n in ("q", "k", "v", "do"))
    to = G.dev(o_bits)
    tlse = torch.from_numpy(lse).cuda()
    ws = sb.prepare(tq, tk, tv, to, tlse, tdo, w.causal, w.smooth_q, w.smooth_k, int8_dp=int8_dp, qk_norm=qk_norm)
    torch.cuda.synchronize()
    wsh = ws.cpu().numpy()
    p = sb.make_params(w.B, w.H, w.N, w.causal, w.smooth_q, w.smooth_k, int8_dp=int8_dp, qk_norm=qk_norm)
    BH, T = w.B * w.H, (w.N + 63) // 64
    Np = 64 * T
    got = {
        "mu_q": G.region(wsh, p, "MU_Q", np.float32).reshape(BH, 64),
        "mu_k": G.region(wsh, p, "MU_K", np.float32).reshape(BH, 64),
        "q_r": G.decode_codes(wsh, p, "Q_R", "row", BH, T), "k_r": G.decode_codes(wsh, p, "K_R", "row", BH, T),
        "q_t": G.decode_codes(wsh, p, "Q_T", "t", BH, T), "k_t": G.decode_codes(wsh, p, "K_T", "t", BH, T),
        "v_t": G.decode_codes(wsh, p, "V_T", "t", BH, T), "do_t": G.decode_codes(wsh, p, "DO_T", "t", BH, T),
        "sq": G.region(wsh, p, "S_Q", np.float32).reshape(BH, T), "sk": G.region(wsh, p, "S_K", np.float32).reshape(BH, T),
        "sv": G.region(wsh, p, "S_V", np.float32).reshape(BH, T), "sdo": G.region(wsh, p, "S_DO", np.float32).reshape(BH, T),
        "corr": G.region(wsh, p, "CORR", np.float32).reshape(BH, Np),
        "bias": G.region(wsh, p, "BIAS", np.float32).reshape(BH, Np),
        "delta": -G.region(wsh, p, "NDELTA", np.float32).reshape(BH, Np),
        "lse2": G.region(wsh, p, "LSE2", np.float32).reshape(BH, Np),
        "do16": G.region(wsh, p, "DO16", np.float16).reshape(BH, Np, 64),
        "v16": G.region(wsh, p, "V16", np.float16).reshape(BH, Np, 64),
    }
    if qk_norm:   # QK-norm factors of every Q and K token
        got["rq"] = G.region(wsh, p, "RQ", np.float32).reshape(BH, Np)
        got["rk"] = G.region(wsh, p, "RK", np.float32).reshape(BH, Np)
    if int8_dp:   # row-operand dO and V codes of the all-INT8 dO V^T
        got["do_r"] = G.decode_codes(wsh, p, "DO_R", "row", BH, T)
        got["v_r"] = G.decode_codes(wsh, p, "V_R", "row", BH, T)
    if heads is None:
        heads = [(b, h) for b in range(w.B) for h in range(w.H)]
    f32 = {n: W.bf16_bits_to_f32(a) for n, a in x.items()}
    of32 = W.bf16_bits_to_f32(o_bits)
    N = w.N
    for b, h in heads:
        i = b * w.H + h
        q, k, v, do = (f32[n][b, h] for n in ("q", "k", "v", "do"))
        pp = F.prepare(q, k, v, w.smooth_q, w.smooth_k, qk_norm=qk_norm)
        for xin, on in ((pp.q_raw, w.smooth_q), (pp.k_in, w.smooth_k)):     # the values the means are taken over
            assert F.sum_order_free(xin.astype(np.float32)) or not on
        if qk_norm:
            for key, rr in (("q", pp.rq), ("k", pp.rk)):
                # the GPU forms the float64 sum of squares in its own order; r
                # is the same for any order on these rows (checked with two)
                x64 = f32[key][b, h].astype(np.float64) ** 2
                for s_other in (np.sum(x64, axis=1), np.sum(x64[:, ::-1], axis=1)):
                    r_other = (1.0 / np.sqrt(s_other / 64.0 + 1e-6)).astype(np.float32)
                    assert np.array_equal(r_other.view(np.uint32), rr.view(np.uint32)), key
                assert np.array_equal(got["r" + key][i][:N].view(np.uint32), rr.view(np.uint32)), key
                assert np.all(got["r" + key][i][N:] == 0)
        bp = F.prepare_bwd(pp, v, of32[b, h], lse[b, h], do)
        assert np.array_equal(got["mu_q"][i].view(np.uint32), np.asarray(pp.mu_q, np.float32).view(np.uint32))
        assert np.array_equal(got["mu_k"][i].view(np.uint32), np.asarray(pp.mu_k, np.float32).view(np.uint32))
        for name, ref in (("q_r", pp.qc), ("q_t", pp.qc), ("k_r", pp.kc), ("k_t", pp.kc), ("v_t", pp.vc),
                          ("do_t", bp.doc)) + ((("do_r", bp.doc), ("v_r", pp.vc)) if int8_dp else ()):
            assert np.array_equal(got[name][i].astype(np.int64), ref.astype(np.int64)), name
        for name, ref in (("sq", pp.sq), ("sk", pp.sk), ("sv", pp.sv), ("sdo", bp.sdo)):
            assert np.array_equal(got[name][i].view(np.uint32), np.asarray(ref, np.float32).view(np.uint32)), name
        # float32 reductions in the kernel's own order
        cscale = float(np.max(np.abs(q) @ np.abs(pp.mu_k.astype(np.float64)))) / 8
        np.testing.assert_allclose(got["corr"][i][:N], pp.corr[:N], rtol=0, atol=1e-6 * cscale + 1e-30)
        assert np.all(got["corr"][i][N:] == 0)
        bias_ref = pp.b * (np.log2(np.e) / 8)
        bscale = (np.abs(pp.kc) @ np.abs(pp.mu_q.astype(np.float64))) * np.repeat(np.asarray(pp.sk, np.float64), 64)
        np.testing.assert_allclose(got["bias"][i], bias_ref, rtol=0, atol=1e-6 * float(bscale.max()) + 1e-30)
        np.testing.assert_allclose(got["delta"][i][:N], bp.delta[:N], rtol=0,
                                   atol=1e-6 * float((np.abs(do) * np.abs(of32[b, h])).sum(axis=1).max()))
        assert np.all(got["delta"][i][N:] == 0)
        lse2_ref = bp.lsep[:N] * np.log2(np.e)
        np.testing.assert_allclose(got["lse2"][i][:N], lse2_ref, rtol=2e-6, atol=2e-6)
        assert np.all(np.isposinf(got["lse2"][i][N:]))
        assert np.array_equal(got["do16"][i][:N], do.astype(np.float16))
        assert np.array_equal(got["v16"][i][:N], v.astype(np.float16))
        assert np.all(got["do16"][i][N:] == 0) and np.all(got["v16"][i][N:] == 0)


@pytest.mark.parametrize("name,w,heads", CASES, ids=[c[0] for c in CASES])
def test_prepare_bitexact(name, w, heads):
    G.assert_perms_are_bijections()
    _run(w if w is not None else W.WORKLOADS[name], heads)


QK_CASES = [
    ("ragged_causal", W.custom(1, 2, 200, True, True, True, "rowscale", 81), None),
    ("ragged_noncausal", W.custom(2, 1, 129, False, True, False, "rowscale", 82), None),
    ("one_token", W.custom(1, 1, 1, True, True, True, "rowscale", 83), None),
    ("pretrain_shape", W.custom(8, 16, 2048, True, True, False, "rowscale", 84), [(0, 0), (7, 15)]),
]


@pytest.mark.parametrize("name,w,heads", QK_CASES, ids=[c[0] for c in QK_CASES])
def test_prepare_bitexact_qk_norm(name, w, heads):
    """The fused QK-norm: per-token factors r and everything derived from the
    normalized rows (means, codes, scales, correction, bias), bit-exact."""
    _run(w, heads, qk_norm=True)


@pytest.mark.parametrize("name,w,heads", [c for c in CASES if c[0] in ("ragged_outlier", "one_token", "llama8k")],
                         ids=["ragged_outlier", "one_token", "llama8k"])
def test_prepare_bitexact_int8_dp(name, w, heads):
    """The all-INT8 dO V^T preparation: dO and V codes in the row-operand
    layout and the V block scales, bit-exact (the V scales come from the
    backward's own preparation and must equal the forward quantizer's)."""
    _run(w if w is not None else W.WORKLOADS[name], heads, int8_dp=True)


def test_prepare_zero_inputs():
    w = W.custom(1, 1, 100, False, True, True, "normal", 45)
    z = torch.zeros(1, 1, 100, 64, dtype=torch.bfloat16, device="cuda")
    lse = torch.zeros(1, 1, 100, dtype=torch.float32, device="cuda")
    ws = sb.prepare(z, z, z, z, lse, z, w.causal, True, True)
    torch.cuda.synchronize()
    wsh = ws.cpu().numpy()
    p = sb.make_params(1, 1, 100, False, True, True)
    for n in ("S_Q", "S_K", "S_V", "S_DO", "MU_Q", "MU_K"):
        assert np.all(G.region(wsh, p, n, np.float32) == 0)
    for n in ("Q_R", "K_R", "V_T", "Q_T", "K_T", "DO_T"):
        assert np.all(G.region(wsh, p, n, np.int8) == 0)


def test_prepare_extreme_block_magnitudes():
    """Blocks of Q and K whose absmax a runs from below the all-zero
    threshold 2^-100 up past 2^126 (where the reciprocal of a is subnormal),
    each block scaled by its own power of two: codes and scales (s = a
    fp32(1/127), inv = fp32(127/a)) bit-exact with the oracle at every
    magnitude.  V goes as low but stops at 2^10 (its FP16 copy stays finite),
    and dO stays at unit scale, so Delta stays finite."""
    exps = [125, 124, 100, 31, 0, -17, -64, -98, -100, -101, -103, 3]
    N = 64 * len(exps) - 20                                  # ragged last block
    w = W.custom(1, 1, N, False, False, False, "normal", 46)
    r = np.random.default_rng(46)
    scale = np.repeat(np.exp2(np.asarray(exps, np.float64)), 64)[:N, None]
    x = {}
    for n in ("q", "k", "v"):
        v = r.standard_normal((1, 1, N, 64)) * (np.minimum(scale, 2.0 ** 10) if n == "v" else scale)
        x[n] = W.f32_to_bf16_bits(np.clip(v, -3.0e38, 3.0e38).astype(np.float32))
    x["do"] = W.f32_to_bf16_bits(r.standard_normal((1, 1, N, 64)).astype(np.float32))
    f = W.bf16_bits_to_f32(x["q"])[0, 0]
    amax = np.array([np.abs(f[i:i + 64]).max() for i in range(0, N, 64)])
    assert np.isfinite(f).all() and amax.max() >= 2.0 ** 126                # the pre-scaled range is reached
    assert (amax < 2.0 ** -100).any() and ((amax >= 2.0 ** -100) & (amax < 2.0 ** -99)).any()
    _run(w, None, x=x)
