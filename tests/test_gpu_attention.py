"""Parity of the HIP forward and backward with the oracle.

Small cases compare every output element with the quantization-faithful
oracle (relative L2 <= 1e-2) and with exact attention (cosine >= 0.999 for O,
>= 0.99 for dQ, dK, dV).  The backward is checked alone (both sides receive
the oracle's O and LSE) and end to end (each side feeds its own forward into
its own backward)."""
import numpy as np
import pytest
import torch

import bit_trainable_attention_amd as sb
import workloads as W
from oracle import exact, faithful as F, metrics as M
from tests import gpu_util as G

pytestmark = pytest.mark.gpu

REL_L2 = 1e-2          # HIP vs faithful oracle, O / dQ / dK / dV
COS_O, COS_G = 0.999, 0.99   # HIP vs exact attention
LSE_ATOL = 2e-3        # natural-log units

SMALL = [
    W.WORKLOADS["tiny"],
    W.custom(1, 2, 200, True, True, True, "kbias", 51),
    W.custom(2, 1, 129, False, True, True, "outlier", 52),
    W.custom(1, 2, 256, True, True, False, "qknorm", 53),
    W.custom(1, 1, 320, False, False, False, "normal", 54),
    W.custom(1, 1, 1, True, True, True, "normal", 55),
    W.custom(1, 1, 63, True, True, False, "normal", 56),
    W.custom(1, 1, 64, False, True, True, "normal", 57),
    W.custom(1, 1, 65, True, True, True, "kbias", 58),
]


def _ids(ws):
    return [f"{w.name}_c{int(w.causal)}q{int(w.smooth_q)}k{int(w.smooth_k)}" for w in ws]


def _oracle_fwd(w, f32):
    o, lse = F.fwd(f32["q"], f32["k"], f32["v"], w.causal, w.smooth_q, w.smooth_k)
    return o, lse


def _bf16(x):
    return W.bf16_bits_to_f32(W.f32_to_bf16_bits(np.asarray(x, np.float32)))


@pytest.mark.parametrize("w", SMALL, ids=_ids(SMALL))
def test_forward_parity(w):
    print(f"[fwd] {w.name} c{w.causal} q{w.smooth_q} k{w.smooth_k}", flush=True)
    x = W.make_inputs(w)
    f32 = {n: W.bf16_bits_to_f32(a) for n, a in x.items()}
    o, lse = sb.fwd(G.dev(x["q"]), G.dev(x["k"]), G.dev(x["v"]), w.causal, w.smooth_q, w.smooth_k)
    torch.cuda.synchronize()
    o_g, lse_g = G.host_f32(o), lse.cpu().numpy()
    o_f, lse_f = _oracle_fwd(w, f32)
    o_e, lse_e = exact.fwd_bh(f32["q"], f32["k"], f32["v"], w.causal)
    assert np.all(np.isfinite(o_g)) and np.all(np.isfinite(lse_g))
    print(f"  O: rel-L2 vs faithful {M.rel_l2(o_g, o_f):.2e}, cos vs exact {M.cos_sim(o_g, o_e):.6f}, "
          f"LSE max err {np.max(np.abs(lse_g - lse_f)):.2e}")
    G.parity("O", o_g, o_f)
    assert np.max(np.abs(lse_g - lse_f)) <= LSE_ATOL
    assert M.cos_sim(o_g, o_e) >= COS_O
    assert np.max(np.abs(lse_g - lse_e)) <= 0.05


@pytest.mark.parametrize("w", SMALL, ids=_ids(SMALL))
def test_backward_parity(w):
    print(f"[bwd] {w.name} c{w.causal} q{w.smooth_q} k{w.smooth_k}", flush=True)
    x = W.make_inputs(w)
    f32 = {n: W.bf16_bits_to_f32(a) for n, a in x.items()}
    o_f, lse_f = _oracle_fwd(w, f32)
    o_bits = W.f32_to_bf16_bits(o_f.astype(np.float32))
    lse32 = lse_f.astype(np.float32)
    # backward alone: both sides take the oracle's O (bf16) and LSE (fp32)
    dq, dk, dv = sb.bwd(G.dev(x["q"]), G.dev(x["k"]), G.dev(x["v"]), G.dev(o_bits), torch.from_numpy(lse32).cuda(),
                        G.dev(x["do"]), w.causal, w.smooth_q, w.smooth_k)
    torch.cuda.synchronize()
    g = [G.host_f32(t) for t in (dq, dk, dv)]
    ref = F.bwd(f32["q"], f32["k"], f32["v"], W.bf16_bits_to_f32(o_bits), lse32, f32["do"], w.causal,
                w.smooth_q, w.smooth_k)
    ex = exact.bwd_bh(f32["q"], f32["k"], f32["v"], f32["do"], w.causal)
    for name, a, b, e in zip(("dQ", "dK", "dV"), g, ref, ex):
        assert np.all(np.isfinite(a)), name
        print(f"  {name}: rel-L2 vs faithful {M.rel_l2(a, b):.2e}, cos vs exact {M.cos_sim(a, e):.6f}")
        if np.linalg.norm(e) > 1e-9 * max(1.0, np.linalg.norm(b)):
            G.parity(name, a, b)
            assert M.cos_sim(a, e) >= COS_G, (name, M.cos_sim(a, e))
        else:
            assert M.rel_l2(a, b) <= REL_L2, (name, M.rel_l2(a, b))
            # degenerate case (one token: dS = 0 exactly, so dQ = dK = 0): the
            # kernel's residue must stay at the size of the O quantization noise
            assert np.linalg.norm(a) <= 1e-2 * max(np.linalg.norm(g[2]), 1e-30), name


@pytest.mark.parametrize("w", SMALL, ids=_ids(SMALL))
def test_backward_parity_int8_dp(w):
    """The all-INT8 ablation (dO V^T from INT8 codes): the backward against the
    oracle's int8_dp mode, same bars as the method's FP16 dO V^T."""
    print(f"[bwd int8_dp] {w.name} c{w.causal} q{w.smooth_q} k{w.smooth_k}", flush=True)
    x = W.make_inputs(w)
    f32 = {n: W.bf16_bits_to_f32(a) for n, a in x.items()}
    o_f, lse_f = _oracle_fwd(w, f32)
    o_bits = W.f32_to_bf16_bits(o_f.astype(np.float32))
    lse32 = lse_f.astype(np.float32)
    dq, dk, dv = sb.bwd(G.dev(x["q"]), G.dev(x["k"]), G.dev(x["v"]), G.dev(o_bits), torch.from_numpy(lse32).cuda(),
                        G.dev(x["do"]), w.causal, w.smooth_q, w.smooth_k, int8_dp=True)
    torch.cuda.synchronize()
    g = [G.host_f32(t) for t in (dq, dk, dv)]
    ref = F.bwd(f32["q"], f32["k"], f32["v"], W.bf16_bits_to_f32(o_bits), lse32, f32["do"], w.causal,
                w.smooth_q, w.smooth_k, int8_dp=True)
    ex = exact.bwd_bh(f32["q"], f32["k"], f32["v"], f32["do"], w.causal)
    for name, a, b, e in zip(("dQ", "dK", "dV"), g, ref, ex):
        assert np.all(np.isfinite(a)), name
        print(f"  {name}: rel-L2 vs faithful {M.rel_l2(a, b):.2e}, cos vs exact {M.cos_sim(a, e):.6f}")
        if np.linalg.norm(e) > 1e-9 * max(1.0, np.linalg.norm(b)):
            G.parity(name, a, b)
            assert M.cos_sim(a, e) >= COS_G, (name, M.cos_sim(a, e))
        else:
            assert M.rel_l2(a, b) <= REL_L2, (name, M.rel_l2(a, b))


@pytest.mark.parametrize("w", SMALL[:4], ids=_ids(SMALL[:4]))
def test_end_to_end_parity_and_determinism(w):
    print(f"[e2e] {w.name}", flush=True)
    x = W.make_inputs(w)
    f32 = {n: W.bf16_bits_to_f32(a) for n, a in x.items()}
    tq, tk, tv, tdo = (G.dev(x[n]) for n in ("q", "k", "v", "do"))
    outs = []
    for reuse in (False, True):
        # second pass: the backward reuses the forward's quantized Q and K
        ws = torch.empty(sb.workspace_size(w.B, w.H, w.N, w.causal, w.smooth_q, w.smooth_k), dtype=torch.uint8,
                         device="cuda") if reuse else None
        o, lse = sb.fwd(tq, tk, tv, w.causal, w.smooth_q, w.smooth_k, workspace=ws)
        dq, dk, dv = sb.bwd(tq, tk, tv, o, lse, tdo, w.causal, w.smooth_q, w.smooth_k, fwd_workspace=ws)
        torch.cuda.synchronize()
        outs.append([G.host_bits(t) for t in (o, dq, dk, dv)] + [lse.cpu().numpy().view(np.uint32)])
    for a, b in zip(*outs):
        assert np.array_equal(a, b)        # no atomics anywhere: bitwise repeatable, with or without reuse
    o_f, lse_f = _oracle_fwd(w, f32)
    o_b = _bf16(o_f)
    ref = F.bwd(f32["q"], f32["k"], f32["v"], o_b, lse_f.astype(np.float32), f32["do"], w.causal,
                w.smooth_q, w.smooth_k)
    for name, a, b in zip(("dQ", "dK", "dV"), outs[0][1:4], ref):
        G.parity(name, W.bf16_bits_to_f32(a), b)


QK_SMALL = [
    W.custom(1, 2, 200, True, True, True, "rowscale", 91),
    W.custom(2, 1, 129, False, True, False, "rowscale", 92),
    W.custom(1, 1, 65, True, False, False, "rowscale", 93),
    W.custom(1, 1, 1, True, True, True, "rowscale", 94),
]


@pytest.mark.parametrize("w", QK_SMALL, ids=_ids(QK_SMALL))
def test_qk_norm_parity(w):
    """Fused QK-norm: forward, and backward end to end (each side feeds its own
    forward), against the faithful oracle with F0/B11 and against exact
    attention on normalized Q, K with gradients through the norm."""
    print(f"[qk_norm] {w.name} c{w.causal} q{w.smooth_q} k{w.smooth_k}", flush=True)
    x = W.make_inputs(w)
    f32 = {n: W.bf16_bits_to_f32(a) for n, a in x.items()}
    tq, tk, tv, tdo = (G.dev(x[n]) for n in ("q", "k", "v", "do"))
    o, lse = sb.fwd(tq, tk, tv, w.causal, w.smooth_q, w.smooth_k, qk_norm=True)
    dq, dk, dv = sb.bwd(tq, tk, tv, o, lse, tdo, w.causal, w.smooth_q, w.smooth_k, qk_norm=True)
    torch.cuda.synchronize()
    o_g, lse_g = G.host_f32(o), lse.cpu().numpy()
    g = [G.host_f32(t) for t in (dq, dk, dv)]
    o_f, lse_f = F.fwd(f32["q"], f32["k"], f32["v"], w.causal, w.smooth_q, w.smooth_k, qk_norm=True)
    ref = F.bwd(f32["q"], f32["k"], f32["v"], _bf16(o_f), lse_f.astype(np.float32), f32["do"], w.causal,
                w.smooth_q, w.smooth_k, qk_norm=True)
    o_e, lse_e = exact.fwd_bh(f32["q"], f32["k"], f32["v"], w.causal, qk_norm=True)
    ex = exact.bwd_bh(f32["q"], f32["k"], f32["v"], f32["do"], w.causal, qk_norm=True)
    print(f"  O: rel-L2 vs faithful {M.rel_l2(o_g, o_f):.2e}, cos vs exact {M.cos_sim(o_g, o_e):.6f}")
    G.parity("O", o_g, o_f)
    assert np.max(np.abs(lse_g - lse_f)) <= LSE_ATOL
    assert M.cos_sim(o_g, o_e) >= COS_O
    for name, a, b, e in zip(("dQ", "dK", "dV"), g, ref, ex):
        assert np.all(np.isfinite(a)), name
        print(f"  {name}: rel-L2 vs faithful {M.rel_l2(a, b):.2e}, cos vs exact {M.cos_sim(a, e):.6f}")
        if np.linalg.norm(e) > 1e-9 * max(1.0, np.linalg.norm(b)):
            G.parity(name, a, b)
            assert M.cos_sim(a, e) >= COS_G, (name, M.cos_sim(a, e))
        else:
            assert M.rel_l2(a, b) <= REL_L2, (name, M.rel_l2(a, b))
            assert np.linalg.norm(a) <= 1e-2 * max(np.linalg.norm(g[2]), 1e-30), name


@pytest.mark.parametrize("w", QK_SMALL[:2], ids=_ids(QK_SMALL[:2]))
def test_qk_norm_int8_dp_parity(w):
    """The two options together: fused QK-norm with the all-INT8 dO V^T, end
    to end against the oracle with both (same bars)."""
    print(f"[qk_norm int8_dp] {w.name} c{w.causal} q{w.smooth_q} k{w.smooth_k}", flush=True)
    x = W.make_inputs(w)
    f32 = {n: W.bf16_bits_to_f32(a) for n, a in x.items()}
    tq, tk, tv, tdo = (G.dev(x[n]) for n in ("q", "k", "v", "do"))
    o, lse = sb.fwd(tq, tk, tv, w.causal, w.smooth_q, w.smooth_k, qk_norm=True)
    dq, dk, dv = sb.bwd(tq, tk, tv, o, lse, tdo, w.causal, w.smooth_q, w.smooth_k, qk_norm=True, int8_dp=True)
    torch.cuda.synchronize()
    g = [G.host_f32(t) for t in (dq, dk, dv)]
    o_f, lse_f = F.fwd(f32["q"], f32["k"], f32["v"], w.causal, w.smooth_q, w.smooth_k, qk_norm=True)
    ref = F.bwd(f32["q"], f32["k"], f32["v"], _bf16(o_f), lse_f.astype(np.float32), f32["do"], w.causal,
                w.smooth_q, w.smooth_k, qk_norm=True, int8_dp=True)
    ex = exact.bwd_bh(f32["q"], f32["k"], f32["v"], f32["do"], w.causal, qk_norm=True)
    for name, a, b, e in zip(("dQ", "dK", "dV"), g, ref, ex):
        assert np.all(np.isfinite(a)), name
        print(f"  {name}: rel-L2 vs faithful {M.rel_l2(a, b):.2e}, cos vs exact {M.cos_sim(a, e):.6f}")
        if np.linalg.norm(e) > 1e-9 * max(1.0, np.linalg.norm(b)):
            G.parity(name, a, b)
            assert M.cos_sim(a, e) >= COS_G, (name, M.cos_sim(a, e))
        else:
            assert M.rel_l2(a, b) <= REL_L2, (name, M.rel_l2(a, b))


def test_zero_inputs():
    z = torch.zeros(1, 2, 100, 64, dtype=torch.bfloat16, device="cuda")
    for causal in (False, True):
        o, lse = sb.fwd(z, z, z, causal, True, True)
        dq, dk, dv = sb.bwd(z, z, z, o, lse, z, causal, True, True)
        torch.cuda.synchronize()
        for t in (o, dq, dk, dv):
            assert torch.all(t == 0)
        n = torch.arange(1, 101, device="cuda", dtype=torch.float32) if causal else torch.full((100,), 100.0, device="cuda")
        assert torch.allclose(lse[0, 0], torch.log(n), atol=1e-5)


@pytest.mark.parametrize("qk_norm,mxfp8", [(False, False), (True, False), (False, True)],
                         ids=["plain", "qknorm", "mxfp8"])
def test_autograd_wrapper(qk_norm, mxfp8):
    w = W.custom(1, 1, 96, True, True, True, "rowscale" if qk_norm else "kbias", 59)
    x = W.make_inputs(w)
    q, k, v = (G.dev(x[n]).requires_grad_(True) for n in ("q", "k", "v"))
    o = sb.SageBwdAttention.apply(q, k, v, True, True, True, qk_norm, mxfp8)
    o.backward(G.dev(x["do"]))
    dq, dk, dv = sb.bwd(q.detach(), k.detach(), v.detach(),
                        *sb.fwd(q.detach(), k.detach(), v.detach(), True, True, True, qk_norm=qk_norm, mxfp8=mxfp8),
                        G.dev(x["do"]), True, True, True, qk_norm=qk_norm, mxfp8=mxfp8)
    torch.cuda.synchronize()
    for a, b in ((q.grad, dq), (k.grad, dk), (v.grad, dv)):
        assert torch.equal(a, b)
