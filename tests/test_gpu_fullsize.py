"""Parity at the full workload sizes, in the launch configuration bench.py
times (the whole forward and backward over every head on the GPU, the
backward reusing the forward's quantized Q and K).

The oracle cannot afford every head of these workloads, so it is run on one
sampled head per workload: its forward over all query rows of that head (the
backward of a key block needs every row's O, LSE and Delta), then its
backward for sampled query blocks (dQ) and key blocks (dK, dV): first, middle
and last, which covers the causal diagonal and the ragged tail.  Each side
feeds its own forward into its own backward (end to end)."""
import numpy as np
import pytest
import torch

import bit_trainable_attention_amd as sb
import workloads as W
from oracle import exact, faithful as F, metrics as M
from tests import gpu_util as G

pytestmark = pytest.mark.gpu

CASES = [
    ("tiny", None, (0, 1), False),
    ("pretrain", None, (7, 15), False),
    ("llama8k", None, (0, 17), False),
    ("llama16k", None, (0, 29), False),
    ("video", None, (1, 3), False),
    ("video", False, (0, 11), False),   # the same layer with Q-smoothing off
    ("llama8k", None, (0, 17), True),   # the all-INT8 dO V^T ablation, same head as above
]


def _blocks(T):
    return sorted({0, T // 2, T - 1})


@pytest.mark.parametrize("name,smooth_q,head,int8_dp", CASES,
                         ids=[f"{c[0]}{'' if c[1] is None else '_q' + str(int(c[1]))}{'_int8dp' if c[3] else ''}"
                              for c in CASES])
def test_fullsize_sampled_parity(name, smooth_q, head, int8_dp):
    w = W.WORKLOADS[name]
    sq = w.smooth_q if smooth_q is None else smooth_q
    b, h = head
    print(f"[fullsize] {name} B{w.B} H{w.H} N{w.N} causal={w.causal} smooth_q={sq} head={head} int8_dp={int8_dp}",
          flush=True)
    x = W.make_inputs(w)
    tq, tk, tv, tdo = (G.dev(x[n]) for n in ("q", "k", "v", "do"))
    fws = torch.empty(sb.workspace_size(w.B, w.H, w.N, w.causal, sq, w.smooth_k), dtype=torch.uint8, device="cuda")
    o, lse = sb.fwd(tq, tk, tv, w.causal, sq, w.smooth_k, workspace=fws)
    dq, dk, dv = sb.bwd(tq, tk, tv, o, lse, tdo, w.causal, sq, w.smooth_k, fwd_workspace=fws, int8_dp=int8_dp)
    torch.cuda.synchronize()
    o_g = G.host_f32(o[b, h])
    lse_g = lse[b, h].cpu().numpy()
    dq_g, dk_g, dv_g = (G.host_f32(t[b, h]) for t in (dq, dk, dv))
    for t in (o_g, lse_g, dq_g, dk_g, dv_g):
        assert np.all(np.isfinite(t))
    del x, tq, tk, tv, tdo, o, lse, dq, dk, dv, fws

    f = {n: W.bf16_bits_to_f32(a) for n, a in W.make_head(w, b, h).items()}
    N, T = w.N, (w.N + 63) // 64
    pp = F.prepare(f["q"], f["k"], f["v"], sq, w.smooth_k)
    o_f, lse_f = F.fwd_head(pp, w.causal)
    o_f, lse_f = o_f[:N], lse_f[:N]
    blocks = _blocks(T)
    rows = np.concatenate([np.arange(i * 64, min(N, i * 64 + 64)) for i in blocks])
    assert M.rel_l2(o_g[rows], o_f[rows]) <= 1e-2, M.rel_l2(o_g[rows], o_f[rows])
    assert M.rel_l2(o_g, o_f) <= 1e-2
    assert np.max(np.abs(lse_g - lse_f)) <= 2e-3
    # end to end: the oracle's backward takes the oracle's O (bf16) and LSE
    o_b = W.bf16_bits_to_f32(W.f32_to_bf16_bits(o_f.astype(np.float32)))
    bp = F.prepare_bwd(pp, f["v"], o_b, lse_f.astype(np.float32), f["do"], int8_dp)
    dq_f, dk_f, dv_f = F.bwd_head(bp, w.causal, blocks, blocks)
    sel = np.concatenate([np.arange(j * 64, j * 64 + min(64, N - i * 64)) for j, i in enumerate(blocks)])
    errs = {"dQ": M.rel_l2(dq_g[rows], dq_f[sel]), "dK": M.rel_l2(dk_g[rows], dk_f[sel]),
            "dV": M.rel_l2(dv_g[rows], dv_f[sel])}
    print("  rel-L2 vs faithful:", {k: f"{v:.2e}" for k, v in errs.items()},
          f"O {M.rel_l2(o_g, o_f):.2e}", flush=True)
    for k, v in errs.items():
        assert v <= 1e-2, (k, v)
    # against exact attention, on the same sampled rows
    oe, le, dqe, dke, dve = exact.sampled(f["q"], f["k"], f["v"], f["do"], w.causal, rows, rows)
    cos = {"O": M.cos_sim(o_g[rows], oe), "dQ": M.cos_sim(dq_g[rows], dqe), "dK": M.cos_sim(dk_g[rows], dke),
           "dV": M.cos_sim(dv_g[rows], dve)}
    print("  cos vs exact:", {k: f"{v:.6f}" for k, v in cos.items()}, flush=True)
    assert cos["O"] >= 0.999
    for k in ("dQ", "dK", "dV"):
        assert cos[k] >= 0.99, (k, cos[k])


def test_fullsize_qk_norm_sampled_parity():
    """The fused QK-norm at the pretraining shape (B8 H16 N2048 causal) on raw
    rows of very different sizes: one sampled head, forward over all rows and
    the backward's first, middle and last blocks, with gradients through the
    norm."""
    w = W.custom(8, 16, 2048, True, True, False, "rowscale", 95)
    b, h = 5, 9
    print(f"[fullsize qk_norm] B{w.B} H{w.H} N{w.N} head=({b}, {h})", flush=True)
    x = W.make_inputs(w)
    tq, tk, tv, tdo = (G.dev(x[n]) for n in ("q", "k", "v", "do"))
    fws = torch.empty(sb.workspace_size(w.B, w.H, w.N, True, False, True, qk_norm=True), dtype=torch.uint8,
                      device="cuda")
    o, lse = sb.fwd(tq, tk, tv, True, False, True, workspace=fws, qk_norm=True)
    dq, dk, dv = sb.bwd(tq, tk, tv, o, lse, tdo, True, False, True, fwd_workspace=fws, qk_norm=True)
    torch.cuda.synchronize()
    o_g, lse_g = G.host_f32(o[b, h]), lse[b, h].cpu().numpy()
    dq_g, dk_g, dv_g = (G.host_f32(t[b, h]) for t in (dq, dk, dv))
    del x, tq, tk, tv, tdo, o, lse, dq, dk, dv, fws
    f = {n: W.bf16_bits_to_f32(a) for n, a in W.make_head(w, b, h).items()}
    N, T = w.N, w.N // 64
    pp = F.prepare(f["q"], f["k"], f["v"], False, True, qk_norm=True)
    o_f, lse_f = F.fwd_head(pp, True)
    o_f, lse_f = o_f[:N], lse_f[:N]
    assert M.rel_l2(o_g, o_f) <= 1e-2 and np.max(np.abs(lse_g - lse_f)) <= 2e-3
    blocks = _blocks(T)
    rows = np.concatenate([np.arange(i * 64, i * 64 + 64) for i in blocks])
    o_b = W.bf16_bits_to_f32(W.f32_to_bf16_bits(o_f.astype(np.float32)))
    bp = F.prepare_bwd(pp, f["v"], o_b, lse_f.astype(np.float32), f["do"])
    dq_f, dk_f, dv_f = F.bwd_head(bp, True, blocks, blocks)
    dq_f, dk_f = F.norm_grads(pp, dq_f, dk_f, rows, rows)
    errs = {"dQ": M.rel_l2(dq_g[rows], dq_f), "dK": M.rel_l2(dk_g[rows], dk_f), "dV": M.rel_l2(dv_g[rows], dv_f)}
    print("  rel-L2 vs faithful:", {k: f"{v:.2e}" for k, v in errs.items()}, flush=True)
    for k, v in errs.items():
        assert v <= 1e-2, (k, v)
    oe, le, dqe, dke, dve = exact.sampled(f["q"], f["k"], f["v"], f["do"], True, rows, rows, qk_norm=True)
    cos = {"O": M.cos_sim(o_g[rows], oe), "dQ": M.cos_sim(dq_g[rows], dqe), "dK": M.cos_sim(dk_g[rows], dke),
           "dV": M.cos_sim(dv_g[rows], dve)}
    print("  cos vs exact:", {k: f"{v:.6f}" for k, v in cos.items()}, flush=True)
    assert cos["O"] >= 0.999
    for k in ("dQ", "dK", "dV"):
        assert cos[k] >= 0.99, (k, cos[k])


def test_head_groups_bitwise():
    """The video layer (B2 H30 N17776, non-causal) keeps more dS codes than
    one head group holds, so its backward runs in two groups of 30 heads.
    Heads are independent, so the second batch's results must equal, bit for
    bit, those of the same batch run on its own (a single group)."""
    w = W.WORKLOADS["video"]
    T = (w.N + 63) // 64
    full = sb.make_params(w.B, w.H, w.N, w.causal, w.smooth_q, w.smooth_k)
    half = sb.make_params(1, w.H, w.N, w.causal, w.smooth_q, w.smooth_k)
    assert sb.ws_region(full, "DS")[1] == sb.ws_region(half, "DS")[1] == w.H * T * T * 4096
    print(f"[groups] video B{w.B} H{w.H} N{w.N}: two groups of {w.H} heads vs one", flush=True)
    x = W.make_inputs(w)
    t = {n: G.dev(x[n]) for n in ("q", "k", "v", "do")}
    del x
    o, lse = sb.fwd(t["q"], t["k"], t["v"], w.causal, w.smooth_q, w.smooth_k)
    g_full = sb.bwd(t["q"], t["k"], t["v"], o, lse, t["do"], w.causal, w.smooth_q, w.smooth_k)
    s = {n: a[1:2].contiguous() for n, a in t.items()}
    g_one = sb.bwd(s["q"], s["k"], s["v"], o[1:2].contiguous(), lse[1:2].contiguous(), s["do"], w.causal,
                   w.smooth_q, w.smooth_k)
    torch.cuda.synchronize()
    for name, a, b in zip(("dQ", "dK", "dV"), g_full, g_one):
        assert torch.equal(a[1:2].view(torch.int16), b.view(torch.int16)), name


MAXN_MODES = ["int8", "mxfp8", "fp4"]


@pytest.mark.parametrize("mode", MAXN_MODES)
def test_max_n(mode):
    """The largest N the ABI accepts (2^18, one causal head with both
    smoothings; its backward keeps 34 GB of dS codes): O and LSE of the first,
    a middle and the last query block against the oracle (each side its own
    forward), and for the trainable modes dQ of the same blocks end to end
    (a row's dQ needs only that row's O, LSE and Delta, so the oracle's
    forward of those blocks feeds its backward)."""
    from oracle import fp4 as Y, mxfp8 as X
    N = 1 << 18
    w = W.custom(1, 1, N, True, True, True, "kbias", 310)
    T = N // 64
    blocks = [0, T // 2 + 3, T - 1]
    rows = np.concatenate([np.arange(i * 64, i * 64 + 64) for i in blocks])
    print(f"[max N] mode={mode} N={N} blocks={blocks}", flush=True)
    x = W.make_inputs(w)
    tq, tk, tv, tdo = (G.dev(x[n]) for n in ("q", "k", "v", "do"))
    kw = {"mxfp8": mode == "mxfp8", "fp4": mode == "fp4"}
    o, lse = sb.fwd(tq, tk, tv, True, True, True, **kw)
    dq_g = None
    if mode != "fp4":
        dq, dk, dv = sb.bwd(tq, tk, tv, o, lse, tdo, True, True, True, mxfp8=kw["mxfp8"])
        torch.cuda.synchronize()
        dq_g = G.host_f32(dq[0, 0])[rows]
        for t in (dk, dv):
            assert bool(torch.isfinite(t.float()).all())
        del dq, dk, dv
    torch.cuda.synchronize()
    o_g, lse_g = G.host_f32(o[0, 0])[rows], lse[0, 0].cpu().numpy()[rows]
    del tq, tk, tv, tdo, o, lse
    f = {n: W.bf16_bits_to_f32(a)[0, 0] for n, a in x.items()}
    mod = {"int8": F, "mxfp8": X, "fp4": Y}[mode]
    pp = mod.prepare(f["q"], f["k"], f["v"], True, True)
    o_f, lse_f = mod.fwd_head(pp, True, qblocks=blocks)
    err_o = M.rel_l2(o_g, o_f)
    print(f"  O rel-L2 vs oracle {err_o:.2e}, LSE max err {np.max(np.abs(lse_g - lse_f)):.2e}", flush=True)
    assert np.all(np.isfinite(o_g)) and err_o <= 1e-2
    assert np.max(np.abs(lse_g - lse_f)) <= (2e-3 if mode == "int8" else 0.0625 if mode == "mxfp8" else 0.406)
    assert np.mean(np.abs(lse_g - lse_f)) <= 2e-4
    if dq_g is not None:
        o_all = np.zeros((N, 64), np.float32)
        lse_all = np.zeros(N, np.float32)
        o_all[rows] = W.bf16_bits_to_f32(W.f32_to_bf16_bits(o_f.astype(np.float32)))
        lse_all[rows] = lse_f
        bp = mod.prepare_bwd(pp, f["v"], o_all, lse_all, f["do"])
        dq_f, _, _ = mod.bwd_head(bp, True, qblocks=blocks, kblocks=[])
        err = M.rel_l2(dq_g, dq_f)
        print(f"  dQ rel-L2 vs oracle {err:.2e}", flush=True)
        assert np.all(np.isfinite(dq_g)) and err <= 1e-2
