"""Parity at the full workload sizes, in the launch configuration bench.py
times (the whole forward and backward over every head on the GPU, the
backward reusing the forward's quantized Q and K).

The oracle cannot afford every head of these workloads, so it runs on sampled
heads: its forward over all query rows of a head (the backward of a key block
needs every row's O, LSE and Delta), then its backward for eight sampled
query blocks (dQ) and key blocks (dK, dV): the first two, four spread over
the sequence and the last two, which covers causal diagonals, the ragged
tail and blocks of every length.  Each side feeds its own forward into its
own backward (end to end).  Every output is checked element-wise: relative L2
over the sampled rows, and the worst single row and 64-row tile.  The
headline workload (llama16k) is checked on four heads, one on each of four
different XCDs (head index mod 8)."""
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
    ("llama16k", None, (0, 2), False),
    ("llama16k", None, (0, 12), False),
    ("llama16k", None, (0, 23), False),
    ("video", None, (1, 3), False),
    ("video", False, (0, 11), False),   # the same layer with Q-smoothing off
    ("llama8k", None, (0, 17), True),   # the all-INT8 dO V^T ablation, same head as above
]


def _blocks(T):
    return sorted({0, min(1, T - 1), T // 5, (2 * T) // 5, (3 * T) // 5, (4 * T) // 5, max(T - 2, 0), T - 1})


def _run_gpu(w, sq, int8_dp=False):
    x = W.make_inputs(w)
    tq, tk, tv, tdo = (G.dev(x[n]) for n in ("q", "k", "v", "do"))
    fws = torch.empty(sb.workspace_size(w.B, w.H, w.N, w.causal, sq, w.smooth_k), dtype=torch.uint8, device="cuda")
    o, lse = sb.fwd(tq, tk, tv, w.causal, sq, w.smooth_k, workspace=fws)
    dq, dk, dv = sb.bwd(tq, tk, tv, o, lse, tdo, w.causal, sq, w.smooth_k, fwd_workspace=fws, int8_dp=int8_dp)
    torch.cuda.synchronize()
    return o, lse, dq, dk, dv


@pytest.mark.parametrize("name,smooth_q,head,int8_dp", CASES,
                         ids=[f"{c[0]}_h{c[2][0]}.{c[2][1]}{'' if c[1] is None else '_q' + str(int(c[1]))}"
                              f"{'_int8dp' if c[3] else ''}" for c in CASES])
def test_fullsize_sampled_parity(name, smooth_q, head, int8_dp):
    w = W.WORKLOADS[name]
    sq = w.smooth_q if smooth_q is None else smooth_q
    b, h = head
    print(f"[fullsize] {name} B{w.B} H{w.H} N{w.N} causal={w.causal} smooth_q={sq} head={head} int8_dp={int8_dp}",
          flush=True)
    o, lse, dq, dk, dv = _run_gpu(w, sq, int8_dp)
    o_g = G.host_f32(o[b, h])
    lse_g = lse[b, h].cpu().numpy()
    dq_g, dk_g, dv_g = (G.host_f32(t[b, h]) for t in (dq, dk, dv))
    for t in (o_g, lse_g, dq_g, dk_g, dv_g):
        assert np.all(np.isfinite(t))
    del o, lse, dq, dk, dv

    f = {n: W.bf16_bits_to_f32(a) for n, a in W.make_head(w, b, h).items()}
    N, T = w.N, (w.N + 63) // 64
    pp = F.prepare(f["q"], f["k"], f["v"], sq, w.smooth_k)
    o_f, lse_f = F.fwd_head(pp, w.causal)
    o_f, lse_f = o_f[:N], lse_f[:N]
    G.parity("O", o_g, o_f, where=" (all rows)")
    assert np.max(np.abs(lse_g - lse_f)) <= 2e-3
    blocks = _blocks(T)
    rows = np.concatenate([np.arange(i * 64, min(N, i * 64 + 64)) for i in blocks])
    # end to end: the oracle's backward takes the oracle's O (bf16) and LSE
    o_b = W.bf16_bits_to_f32(W.f32_to_bf16_bits(o_f.astype(np.float32)))
    bp = F.prepare_bwd(pp, f["v"], o_b, lse_f.astype(np.float32), f["do"], int8_dp)
    dq_f, dk_f, dv_f = F.bwd_head(bp, w.causal, blocks, blocks)
    sel = np.concatenate([np.arange(j * 64, j * 64 + min(64, N - i * 64)) for j, i in enumerate(blocks)])
    for k, a, r in (("dQ", dq_g, dq_f), ("dK", dk_g, dk_f), ("dV", dv_g, dv_f)):
        G.parity(k, a[rows], r[sel], where=f" (blocks {blocks})")
    # against exact attention, on the same sampled rows
    oe, le, dqe, dke, dve = exact.sampled(f["q"], f["k"], f["v"], f["do"], w.causal, rows, rows)
    cos = {"O": M.cos_sim(o_g[rows], oe), "dQ": M.cos_sim(dq_g[rows], dqe), "dK": M.cos_sim(dk_g[rows], dke),
           "dV": M.cos_sim(dv_g[rows], dve)}
    print("  cos vs exact:", {k: f"{v:.6f}" for k, v in cos.items()}, flush=True)
    assert cos["O"] >= 0.999
    for k in ("dQ", "dK", "dV"):
        assert cos[k] >= 0.99, (k, cos[k])


QSMOOTH = [("video", (1, 3)), ("video", (0, 11)), ("llama16k", (0, 29))]


@pytest.mark.parametrize("name,head", QSMOOTH, ids=[f"{c[0]}_h{c[1][0]}.{c[1][1]}" for c in QSMOOTH])
def test_q_smoothing_comparison(name, head):
    """The same heads with Q-smoothing on and off (SageBwd abstract, insight
    (iv): Q-smoothing is optional and of limited benefit in pretraining; the
    SageAttention3 summary's table lists "Add Q smoothing" among its measured
    effects): cosine similarity, relative L1 and relative L2 against exact
    attention of O, dQ, dK, dV on the sampled blocks, for both modes.  Both
    must meet the bars (cosine >= 0.999 for O, >= 0.99 for the gradients)."""
    w = W.WORKLOADS[name]
    b, h = head
    f = {n: W.bf16_bits_to_f32(a) for n, a in W.make_head(w, b, h).items()}
    N, T = w.N, (w.N + 63) // 64
    blocks = _blocks(T)
    rows = np.concatenate([np.arange(i * 64, min(N, i * 64 + 64)) for i in blocks])
    ex = dict(zip(("O", "LSE", "dQ", "dK", "dV"), exact.sampled(f["q"], f["k"], f["v"], f["do"], w.causal, rows, rows)))
    for sq in (True, False):
        o, lse, dq, dk, dv = _run_gpu(w, sq)
        got = {"O": G.host_f32(o[b, h])[rows], "dQ": G.host_f32(dq[b, h])[rows], "dK": G.host_f32(dk[b, h])[rows],
               "dV": G.host_f32(dv[b, h])[rows]}
        del o, lse, dq, dk, dv
        res = {k: (M.cos_sim(a, ex[k]), M.l1(a, ex[k]), M.rel_l2(a, ex[k])) for k, a in got.items()}
        print(f"[q-smoothing {'on ' if sq else 'off'}] {name} head={head}: " +
              ", ".join(f"{k} cos {c:.6f} L1 {l:.3e} relL2 {r:.3e}" for k, (c, l, r) in res.items()), flush=True)
        assert res["O"][0] >= 0.999
        for k in ("dQ", "dK", "dV"):
            assert res[k][0] >= 0.99, (sq, k, res[k])


def test_fullsize_qk_norm_sampled_parity():
    """The fused QK-norm at the pretraining shape (B8 H16 N2048 causal) on raw
    rows of very different sizes: one sampled head, forward over all rows and
    the backward's sampled blocks, with gradients through the norm."""
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
    G.parity("O", o_g, o_f)
    assert np.max(np.abs(lse_g - lse_f)) <= 2e-3
    blocks = _blocks(T)
    rows = np.concatenate([np.arange(i * 64, i * 64 + 64) for i in blocks])
    o_b = W.bf16_bits_to_f32(W.f32_to_bf16_bits(o_f.astype(np.float32)))
    bp = F.prepare_bwd(pp, f["v"], o_b, lse_f.astype(np.float32), f["do"])
    dq_f, dk_f, dv_f = F.bwd_head(bp, True, blocks, blocks)
    dq_f, dk_f = F.norm_grads(pp, dq_f, dk_f, rows, rows)
    for k, a, r in (("dQ", dq_g, dq_f), ("dK", dk_g, dk_f), ("dV", dv_g, dv_f)):
        G.parity(k, a[rows], r)
    oe, le, dqe, dke, dve = exact.sampled(f["q"], f["k"], f["v"], f["do"], True, rows, rows, qk_norm=True)
    cos = {"O": M.cos_sim(o_g[rows], oe), "dQ": M.cos_sim(dq_g[rows], dqe), "dK": M.cos_sim(dk_g[rows], dke),
           "dV": M.cos_sim(dv_g[rows], dve)}
    print("  cos vs exact:", {k: f"{v:.6f}" for k, v in cos.items()}, flush=True)
    assert cos["O"] >= 0.999
    for k in ("dQ", "dK", "dV"):
        assert cos[k] >= 0.99, (k, cos[k])


def test_heads_independent_bitwise():
    """Every (batch, head) is computed on its own: the second batch of the
    video layer (B2 H30 N17776, non-causal) run alone gives, bit for bit, the
    forward and backward outputs it has inside the full batch."""
    w = W.WORKLOADS["video"]
    print(f"[heads] video B{w.B} H{w.H} N{w.N}: batch 1 alone vs inside the full batch", flush=True)
    x = W.make_inputs(w)
    t = {n: G.dev(x[n]) for n in ("q", "k", "v", "do")}
    del x
    o, lse = sb.fwd(t["q"], t["k"], t["v"], w.causal, w.smooth_q, w.smooth_k)
    g_full = sb.bwd(t["q"], t["k"], t["v"], o, lse, t["do"], w.causal, w.smooth_q, w.smooth_k)
    s = {n: a[1:2].contiguous() for n, a in t.items()}
    o1, lse1 = sb.fwd(s["q"], s["k"], s["v"], w.causal, w.smooth_q, w.smooth_k)
    g_one = sb.bwd(s["q"], s["k"], s["v"], o1, lse1, s["do"], w.causal, w.smooth_q, w.smooth_k)
    torch.cuda.synchronize()
    assert torch.equal(o[1:2].view(torch.int16), o1.view(torch.int16)) and torch.equal(lse[1:2], lse1)
    for name, a, b in zip(("dQ", "dK", "dV"), g_full, g_one):
        assert torch.equal(a[1:2].view(torch.int16), b.view(torch.int16)), name


MAXN_MODES = ["int8", "mxfp8", "fp4"]


@pytest.mark.parametrize("mode", MAXN_MODES)
def test_max_n(mode):
    """The largest N the ABI accepts (2^18, one causal head with both
    smoothings): O and LSE of the first,
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


def test_max_heads():
    """The largest B*H the ABI accepts (65 535 heads of N = 65, causal, both
    smoothings): forward and backward run over the whole grid, and four heads
    spread over it (first, second, middle, last) are compared with the
    oracle: O and LSE, and dQ, dK, dV with both sides given the GPU's O and
    LSE.  The other heads hold a copy of head 0's inputs (heads are
    independent; only the grid size matters there)."""
    B, H, N = 1, 65535, 65
    w = W.custom(B, H, N, True, True, True, "kbias", 320)
    sample = [0, 1, 32767, 65534]
    print(f"[max heads] B{B} H{H} N{N} causal sampled heads {sample}", flush=True)
    heads = {h: W.make_head(w, 0, h) for h in sample}
    x = {n: np.empty((B, H, N, 64), np.uint16) for n in ("q", "k", "v", "do")}
    for n in x:
        x[n][0, :] = heads[0][n]
        for h in sample:
            x[n][0, h] = heads[h][n]
    tq, tk, tv, tdo = (G.dev(x[n]) for n in ("q", "k", "v", "do"))
    del x
    o, lse = sb.fwd(tq, tk, tv, True, True, True)
    dq, dk, dv = sb.bwd(tq, tk, tv, o, lse, tdo, True, True, True)
    torch.cuda.synchronize()
    for t in (o, dq, dk, dv):
        assert bool(torch.isfinite(t.float()).all())
    for h in sample:
        f = {n: W.bf16_bits_to_f32(heads[h][n])[None, None] for n in heads[h]}
        o_f, lse_f = F.fwd(f["q"], f["k"], f["v"], True, True, True)
        o_g = G.host_f32(o[0, h:h + 1])[None]
        lse_g = lse[0, h].cpu().numpy()
        G.parity("O", o_g, o_f, "int8", f" (head {h})")
        assert np.max(np.abs(lse_g - lse_f[0, 0])) <= 2e-3
        ref = F.bwd(f["q"], f["k"], f["v"], o_g, lse_g[None, None].astype(np.float32), f["do"], True, True, True)
        for name, t, r in zip(("dQ", "dK", "dV"), (dq, dk, dv), ref):
            G.parity(name, G.host_f32(t[0, h:h + 1])[None], r, "int8", f" (head {h})")
