"""A forward + backward captured in one HIP graph (torch.cuda.graph) replays
bit for bit like the eager calls: the library only launches kernels on the
caller's stream (no allocation, memset, copy or synchronization), and its
kernels use no atomics.  Each replay follows eager work of the program's own
(the outputs are overwritten with garbage and the device synchronized) and is
compared with the eager results."""
import pytest
import torch

import bit_trainable_attention_amd as sb
import workloads as W
from tests import gpu_util as G

pytestmark = pytest.mark.gpu

CASES = [
    (W.custom(1, 2, 300, True, True, True, "kbias", 71), dict()),
    (W.custom(1, 2, 200, False, True, True, "normal", 72), dict(mxfp8=True)),
]


@pytest.mark.parametrize("w,mode", CASES, ids=["int8_causal_N300", "mxfp8_noncausal_N200"])
def test_graph_replay_bitwise(w, mode):
    print(f"[graph] {w.name} B{w.B} H{w.H} N{w.N} causal={w.causal} {mode}", flush=True)
    x = W.make_inputs(w)
    q, k, v, do = (G.dev(x[n]) for n in ("q", "k", "v", "do"))
    flags = (w.causal, w.smooth_q, w.smooth_k)
    B, H, N, _ = q.shape
    nf = sb.workspace_size(B, H, N, *flags, **mode)
    nb = sb.workspace_size(B, H, N, *flags, backward=True, **mode)

    # eager reference
    ws_f = torch.empty(nf, dtype=torch.uint8, device="cuda")
    ws_b = torch.empty(nb, dtype=torch.uint8, device="cuda")
    o_e, lse_e = sb.fwd(q, k, v, *flags, workspace=ws_f, **mode)
    dq_e, dk_e, dv_e = sb.bwd(q, k, v, o_e, lse_e, do, *flags, workspace=ws_b, fwd_workspace=ws_f, **mode)
    torch.cuda.synchronize()

    # the same two calls captured, on buffers allocated before the capture
    ws_f2 = torch.empty_like(ws_f)
    ws_b2 = torch.empty_like(ws_b)
    o, lse = torch.empty_like(o_e), torch.empty_like(lse_e)
    dq, dk, dv = torch.empty_like(dq_e), torch.empty_like(dk_e), torch.empty_like(dv_e)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        sb.fwd(q, k, v, *flags, workspace=ws_f2, out=(o, lse), **mode)
        sb.bwd(q, k, v, o, lse, do, *flags, workspace=ws_b2, out=(dq, dk, dv), fwd_workspace=ws_f2, **mode)
    torch.cuda.synchronize()

    outs = (o, lse, dq, dk, dv)
    refs = (o_e, lse_e, dq_e, dk_e, dv_e)
    for rep in range(3):
        for t in outs:
            t.fill_(float("nan"))          # eager work between replays
        ws_f2.fill_(0x5A)
        ws_b2.fill_(0xA5)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for name, t, r in zip(("O", "LSE", "dQ", "dK", "dV"), outs, refs):
            assert torch.equal(t.view(torch.int16) if t.dtype == torch.bfloat16 else t.view(torch.int32),
                               r.view(torch.int16) if r.dtype == torch.bfloat16 else r.view(torch.int32)), \
                f"replay {rep}: {name} differs from the eager call"
        print(f"  replay {rep}: O, LSE, dQ, dK, dV bitwise equal to the eager calls", flush=True)


def test_graph_replay_fp4_forward():
    """The FP4 inference forward captured alone replays bit for bit too."""
    w = W.custom(1, 2, 260, True, True, True, "kbias", 73)
    print(f"[graph fp4] {w.name} B{w.B} H{w.H} N{w.N} causal={w.causal}", flush=True)
    x = W.make_inputs(w)
    q, k, v = (G.dev(x[n]) for n in ("q", "k", "v"))
    flags = (w.causal, w.smooth_q, w.smooth_k)
    B, H, N, _ = q.shape
    nf = sb.workspace_size(B, H, N, *flags, fp4=True)
    ws = torch.empty(nf, dtype=torch.uint8, device="cuda")
    o_e, lse_e = sb.fwd(q, k, v, *flags, workspace=ws, fp4=True)
    torch.cuda.synchronize()
    ws2 = torch.empty_like(ws)
    o, lse = torch.empty_like(o_e), torch.empty_like(lse_e)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        sb.fwd(q, k, v, *flags, workspace=ws2, out=(o, lse), fp4=True)
    torch.cuda.synchronize()
    for rep in range(3):
        o.fill_(float("nan"))
        lse.fill_(float("nan"))
        ws2.fill_(0x3C)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(o.view(torch.int16), o_e.view(torch.int16)), f"replay {rep}: O"
        assert torch.equal(lse.view(torch.int32), lse_e.view(torch.int32)), f"replay {rep}: LSE"
        print(f"  replay {rep}: O, LSE bitwise equal to the eager call", flush=True)
