"""Parity across sequence lengths around the 64-token tile boundaries.

The attention kernels walk 64-token blocks in loops unrolled two (forward) or
three (backward) blocks deep over rotating LDS buffers, with the masked
causal-diagonal and ragged-tail tiles on separate paths; the number of steps
a workgroup takes, and so which remainder path and which buffer it ends on,
depends on N and on the causal start block.  This sweep runs one head at
every N from 2 to 448 that sits on or next to a multiple of 64 (plus a few
in between), causal and not, both smoothings, for the INT8 method and the
MXFP8 mode, and compares the forward (O, LSE) and the backward alone (both
sides given the oracle's O and LSE) element-wise with the oracle of the same
mode (the bars of tests/gpu_util.py)."""
import numpy as np
import pytest
import torch

import bit_trainable_attention_amd as sb
import workloads as W
from oracle import faithful as F, mxfp8 as X
from tests import gpu_util as G

pytestmark = pytest.mark.gpu

SIZES = [2, 31, 63, 64, 65, 100, 127, 128, 129, 191, 192, 193, 255, 256, 257, 320, 383, 384, 385, 448]


@pytest.mark.parametrize("mode", ["int8", "mxfp8"])
@pytest.mark.parametrize("causal", [True, False], ids=["causal", "full"])
@pytest.mark.parametrize("N", SIZES)
def test_size_sweep_parity(N, causal, mode):
    mx = mode == "mxfp8"
    w = W.custom(1, 1, N, causal, True, True, "kbias", 400 + N)
    print(f"[sizes] N={N} causal={causal} mode={mode}", flush=True)
    x = W.make_inputs(w)
    f32 = {n: W.bf16_bits_to_f32(a) for n, a in x.items()}
    tq, tk, tv, tdo = (G.dev(x[n]) for n in ("q", "k", "v", "do"))
    oracle = X if mx else F
    o_f, lse_f = oracle.fwd(f32["q"], f32["k"], f32["v"], causal, True, True)
    o, lse = sb.fwd(tq, tk, tv, causal, True, True, mxfp8=mx)
    torch.cuda.synchronize()
    o_g, lse_g = G.host_f32(o), lse.cpu().numpy()
    assert np.all(np.isfinite(o_g)) and np.all(np.isfinite(lse_g))
    G.parity("O", o_g, o_f, mode)
    assert np.all(np.abs(lse_g - lse_f) <= (0.0625 if mx else 2e-3) + 1e-5 * np.abs(lse_f))
    o_bits = W.f32_to_bf16_bits(o_f.astype(np.float32))
    lse32 = lse_f.astype(np.float32)
    dq, dk, dv = sb.bwd(tq, tk, tv, G.dev(o_bits), torch.from_numpy(lse32).cuda(), tdo, causal, True, True,
                        mxfp8=mx)
    torch.cuda.synchronize()
    ref = oracle.bwd(f32["q"], f32["k"], f32["v"], W.bf16_bits_to_f32(o_bits), lse32, f32["do"], causal, True, True)
    for name, t, b in zip(("dQ", "dK", "dV"), (dq, dk, dv), ref):
        a = G.host_f32(t)
        assert np.all(np.isfinite(a)), name
        G.parity(name, a, b, mode, " (backward alone)")
