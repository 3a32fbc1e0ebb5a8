"""The forward entry point that allocates nothing (sagebwd_fwd_noalloc): its
outputs equal, bit for bit, those of sagebwd_fwd with a caller-owned
workspace, on two calls in a row with the second on a smaller input, and a
problem whose workspace exceeds the built-in scratch buffer is rejected
before anything runs."""
import ctypes

import numpy as np
import pytest
import torch

import bit_trainable_attention_amd as sb
import workloads as W
from tests import gpu_util as G

pytestmark = pytest.mark.gpu

SCRATCH_ERR = -5


def _noalloc(lib, p, q, k, v):
    o = torch.full_like(q, 7.0)                      # stale contents, to be overwritten
    lse = torch.full(q.shape[:3], -3.0, dtype=torch.float32, device=q.device)
    rc = lib.sagebwd_fwd_noalloc(ctypes.byref(p), sb._ptr(q), sb._ptr(k), sb._ptr(v), sb._ptr(o), sb._ptr(lse),
                                 sb._stream())
    return rc, o, lse


@pytest.mark.parametrize("mode", ["int8", "mxfp8"])
def test_noalloc_forward_matches_workspace_forward(mode):
    lib = sb.load_library()
    mx = mode == "mxfp8"
    cases = [W.custom(2, 4, 4096, True, True, True, "kbias", 401),   # 7 MB of workspace
             W.custom(1, 2, 1000, False, True, True, "outlier", 402)]  # a smaller, ragged one next
    for w in cases:
        print(f"[noalloc] {mode} B{w.B} H{w.H} N{w.N} causal={w.causal}", flush=True)
        x = W.make_inputs(w)
        q, k, v = (G.dev(x[n]) for n in ("q", "k", "v"))
        p = sb.make_params(w.B, w.H, w.N, w.causal, w.smooth_q, w.smooth_k, mxfp8=mx)
        rc, o, lse = _noalloc(lib, p, q, k, v)
        torch.cuda.synchronize()
        assert rc == 0, sb.load_library().sagebwd_status_string(rc)
        o_ref, lse_ref = sb.fwd(q, k, v, w.causal, w.smooth_q, w.smooth_k, mxfp8=mx)
        torch.cuda.synchronize()
        assert torch.equal(o.view(torch.int16), o_ref.view(torch.int16))
        assert torch.equal(lse.view(torch.int32), lse_ref.view(torch.int32))


def test_noalloc_forward_rejects_oversized_problem():
    lib = sb.load_library()
    p = sb.make_params(1, 32, 32768, True, True, True)
    assert lib.sagebwd_fwd_workspace_size(ctypes.byref(p)) > (256 << 20)
    q = torch.zeros(1, 1, 64, 64, dtype=torch.bfloat16, device="cuda")     # never read: the size check comes first
    rc = lib.sagebwd_fwd_noalloc(ctypes.byref(p), sb._ptr(q), sb._ptr(q), sb._ptr(q), sb._ptr(q), sb._ptr(q),
                                 sb._stream())
    assert rc == SCRATCH_ERR
    assert lib.sagebwd_status_string(rc) == b"workspace exceeds the built-in scratch buffer"
