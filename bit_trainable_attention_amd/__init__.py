"""MI355X (gfx950) SageBwd trainable INT8 attention: Python binding.

A thin ctypes layer over ``libsagebwd.so`` (declared in include/sagebwd.h).
It only checks and marshals arguments -- device pointers, sizes, flags and the
current HIP stream -- and allocates the caller-side buffers with torch; every
step of the computation runs in the library's HIP kernels.  There is no
fallback: if the library is not built, or no GPU is present, the calls raise.

    o, lse = fwd(q, k, v, causal=True, smooth_q=False, smooth_k=True)
    dq, dk, dv = bwd(q, k, v, o, lse, do, causal=True, smooth_q=False, smooth_k=True)
    o = SageBwdAttention.apply(q, k, v, causal, smooth_q, smooth_k)   # autograd

q, k, v, do: torch.bfloat16 CUDA tensors [B, H, N, 64], contiguous.
"""
from __future__ import annotations

import ctypes
import os

import torch

__all__ = ["check_block_scale", "debug_tile", "DUMP_BYTES", "fwd", "bwd", "fwd_stage", "bwd_stage", "STAGES", "prepare", "ws_region", "workspace_size", "Params", "SageBwdAttention",
           "SageBwdError", "REGIONS", "load_library", "LIB_PATH"]

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libsagebwd.so")

REGIONS = {"MU_Q": 0, "MU_K": 1, "Q_R": 2, "K_R": 3, "V_T": 4, "Q_T": 5, "K_T": 6, "DO_T": 7,
           "S_Q": 8, "S_K": 9, "S_V": 10, "S_DO": 11, "CORR": 12, "BIAS": 13, "NDELTA": 14,
           "LSE2": 15, "DO16": 16, "V16": 17, "DO_R": 18, "V_R": 19, "RQ": 20, "RK": 21}


STAGES = {"FWD_PREPARE": 0, "FWD_ATTN": 1, "BWD_PREPARE": 2, "BWD_DKDV": 3, "BWD_DQ": 4, "BWD_ATTN": 5}


class SageBwdError(RuntimeError):
    pass


class Params(ctypes.Structure):
    _fields_ = [("B", ctypes.c_int32), ("H", ctypes.c_int32), ("N", ctypes.c_int32), ("D", ctypes.c_int32),
                ("causal", ctypes.c_int32), ("smooth_q", ctypes.c_int32), ("smooth_k", ctypes.c_int32),
                ("int8_dp", ctypes.c_int32), ("qk_norm", ctypes.c_int32), ("mxfp8", ctypes.c_int32),
                ("fp4", ctypes.c_int32)]


_lib = None
_P = ctypes.POINTER(Params)
_vp = ctypes.c_void_p
_sz = ctypes.c_size_t


def load_library() -> ctypes.CDLL:
    """Load libsagebwd.so (built in-tree); raise if it is missing."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise SageBwdError(f"{LIB_PATH} is not built (run: python bit_trainable_attention_amd/build.py)")
        lib = ctypes.CDLL(LIB_PATH)
        lib.sagebwd_fwd_workspace_size.argtypes = [_P]
        lib.sagebwd_fwd_workspace_size.restype = _sz
        lib.sagebwd_bwd_workspace_size.argtypes = [_P]
        lib.sagebwd_bwd_workspace_size.restype = _sz
        lib.sagebwd_fwd.argtypes = [_P, _vp, _vp, _vp, _vp, _vp, _vp, _sz, _vp]
        lib.sagebwd_fwd.restype = ctypes.c_int
        lib.sagebwd_bwd.argtypes = [_P, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _sz, _vp, _sz, _vp]
        lib.sagebwd_bwd.restype = ctypes.c_int
        lib.sagebwd_fwd_stage.argtypes = [_P, ctypes.c_int, _vp, _vp, _vp, _vp, _vp, _vp, _sz, _vp]
        lib.sagebwd_fwd_stage.restype = ctypes.c_int
        lib.sagebwd_bwd_stage.argtypes = [_P, ctypes.c_int, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _sz,
                                          _vp, _sz, _vp]
        lib.sagebwd_bwd_stage.restype = ctypes.c_int
        lib.sagebwd_debug_tile.argtypes = [_P, ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                           _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _sz, _vp, _sz, _vp]
        lib.sagebwd_debug_tile.restype = ctypes.c_int
        lib.sagebwd_prepare.argtypes = [_P, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _sz, _vp]
        lib.sagebwd_prepare.restype = ctypes.c_int
        lib.sagebwd_ws_region.argtypes = [_P, ctypes.c_int, ctypes.POINTER(_sz), ctypes.POINTER(_sz)]
        lib.sagebwd_ws_region.restype = ctypes.c_int
        lib.sagebwd_fwd_noalloc.argtypes = [_P, _vp, _vp, _vp, _vp, _vp, _vp]
        lib.sagebwd_fwd_noalloc.restype = ctypes.c_int
        lib.sagebwd_check_block_scale.argtypes = [ctypes.c_int, ctypes.c_int, _vp, _vp, _vp, _vp]
        lib.sagebwd_check_block_scale.restype = ctypes.c_int
        lib.sagebwd_status_string.argtypes = [ctypes.c_int]
        lib.sagebwd_status_string.restype = ctypes.c_char_p
        _lib = lib
    return _lib


def make_params(B, H, N, causal, smooth_q, smooth_k, D=64, int8_dp=False, qk_norm=False, mxfp8=False,
                fp4=False) -> Params:
    """int8_dp: the all-INT8 ablation (dO V^T from INT8 codes); backward only.
    qk_norm: QK-norm fused in; mxfp8: E4M3 codes with E8M0 32x32 block scales
    instead of INT8 (both: same value for forward and backward); fp4: the
    MXFP4 inference forward (forward only)."""
    return Params(int(B), int(H), int(N), int(D), int(bool(causal)), int(bool(smooth_q)), int(bool(smooth_k)),
                  int(bool(int8_dp)), int(bool(qk_norm)), int(bool(mxfp8)), int(bool(fp4)))


def _check(rc: int, what: str):
    if rc != 0:
        msg = load_library().sagebwd_status_string(rc).decode()
        raise SageBwdError(f"{what} failed: {msg} ({rc})")


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream():
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def _check_qkv(*ts):
    ref = ts[0]
    for t in ts:
        if not (t.is_cuda and t.dtype == torch.bfloat16 and t.is_contiguous()):
            raise SageBwdError("inputs must be contiguous bfloat16 CUDA tensors [B, H, N, 64]")
        if t.shape != ref.shape or t.dim() != 4:
            raise SageBwdError(f"shape mismatch: {tuple(t.shape)} vs {tuple(ref.shape)}")


def workspace_size(B, H, N, causal=False, smooth_q=False, smooth_k=True, backward=False, int8_dp=False,
                   qk_norm=False, mxfp8=False, fp4=False) -> int:
    p = make_params(B, H, N, causal, smooth_q, smooth_k, int8_dp=int8_dp, qk_norm=qk_norm, mxfp8=mxfp8, fp4=fp4)
    lib = load_library()
    n = (lib.sagebwd_bwd_workspace_size if backward else lib.sagebwd_fwd_workspace_size)(ctypes.byref(p))
    if n == 0:
        raise SageBwdError("invalid parameters")
    return int(n)


def _workspace(nbytes, device, ws=None):
    if ws is not None:
        if ws.numel() * ws.element_size() < nbytes:
            raise SageBwdError("workspace too small")
        return ws
    return torch.empty(nbytes, dtype=torch.uint8, device=device)


def fwd(q, k, v, causal=False, smooth_q=False, smooth_k=True, workspace=None, out=None, qk_norm=False,
        mxfp8=False, fp4=False):
    """Forward.  Returns (O bf16 [B,H,N,64], LSE fp32 [B,H,N]).  Pass a
    forward-sized uint8 ``workspace`` to keep the quantized Q and K for a
    backward that reuses them (``bwd(..., fwd_workspace=workspace)``)."""
    _check_qkv(q, k, v)
    B, H, N, D = q.shape
    p = make_params(B, H, N, causal, smooth_q, smooth_k, D, qk_norm=qk_norm, mxfp8=mxfp8, fp4=fp4)
    lib = load_library()
    ws = _workspace(lib.sagebwd_fwd_workspace_size(ctypes.byref(p)), q.device, workspace)
    if out is None:
        o = torch.empty_like(q)
        lse = torch.empty((B, H, N), dtype=torch.float32, device=q.device)
    else:
        o, lse = out
    rc = lib.sagebwd_fwd(ctypes.byref(p), _ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), _ptr(ws),
                         ws.numel() * ws.element_size(), _stream())
    _check(rc, "sagebwd_fwd")
    return o, lse


def bwd(q, k, v, o, lse, do, causal=False, smooth_q=False, smooth_k=True, workspace=None, out=None,
        fwd_workspace=None, int8_dp=False, qk_norm=False, mxfp8=False):
    """Backward.  Returns (dQ, dK, dV) bf16 [B,H,N,64].  ``fwd_workspace``:
    the workspace of the forward call on the same q, k, v and flags, whose
    quantized Q and K are then reused (bit-identical results).  ``int8_dp``:
    the all-INT8 ablation (dO V^T from INT8 codes instead of FP16)."""
    _check_qkv(q, k, v, o, do)
    if not (lse.is_cuda and lse.dtype == torch.float32 and lse.is_contiguous() and lse.shape == q.shape[:3]):
        raise SageBwdError("lse must be a contiguous float32 CUDA tensor [B, H, N]")
    B, H, N, D = q.shape
    p = make_params(B, H, N, causal, smooth_q, smooth_k, D, int8_dp, qk_norm, mxfp8)
    lib = load_library()
    ws = _workspace(lib.sagebwd_bwd_workspace_size(ctypes.byref(p)), q.device, workspace)
    if out is None:
        dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    else:
        dq, dk, dv = out
    fws = fwd_workspace
    rc = lib.sagebwd_bwd(ctypes.byref(p), _ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), _ptr(do),
                         _ptr(dq), _ptr(dk), _ptr(dv), _ptr(fws), 0 if fws is None else fws.numel() * fws.element_size(),
                         _ptr(ws), ws.numel() * ws.element_size(), _stream())
    _check(rc, "sagebwd_bwd")
    return dq, dk, dv


def fwd_stage(stage, q, k, v, o, lse, ws, params: Params):
    """Run one forward stage (see STAGES) on caller-owned buffers; no checks
    beyond the library's own."""
    rc = load_library().sagebwd_fwd_stage(ctypes.byref(params), STAGES[stage] if isinstance(stage, str) else stage,
                                          _ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), _ptr(ws),
                                          ws.numel() * ws.element_size(), _stream())
    _check(rc, f"sagebwd_fwd_stage({stage})")


def bwd_stage(stage, q, k, v, o, lse, do, dq, dk, dv, ws, params: Params, fwd_ws=None):
    """Run one backward stage (see STAGES) on caller-owned buffers; fwd_ws as
    in bwd()."""
    rc = load_library().sagebwd_bwd_stage(ctypes.byref(params), STAGES[stage] if isinstance(stage, str) else stage,
                                          _ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), _ptr(do), _ptr(dq),
                                          _ptr(dk), _ptr(dv), _ptr(fwd_ws),
                                          0 if fwd_ws is None else fwd_ws.numel() * fwd_ws.element_size(),
                                          _ptr(ws), ws.numel() * ws.element_size(), _stream())
    _check(rc, f"sagebwd_bwd_stage({stage})")


def prepare(q, k, v, o=None, lse=None, do=None, causal=False, smooth_q=False, smooth_k=True, int8_dp=False,
            qk_norm=False, mxfp8=False, fp4=False):
    """Run only the preparation kernels into a fresh backward-sized workspace
    (uint8 tensor) for inspection; see ws_region for the layout."""
    _check_qkv(q, k, v)
    B, H, N, D = q.shape
    p = make_params(B, H, N, causal, smooth_q, smooth_k, D, int8_dp, qk_norm, mxfp8, fp4)
    lib = load_library()
    nbytes = lib.sagebwd_bwd_workspace_size(ctypes.byref(p))
    ws = torch.zeros(nbytes, dtype=torch.uint8, device=q.device)
    rc = lib.sagebwd_prepare(ctypes.byref(p), _ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), _ptr(do),
                             _ptr(ws), nbytes, _stream())
    _check(rc, "sagebwd_prepare")
    return ws


DUMP_BYTES = 90368
DEBUG_KERNELS = {"fwd": 0, "dkdv": 1, "dq": 2}


def debug_tile(kernel, bh, qblock, kblock, q, k, v, o, lse, do=None, causal=False, smooth_q=False,
               smooth_k=True, int8_dp=False, qk_norm=False, mxfp8=False, return_grads=False, fp4=False):
    """Run one attention kernel's debug instantiation and return the raw
    SAGEBWD_DUMP_BYTES dump of tile (bh, qblock, kblock) as a CPU uint8
    tensor (see include/sagebwd.h for the layout).  kernel: "fwd" writes into
    o and lse; "dkdv" and "dq" read o, lse and do.  With return_grads, also
    the (dQ, dK, dV) buffers the backward kernels wrote (None for "fwd").
    fp4: the FP4 inference forward ("fwd" only)."""
    _check_qkv(q, k, v)
    B, H, N, D = q.shape
    p = make_params(B, H, N, causal, smooth_q, smooth_k, D, int8_dp, qk_norm, mxfp8, fp4)
    lib = load_library()
    nbytes = (lib.sagebwd_fwd_workspace_size if fp4 else lib.sagebwd_bwd_workspace_size)(ctypes.byref(p))
    ws = torch.empty(nbytes, dtype=torch.uint8, device=q.device)
    dump = torch.zeros(DUMP_BYTES, dtype=torch.uint8, device=q.device)
    kid = DEBUG_KERNELS[kernel]
    grads = [torch.empty_like(q) for _ in range(3)] if kid else [None, None, None]
    rc = lib.sagebwd_debug_tile(ctypes.byref(p), kid, int(bh), int(qblock), int(kblock), _ptr(q), _ptr(k), _ptr(v),
                                _ptr(o), _ptr(lse), _ptr(do), _ptr(grads[0]), _ptr(grads[1]), _ptr(grads[2]),
                                _ptr(dump), DUMP_BYTES, _ptr(ws), ws.numel(), _stream())
    _check(rc, "sagebwd_debug_tile")
    torch.cuda.synchronize()
    if return_grads:
        return dump.cpu(), grads
    return dump.cpu()


def check_block_scale(e_lo: int, e_hi: int, keep_first: bool = False):
    """Run the library's exhaustive block-scale check over the exponents
    [e_lo, e_hi]; returns (mismatches of a/127, mismatches of 127/a), plus
    with keep_first the fast quotients (a/127, 127/a) of every mantissa of
    exponent e_lo as CPU float32 tensors."""
    counts = torch.zeros(2, dtype=torch.int64, device="cuda")
    outs = [torch.empty(1 << 23, dtype=torch.float32, device="cuda") for _ in range(2)] if keep_first else [None, None]
    rc = load_library().sagebwd_check_block_scale(int(e_lo), int(e_hi), _ptr(counts), _ptr(outs[0]), _ptr(outs[1]),
                                                  _stream())
    _check(rc, "sagebwd_check_block_scale")
    torch.cuda.synchronize()
    res = tuple(int(c) for c in counts.cpu().tolist())
    if keep_first:
        return res + (outs[0].cpu(), outs[1].cpu())
    return res


def ws_region(params: Params, region) -> tuple:
    """(byte offset, byte size) of a workspace region (name or id)."""
    rid = REGIONS[region] if isinstance(region, str) else int(region)
    off, nb = _sz(), _sz()
    _check(load_library().sagebwd_ws_region(ctypes.byref(params), rid, ctypes.byref(off), ctypes.byref(nb)),
           "sagebwd_ws_region")
    return int(off.value), int(nb.value)


class SageBwdAttention(torch.autograd.Function):
    """Autograd wrapper: forward and backward both run the HIP library; the
    backward reuses the forward's quantized Q and K (its workspace is kept)."""

    @staticmethod
    def forward(ctx, q, k, v, causal=False, smooth_q=False, smooth_k=True, qk_norm=False, mxfp8=False):
        q, k, v = q.contiguous(), k.contiguous(), v.contiguous()
        B, H, N, D = q.shape
        ws = torch.empty(workspace_size(B, H, N, causal, smooth_q, smooth_k, qk_norm=qk_norm, mxfp8=mxfp8),
                         dtype=torch.uint8, device=q.device)
        o, lse = fwd(q, k, v, causal, smooth_q, smooth_k, workspace=ws, qk_norm=qk_norm, mxfp8=mxfp8)
        ctx.save_for_backward(q, k, v, o, lse, ws)
        ctx.flags = (causal, smooth_q, smooth_k)
        ctx.modes = dict(qk_norm=qk_norm, mxfp8=mxfp8)
        return o

    @staticmethod
    def backward(ctx, do):
        q, k, v, o, lse, ws = ctx.saved_tensors
        dq, dk, dv = bwd(q, k, v, o, lse, do.contiguous(), *ctx.flags, fwd_workspace=ws, **ctx.modes)
        return dq, dk, dv, None, None, None, None, None
