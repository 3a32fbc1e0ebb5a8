"""Host-side checks of the C ABI that need no GPU: the library loads, exports
every function include/sagebwd.h declares, and rejects bad arguments with the
documented status codes before launching anything."""
import ctypes
import os
import re

import pytest

import bit_trainable_attention_amd as sb

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
OK, INVALID, UNSUPPORTED, WORKSPACE, HIPERR = 0, -1, -2, -3, -4


@pytest.fixture(scope="module")
def lib():
    return sb.load_library()


def declared_functions():
    names = set()
    for f in os.listdir(os.path.join(ROOT, "include")):
        if f.endswith(".h"):
            txt = open(os.path.join(ROOT, "include", f)).read()
            txt = re.sub(r"/\*.*?\*/", "", txt, flags=re.S)
            names |= set(re.findall(r"\b(sagebwd_\w+)\s*\(", txt))
    return sorted(names)


def test_exports_every_declared_symbol(lib):
    names = declared_functions()
    assert {"sagebwd_fwd", "sagebwd_bwd", "sagebwd_fwd_workspace_size", "sagebwd_bwd_workspace_size",
            "sagebwd_status_string", "sagebwd_prepare", "sagebwd_ws_region"} <= set(names)
    for n in names:
        assert hasattr(lib, n), n


def P(**kw):
    d = dict(B=1, H=2, N=128, causal=0, smooth_q=0, smooth_k=1, D=64, int8_dp=0, qk_norm=0, mxfp8=0, fp4=0)
    d.update(kw)
    return sb.Params(d["B"], d["H"], d["N"], d["D"], d["causal"], d["smooth_q"], d["smooth_k"], d["int8_dp"],
                     d["qk_norm"], d["mxfp8"], d["fp4"])


FAKE = 1 << 20          # aligned, never dereferenced: every call below fails validation first


def call_fwd(lib, p, q=FAKE, k=FAKE, v=FAKE, o=FAKE, lse=FAKE, ws=FAKE, nbytes=1 << 40):
    return lib.sagebwd_fwd(None if p is None else ctypes.byref(p), q, k, v, o, lse, ws, nbytes, None)


def call_bwd(lib, p, ptrs=None, lse=FAKE, ws=FAKE, nbytes=1 << 40, fwd_ws=None, fwd_nbytes=0):
    q, k, v, o, do, dq, dk, dv = ptrs or [FAKE] * 8
    return lib.sagebwd_bwd(None if p is None else ctypes.byref(p), q, k, v, o, lse, do, dq, dk, dv, fwd_ws, fwd_nbytes,
                           ws, nbytes, None)


def test_param_validation(lib):
    assert call_fwd(lib, None) == INVALID
    assert call_fwd(lib, P(B=0)) == INVALID
    assert call_fwd(lib, P(H=-1)) == INVALID
    assert call_fwd(lib, P(N=0)) == INVALID
    assert call_fwd(lib, P(causal=2)) == INVALID
    assert call_fwd(lib, P(smooth_q=-1)) == INVALID
    assert call_fwd(lib, P(smooth_k=7)) == INVALID
    assert call_fwd(lib, P(int8_dp=2)) == INVALID
    assert call_bwd(lib, P(int8_dp=-1)) == INVALID
    assert call_fwd(lib, P(qk_norm=3)) == INVALID
    assert call_fwd(lib, P(mxfp8=2)) == INVALID
    assert call_bwd(lib, P(mxfp8=1, int8_dp=1)) == UNSUPPORTED     # the INT8 ablation has no MXFP8 form
    assert lib.sagebwd_bwd_workspace_size(ctypes.byref(P(mxfp8=1, int8_dp=1))) == 0
    assert lib.sagebwd_bwd_workspace_size(ctypes.byref(P(mxfp8=1))) == lib.sagebwd_bwd_workspace_size(ctypes.byref(P()))
    assert call_fwd(lib, P(fp4=2)) == INVALID
    assert call_fwd(lib, P(fp4=1, mxfp8=1)) == UNSUPPORTED
    assert call_bwd(lib, P(fp4=1, int8_dp=1)) == UNSUPPORTED
    assert call_bwd(lib, P(fp4=1)) == UNSUPPORTED                     # the FP4 mode is a forward only
    for stage in range(2, 6):
        assert lib.sagebwd_bwd_stage(ctypes.byref(P(fp4=1)), stage, *([FAKE] * 9), None, 0, FAKE, 1 << 40,
                                     None) == UNSUPPORTED
    assert lib.sagebwd_prepare(ctypes.byref(P(fp4=1)), FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 1 << 40,
                               None) == UNSUPPORTED
    # FP4 has no backward kernels to dump
    for kernel in (1, 2):
        assert lib.sagebwd_debug_tile(ctypes.byref(P(fp4=1)), kernel, 0, 0, 0, *([FAKE] * 10), FAKE, 1 << 20, FAKE,
                                      1 << 40, None) == UNSUPPORTED
    assert call_fwd(lib, P(D=128)) == UNSUPPORTED
    assert call_fwd(lib, P(N=(1 << 18) + 1)) == UNSUPPORTED
    assert call_fwd(lib, P(B=256, H=256)) == UNSUPPORTED
    assert call_bwd(lib, P(D=32)) == UNSUPPORTED
    assert call_bwd(lib, P(N=-5)) == INVALID


def test_pointer_validation(lib):
    p = P()
    assert call_fwd(lib, p, q=None) == INVALID
    assert call_fwd(lib, p, v=FAKE + 2) == INVALID          # bf16 tensors need 16-byte alignment
    assert call_fwd(lib, p, lse=None) == INVALID
    assert call_fwd(lib, p, lse=FAKE + 2) == INVALID
    assert call_fwd(lib, p, ws=None) == INVALID
    assert call_fwd(lib, p, ws=FAKE + 128) == INVALID       # workspace needs 256-byte alignment
    for i in range(8):
        ptrs = [FAKE] * 8
        ptrs[i] = None
        assert call_bwd(lib, p, ptrs) == INVALID
        ptrs[i] = FAKE + 8
        assert call_bwd(lib, p, ptrs) == INVALID
    assert call_bwd(lib, p, lse=None) == INVALID


def test_workspace_validation(lib):
    p = P(N=1000, causal=1, smooth_q=1)
    nf = lib.sagebwd_fwd_workspace_size(ctypes.byref(p))
    nb = lib.sagebwd_bwd_workspace_size(ctypes.byref(p))
    assert 0 < nf < nb
    assert call_fwd(lib, p, nbytes=nf - 1) == WORKSPACE
    assert call_bwd(lib, p, nbytes=nb - 1) == WORKSPACE
    assert call_bwd(lib, p, nbytes=nf) == WORKSPACE
    bad = P(D=16)
    assert lib.sagebwd_fwd_workspace_size(ctypes.byref(bad)) == 0
    assert lib.sagebwd_bwd_workspace_size(ctypes.byref(bad)) == 0
    assert lib.sagebwd_fwd_workspace_size(None) == 0


def test_prepare_validation(lib):
    p = P()
    f = lambda *a: lib.sagebwd_prepare(ctypes.byref(p), *a, None)
    assert f(FAKE, FAKE, FAKE, None, FAKE, None, FAKE, 1 << 40) == INVALID   # LSE without dO
    assert f(FAKE, FAKE, FAKE, FAKE, None, FAKE, FAKE, 1 << 40) == INVALID   # dO without LSE
    assert f(None, FAKE, FAKE, None, None, None, FAKE, 1 << 40) == INVALID
    assert f(FAKE, FAKE, FAKE, None, None, None, FAKE, 10) == WORKSPACE


@pytest.mark.parametrize("int8_dp,qk_norm,mxfp8", [(0, 0, 0), (1, 0, 0), (0, 1, 0), (1, 1, 0), (0, 0, 1), (0, 1, 1)])
def test_ws_regions_layout(lib, int8_dp, qk_norm, mxfp8):
    for N in (1, 63, 64, 65, 1000, 17776):
        p = P(B=2, H=3, N=N, int8_dp=int8_dp, qk_norm=qk_norm, mxfp8=mxfp8)
        BH, T = 6, (N + 63) // 64
        Np = 64 * T
        expect = {"MU_Q": BH * 256, "MU_K": BH * 256, "Q_R": BH * T * 4096, "K_R": BH * T * 4096,
                  "V_T": BH * T * 4096, "Q_T": BH * T * 4096, "K_T": BH * T * 4096, "DO_T": BH * T * 4096,
                  "S_Q": BH * T * 4, "S_K": BH * T * 4, "S_V": BH * T * 4, "S_DO": BH * T * 4,
                  "CORR": BH * Np * 4, "BIAS": BH * Np * 4, "NDELTA": BH * Np * 4, "LSE2": BH * Np * 4,
                  "DO16": BH * Np * 128, "V16": BH * Np * 128,
                  "DO_R": int8_dp * BH * T * 4096, "V_R": int8_dp * BH * T * 4096,
                  "RQ": qk_norm * BH * Np * 4, "RK": qk_norm * BH * Np * 4}
        spans = []
        for name, rid in sb.REGIONS.items():
            off, nb = sb.ws_region(p, rid)
            assert off % 256 == 0
            assert nb == expect[name], (name, nb)
            if nb:
                spans.append((off, off + nb))
        spans.sort()
        for (a0, a1), (b0, b1) in zip(spans, spans[1:]):
            assert a1 <= b0
        total = lib.sagebwd_bwd_workspace_size(ctypes.byref(p))
        assert spans[-1][1] <= total
    off, nb = ctypes.c_size_t(), ctypes.c_size_t()
    assert lib.sagebwd_ws_region(ctypes.byref(P()), len(sb.REGIONS), ctypes.byref(off), ctypes.byref(nb)) == INVALID
    assert lib.sagebwd_ws_region(ctypes.byref(P()), -1, ctypes.byref(off), ctypes.byref(nb)) == INVALID


def test_status_strings(lib):
    for rc, s in ((OK, b"ok"), (INVALID, b"invalid argument"), (UNSUPPORTED, b"unsupported shape"),
                  (WORKSPACE, b"workspace too small"), (HIPERR, b"HIP launch error"),
                  (-5, b"workspace exceeds the built-in scratch buffer"), (-99, b"unknown status")):
        assert lib.sagebwd_status_string(rc) == s


def test_binding_rejects_cpu_tensors():
    import torch
    q = torch.zeros(1, 1, 8, 64, dtype=torch.bfloat16)
    with pytest.raises(sb.SageBwdError):
        sb.fwd(q, q, q)


def test_stage_validation(lib):
    p = P()
    f = lambda stage, nb=1 << 40: lib.sagebwd_fwd_stage(ctypes.byref(p), stage, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, nb, None)
    b = lambda stage, nb=1 << 40: lib.sagebwd_bwd_stage(ctypes.byref(p), stage, *([FAKE] * 9), None, 0, FAKE, nb, None)
    for bad in (-1, 2, 3, 4, 5):
        assert f(bad) == INVALID
    for bad in (-1, 0, 1, 6):
        assert b(bad) == INVALID
    assert f(0, nb=1) == WORKSPACE and f(1, nb=1) == WORKSPACE
    assert b(2, nb=1) == WORKSPACE and b(3, nb=1) == WORKSPACE and b(4, nb=1) == WORKSPACE and b(5, nb=1) == WORKSPACE


def test_forward_workspace_validation(lib):
    """A reused forward workspace is checked like the backward's own: aligned,
    large enough, and not overlapping it (every case fails before any HIP
    call)."""
    p = P(causal=1, smooth_q=1)
    fsz = lib.sagebwd_fwd_workspace_size(ctypes.byref(p))
    bsz = lib.sagebwd_bwd_workspace_size(ctypes.byref(p))
    ws = 1 << 30
    assert call_bwd(lib, p, ws=ws, nbytes=bsz, fwd_ws=(1 << 34) + 16, fwd_nbytes=fsz) == INVALID     # misaligned
    assert call_bwd(lib, p, ws=ws, nbytes=bsz, fwd_ws=1 << 34, fwd_nbytes=fsz - 1) == WORKSPACE
    assert call_bwd(lib, p, ws=ws, nbytes=bsz, fwd_ws=ws, fwd_nbytes=fsz) == INVALID                  # same buffer
    assert call_bwd(lib, p, ws=ws, nbytes=bsz, fwd_ws=ws + bsz - 256, fwd_nbytes=fsz) == INVALID      # overlaps the end
    assert call_bwd(lib, p, ws=ws, nbytes=bsz, fwd_ws=ws - fsz + 256, fwd_nbytes=fsz) == INVALID      # overlaps the start
    # the forward layout holds every region the backward reads from it
    assert fsz < bsz


@pytest.mark.parametrize("B,H,N,causal", [(1, 32, 16384, 1), (2, 30, 17776, 0), (1, 4, 1 << 18, 1), (8, 16, 2048, 1),
                                          (3, 1, 100, 0)])
def test_backward_workspace_is_linear_in_n(lib, B, H, N, causal):
    """The backward keeps nothing of size N^2: its workspace is the forward's
    regions plus per-token rows (dO codes, FP16 dO and V, -Delta, log2 LSE),
    so doubling N at most doubles it (plus alignment), and the two attention
    stages run on their own for any shape.  Every call fails before any HIP
    call (the pointers are never dereferenced)."""
    p = P(B=B, H=H, N=N, causal=causal)
    p2 = P(B=B, H=H, N=min(2 * N, 1 << 18), causal=causal)
    n1 = lib.sagebwd_bwd_workspace_size(ctypes.byref(p))
    n2 = lib.sagebwd_bwd_workspace_size(ctypes.byref(p2))
    T = (N + 63) // 64
    assert n1 <= B * H * T * 64 * 64 * 12 + 64 * 256       # about 10.5 bytes per token-channel plus alignment
    assert n2 <= 2 * n1 + 64 * 256
    b = lambda stage: lib.sagebwd_bwd_stage(ctypes.byref(p), stage, *([FAKE] * 9), None, 0, FAKE, 1, None)
    assert b(3) == WORKSPACE and b(4) == WORKSPACE


def test_block_scale_check_validation(lib):
    """The block-scale self-check rejects exponent ranges outside the normal
    float32 range, reversed ranges, a null counter array and a single output
    pointer before launching anything."""
    for lo, hi in ((-127, 0), (0, 128), (5, 4)):
        assert lib.sagebwd_check_block_scale(lo, hi, FAKE, None, None, None) == INVALID
    assert lib.sagebwd_check_block_scale(0, 0, None, None, None, None) == INVALID
    assert lib.sagebwd_check_block_scale(0, 0, FAKE, FAKE, None, None) == INVALID


def test_noalloc_forward_validation(lib):
    """sagebwd_fwd_noalloc validates like sagebwd_fwd and rejects a problem
    whose workspace exceeds the 256 MiB scratch buffer, all before any HIP
    call."""
    f = lambda p, *ptrs: lib.sagebwd_fwd_noalloc(ctypes.byref(p) if p is not None else None, *ptrs, None)
    assert f(None, FAKE, FAKE, FAKE, FAKE, FAKE) == INVALID
    assert f(P(), None, FAKE, FAKE, FAKE, FAKE) == INVALID
    assert f(P(), FAKE + 8, FAKE, FAKE, FAKE, FAKE) == INVALID
    assert f(P(), FAKE, FAKE, FAKE, FAKE, None) == INVALID
    assert f(P(D=32), FAKE, FAKE, FAKE, FAKE, FAKE) == UNSUPPORTED
    big = P(B=1, H=32, N=32768, causal=1)
    assert lib.sagebwd_fwd_workspace_size(ctypes.byref(big)) > (256 << 20)
    assert f(big, FAKE, FAKE, FAKE, FAKE, FAKE) == -5
    fits = P(B=1, H=32, N=16384, causal=1, smooth_q=1)
    assert lib.sagebwd_fwd_workspace_size(ctypes.byref(fits)) <= (256 << 20)
