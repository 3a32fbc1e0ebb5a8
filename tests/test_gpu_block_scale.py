"""The kernels' block-scale arithmetic, exhaustively (SageBwd abstract: INT8
blocks with absmax/127 scales).  Every INT8 block scale s = a/127 and its
inverse 127/a is formed by a fast fused sequence (quot127, div127 in the HIP
sources); this runs the library's check over every float32 absmax the
kernels use, a in [2^-100, 2^128) (exponents -100..127, all 2^23 mantissas),
against the compiled IEEE divisions on the GPU: no mismatch is allowed.  The
quotients of one whole binade are also compared with the host's IEEE float32
division (numpy), so the check does not rest on the device's division alone."""
import numpy as np
import pytest
import torch

import bit_trainable_attention_amd as sb

pytestmark = pytest.mark.gpu


def test_block_scale_quotients_exhaustive():
    bad_s, bad_inv = sb.check_block_scale(-100, 127)
    assert (bad_s, bad_inv) == (0, 0)


@pytest.mark.parametrize("e", [-100, -1, 0, 126, 127])
def test_block_scale_quotients_match_host_division(e):
    bad_s, bad_inv, s, inv = sb.check_block_scale(e, e, keep_first=True)
    assert (bad_s, bad_inv) == (0, 0)
    m = np.arange(1 << 23, dtype=np.uint32)
    a = (np.uint32(e + 127) << 23 | m).view(np.float32)
    assert np.array_equal(s.numpy(), a / np.float32(127.0))
    assert np.array_equal(inv.numpy(), np.float32(127.0) / a)


def test_block_scale_check_rejects_bad_ranges():
    lib = sb.load_library()
    c = torch.zeros(2, dtype=torch.int64, device="cuda")
    for lo, hi in ((-127, 0), (0, 128), (5, 4)):
        assert lib.sagebwd_check_block_scale(lo, hi, sb._ptr(c), None, None, sb._stream()) == -1
