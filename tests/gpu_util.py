"""Helpers shared by the GPU tests: moving seeded inputs to the device and
decoding the library's code-block layouts (index bookkeeping only)."""
import numpy as np
import torch

import bit_trainable_attention_amd as sb
import workloads as W


def dev(bits: np.ndarray) -> torch.Tensor:
    """uint16 bf16 bit patterns -> contiguous bf16 CUDA tensor (same bytes)."""
    t = torch.from_numpy(np.ascontiguousarray(bits).view(np.int16))
    return t.view(torch.bfloat16).cuda()


def host_bits(t: torch.Tensor) -> np.ndarray:
    return t.detach().cpu().contiguous().view(torch.int16).numpy().view(np.uint16)


def host_f32(t: torch.Tensor) -> np.ndarray:
    """bf16 CUDA tensor -> float32 numpy (exact)."""
    return W.bf16_bits_to_f32(host_bits(t))


def _perm(kind: str) -> np.ndarray:
    """perm[r*64 + c] = byte offset of (token r, channel c) in a 4 KB block."""
    r = np.arange(64)[:, None]
    c = np.arange(64)[None, :]
    if kind == "row":
        off = (((r // 32) * 2 + c // 32) * 64 + 32 * ((c % 32) // 16) + r % 32) * 16 + c % 16
    else:
        off = (((c // 32) * 2 + r // 32) * 64 + 32 * ((r % 8) // 4) + c % 32) * 16 + 4 * ((r % 32) // 8) + r % 4
    return off.ravel()


_PERMS = {"row": _perm("row"), "t": _perm("t")}


def region(ws_host: np.ndarray, params, name: str, dtype) -> np.ndarray:
    off, nb = sb.ws_region(params, name)
    return ws_host[off:off + nb].view(dtype)


def decode_codes(ws_host, params, name, kind, BH, T) -> np.ndarray:
    """Code blocks of one region -> int8 [BH, T*64, 64] in natural order."""
    raw = region(ws_host, params, name, np.int8).reshape(BH, T, 4096)
    out = raw[:, :, _PERMS[kind]].reshape(BH, T, 64, 64)
    return out.reshape(BH, T * 64, 64)


def assert_perms_are_bijections():
    for p in _PERMS.values():
        assert np.array_equal(np.sort(p), np.arange(4096))
