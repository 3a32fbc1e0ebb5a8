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


# Bars of the element-wise parity checks (HIP against the oracle of the same
# mode): whole-tensor relative L2 (the stated tolerance), and the worst single
# row and worst 64-row tile, so that one wrong row or block cannot hide in the
# whole-tensor norm.  The 8-bit-float and FP4 modes allow more per row: one P~
# code that lands on the neighbouring E4M3 / E2M1 value (the two sides round
# scores differently) moves that key's weight by up to 1/16 (1/4).
BARS = {"int8": (1e-2, 3e-2, 1.5e-2), "mxfp8": (1e-2, 0.15, 0.05), "fp4": (1e-2, 0.3, 0.1)}


def parity(name, got, ref, mode="int8", where=""):
    """Assert HIP output ``got`` against the oracle's ``ref`` ([..., rows, 64]
    arrays) within the mode's bars; returns and prints the three measures."""
    from oracle import metrics as M
    rel, row, tile = BARS[mode]
    r = {"rel_l2": M.rel_l2(got, ref), "worst_row": M.worst_row_rel(got, ref), "worst_tile": M.worst_tile_rel(got, ref)}
    print(f"  {name}{where}: rel-L2 {r['rel_l2']:.2e}  worst row {r['worst_row']:.2e}  worst tile "
          f"{r['worst_tile']:.2e}", flush=True)
    assert r["rel_l2"] <= rel, (name, r)
    assert r["worst_row"] <= row, (name, r)
    assert r["worst_tile"] <= tile, (name, r)
    return r
