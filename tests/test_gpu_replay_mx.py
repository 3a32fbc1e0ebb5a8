"""Replay checks of single tiles of the MXFP8 kernels (bit-exact E4M3 codes and
E8M0 block exponents, and the dQ kernel's recomputed tile against the dK/dV
kernel's) and of the FP4 inference forward (E2M1 codes and exponents).

The MXFP8 forward and backward apply the block scales inside the FP8 matrix
instruction and accumulate O, dK, dV and dQ in its float32 accumulators, so
there is no per-tile integer product to replay; what the oracle can pin
exactly is every quantization decision.  Each kernel's debug instantiation
dumps one 64x64 tile (the float32 scores as the FP8 MFMA returns them, the
values it quantizes, its code bytes and exponents), and:
  fwd    the P~ codes are E4M3(256 P~) of the dumped P~ (oracle X5 rounding),
         P~ = exp2(z - M) of the dumped log2-domain scores z and running
         maxima M (M >= the tile-row maximum; equal to it on the first tile)
  dkdv   the P and dS codes and their exponents per 32x32 block are X2 of
         the dumped P and dS
  dq     the recomputed scores, dS values, dS codes and exponents are
         bitwise the dK/dV kernel's
  scores the dumped scores are the exact products of the oracle's dequantized
         operands up to the FP8 MFMA's own rounding (2^-14 of the sum of
         |terms|)
The debug instantiations differ from the production kernels only by their
dump stores, so the production forward and backward are also run on the same
inputs and their outputs for the dumped head must equal the debug ones bit for
bit.  The codes the oracle forms from its own float64 values agree except at
rounding boundaries; that rate is reported and bounded."""
import numpy as np
import pytest
import torch

import bit_trainable_attention_amd as sb
import workloads as W
from oracle import fp4 as Y, mxfp8 as X
from tests import gpu_util as G

pytestmark = pytest.mark.gpu

A, F1, C1, ACC1, F2, C2, SC = 0, 16384, 32768, 36864, 53248, 69632, 90112
LOG2E = 1.4426950408889634

CASES = [
    ("tiny", W.WORKLOADS["tiny"], 1, [(0, 0), (1, 1), (0, 1), (1, 0)]),
    ("ragged_causal", W.custom(1, 2, 200, True, True, True, "kbias", 71), 1, [(3, 3), (3, 0), (2, 1)]),
    ("llama16k", W.WORKLOADS["llama16k"], 5, [(255, 255), (255, 0), (100, 99)]),
    ("video", W.WORKLOADS["video"], 33, [(277, 277), (0, 277), (150, 3)]),
]


def _blk(d, off, dtype):
    return np.frombuffer(d, dtype=dtype, count=4096, offset=off).reshape(64, 64)


def _check_scores(s_gpu, pp, rows, cols, keep, what):
    """Dumped FP8 products against the exact products of the dequantized
    operands.  The scaled FP8 MFMA does not sum its 64 products exactly in
    float32 (observed: up to ~1.7e-5 of the sum of |terms|, a few float32
    roundings of partial sums), so the bar is 2^-14 of sum |terms|; the
    ratio is returned for the report."""
    exact = pp.qh[rows] @ pp.kh[cols].T
    bound = np.abs(pp.qh[rows]) @ np.abs(pp.kh[cols]).T
    err = np.abs(s_gpu.astype(np.float64) - exact)
    ratio = float(np.max(np.where(keep, err / np.maximum(bound, 1e-30), 0)))
    assert ratio <= 2.0 ** -14, (what, ratio)
    return ratio


def _x2(x):
    """X2 of a 64x64 tile of float32 values: exponents [2, 2] (row block, column
    block) and E4M3 code bytes."""
    x = x.astype(np.float64)
    _, e, _ = X.quantize_blocks(x)
    scaled = x * np.ldexp(1.0, -np.repeat(np.repeat(e, 32, axis=0), 32, axis=1))
    return e, X.e4m3_encode(scaled)


@pytest.mark.parametrize("name,w,bh,tiles", CASES, ids=[c[0] for c in CASES])
def test_mx_tile_replay_bitexact(name, w, bh, tiles):
    print(f"[replay mxfp8] {name} B{w.B} H{w.H} N{w.N} causal={w.causal} head {bh} tiles {tiles}", flush=True)
    b, h = divmod(bh, w.H)
    x = W.make_inputs(w)
    tq, tk, tv, tdo = (G.dev(x[n]) for n in ("q", "k", "v", "do"))
    f = {n: W.bf16_bits_to_f32(x[n][b, h]) for n in x}
    del x
    N = w.N
    pp = X.prepare(f["q"], f["k"], f["v"], w.smooth_q, w.smooth_k)
    o_f, lse_f = X.fwd_head(pp, w.causal)
    o_all = np.zeros((w.B, w.H, N, 64), np.float32)
    lse_all = np.full((w.B, w.H, N), 50.0, np.float32)
    o_all[b, h] = o_f[:N]
    lse_all[b, h] = lse_f[:N]
    to = G.dev(W.f32_to_bf16_bits(o_all))
    tlse = torch.from_numpy(lse_all).cuda()
    bp = X.prepare_bwd(pp, f["v"], W.bf16_bits_to_f32(W.f32_to_bf16_bits(o_all[b, h])), lse_all[b, h], f["do"])
    po, plse = sb.fwd(tq, tk, tv, w.causal, w.smooth_q, w.smooth_k, mxfp8=True)
    pgrads = sb.bwd(tq, tk, tv, to, tlse, tdo, w.causal, w.smooth_q, w.smooth_k, mxfp8=True)
    torch.cuda.synchronize()
    fresh_total = fresh_diff = fwd_total = fwd_diff = 0
    for (i, t) in tiles:
        rows = np.arange(64 * i, 64 * i + 64)
        cols = np.arange(64 * t, 64 * t + 64)
        keep = (rows[:, None] < N) & (cols[None, :] < N)
        if w.causal:
            keep &= cols[None, :] <= rows[:, None]
        live = keep.any(axis=1)
        # ---- forward
        fo, fl = torch.empty_like(tq), torch.empty(w.B, w.H, N, device="cuda")
        d = sb.debug_tile("fwd", bh, i, t, tq, tk, tv, fo, fl, None, w.causal, w.smooth_q, w.smooth_k,
                          mxfp8=True).numpy().tobytes()
        assert torch.equal(fo[b, h].view(torch.int16), po[b, h].view(torch.int16)), ("fwd prod O", i, t)
        assert torch.equal(fl[b, h], plse[b, h]), ("fwd prod LSE", i, t)
        r_fwd = _check_scores(_blk(d, A, np.float32), pp, rows, cols, keep, ("fwd S", i, t))
        # the forward's padded query rows (>= N) are computed but never stored: checked rows < N
        fr = rows < N
        z = _blk(d, F2, np.float32)
        assert np.all(np.isneginf(z[fr][~keep[fr]])) and np.all(np.isfinite(z[keep])), ("fwd z mask", i, t)
        # z = (S + b_j) log2(e) / 8 of the dumped S (the key bias from the GPU preparation: float32)
        zref = (_blk(d, A, np.float32).astype(np.float64) + pp.b[cols][None, :]) * (LOG2E / 8.0)
        assert np.all(np.abs(z[keep] - zref[keep]) <= 1e-6 * (1.0 + np.abs(zref[keep]))), ("fwd z", i, t)
        M = np.frombuffer(d, np.float32, 64, SC)
        zmax = np.max(np.where(keep, z, -np.inf), axis=1)
        assert np.all(M[live] >= zmax[live]), ("fwd running max", i, t)
        if t == 0:
            assert np.array_equal(M[live], zmax[live]), ("fwd first-tile max", i, t)
        pt = _blk(d, F1, np.float32)
        arg = (z.astype(np.float32) + (-M[:, None]).astype(np.float32)).astype(np.float32)
        with np.errstate(invalid="ignore"):
            pref = np.where(keep, np.exp2(arg.astype(np.float64)), 0.0)
        assert np.all((np.abs(pt - pref) <= 2.0 ** -21 * pref + 2.0 ** -120)[fr]), ("fwd P~", i, t)
        assert np.all((pt >= 0) & (pt <= 1)), ("fwd P~ range", i, t)
        codes = _blk(d, C1, np.uint8)
        assert np.array_equal(codes, X.e4m3_encode(256.0 * pt.astype(np.float64))), ("fwd P~ codes", i, t)
        _, _, fc, _ = X.fwd_head(pp, w.causal, qblocks=[i], return_codes=True)
        nd = int(np.sum((fc[:, cols] != X.E4M3_VALUES[codes]) & keep))
        fwd_total += int(np.sum(keep))
        fwd_diff += nd
        # ---- dK/dV kernel
        d1, g1 = sb.debug_tile("dkdv", bh, i, t, tq, tk, tv, to, tlse, tdo, w.causal, w.smooth_q, w.smooth_k,
                               mxfp8=True, return_grads=True)
        d1 = d1.numpy().tobytes()
        for nm, a_, pr in (("dK", g1[1], pgrads[1]), ("dV", g1[2], pgrads[2])):
            assert torch.equal(a_[b, h].view(torch.int16), pr[b, h].view(torch.int16)), (nm + " prod", i, t)
        r_bwd = _check_scores(_blk(d1, A, np.float32), pp, rows, cols, keep, ("dkdv S", i, t))
        P = _blk(d1, F1, np.float32)
        assert np.all(P[~keep] == 0) and np.all((P >= 0) & (P <= 1)), ("P range", i, t)
        eP, cP = _x2(P)
        ex1 = np.frombuffer(d1, np.int32, 8, SC)
        # dump exponents at [2 key half + query half]
        assert np.array_equal(ex1[:4], eP.T.ravel()), ("P exponents", i, t, ex1[:4], eP)
        assert np.array_equal(_blk(d1, C1, np.uint8), cP), ("P codes", i, t)
        dS = _blk(d1, F2, np.float32)
        assert np.all(dS[~keep] == 0), ("dS mask", i, t)
        eS, cS = _x2(dS)
        assert np.array_equal(ex1[4:], eS.T.ravel()), ("dS exponents", i, t, ex1[4:], eS)
        assert np.array_equal(_blk(d1, C2, np.uint8), cS), ("dS codes", i, t)
        # ---- dQ kernel: the same tile recomputed with the operands swapped
        d2, g2 = sb.debug_tile("dq", bh, i, t, tq, tk, tv, to, tlse, tdo, w.causal, w.smooth_q, w.smooth_k,
                               mxfp8=True, return_grads=True)
        d2 = d2.numpy().tobytes()
        assert torch.equal(g2[0][b, h].view(torch.int16), pgrads[0][b, h].view(torch.int16)), ("dQ prod", i, t)
        assert np.array_equal(_blk(d2, A, np.uint32), _blk(d1, A, np.uint32)), ("dq scores", i, t)
        assert np.array_equal(_blk(d2, F2, np.uint32), _blk(d1, F2, np.uint32)), ("dq dS values", i, t)
        assert np.array_equal(_blk(d2, C1, np.uint8), _blk(d1, C2, np.uint8)), ("dq dS codes", i, t)
        assert np.array_equal(np.frombuffer(d2, np.int32, 4, SC + 16), ex1[4:]), ("dq dS exponents", i, t)
        # ---- codes the oracle forms from its own float64 P and dS
        tl = X.bwd_tiles(bp, [i], [t], w.causal)
        dP = int(np.sum(X.E4M3_VALUES[cP] != tl["cP"]))
        dD = int(np.sum(X.E4M3_VALUES[cS] != tl["cdS"]))
        fresh_total += 2 * 4096
        fresh_diff += dP + dD
        print(f"  tile ({i},{t}): codes and exponents bit-exact, dQ tile equal, production outputs equal; "
              f"fresh-code differences P~ {nd} of {int(np.sum(keep))}, P {dP} dS {dD} of 4096; score error / sum|terms| "
              f"{r_fwd:.1e} (fwd) {r_bwd:.1e} (bwd)", flush=True)
    assert fresh_diff <= 0.02 * fresh_total, (fresh_diff, fresh_total)
    assert fwd_diff <= 0.02 * max(fwd_total, 1), (fwd_diff, fwd_total)


FP4_CASES = [
    ("tiny", W.WORKLOADS["tiny"], 1, [(0, 0), (1, 1), (0, 1)]),
    ("ragged_causal", W.custom(1, 2, 200, True, True, True, "kbias", 71), 1, [(3, 3), (3, 0), (2, 1)]),
    ("llama16k", W.WORKLOADS["llama16k"], 5, [(255, 255), (100, 0)]),
]


@pytest.mark.parametrize("name,w,bh,tiles", FP4_CASES, ids=[c[0] for c in FP4_CASES])
def test_fp4_tile_replay_bitexact(name, w, bh, tiles):
    """The FP4 inference forward's tile: the P~ block exponents (one per query
    and key class (key mod 8) div 4) and E2M1 code nibbles are the oracle's
    Y2 of the dumped P~; P~ = exp2(z - M); the FP4 scores against the exact
    products of the oracle's dequantized operands; production O and LSE
    equal the debug instantiation's."""
    print(f"[replay fp4] {name} B{w.B} H{w.H} N{w.N} causal={w.causal} head {bh} tiles {tiles}", flush=True)
    b, h = divmod(bh, w.H)
    x = W.make_inputs(w)
    tq, tk, tv = (G.dev(x[n]) for n in ("q", "k", "v"))
    f = {n: W.bf16_bits_to_f32(x[n][b, h]) for n in ("q", "k", "v")}
    del x
    N = w.N
    pp = Y.prepare(f["q"], f["k"], f["v"], w.smooth_q, w.smooth_k)
    po, plse = sb.fwd(tq, tk, tv, w.causal, w.smooth_q, w.smooth_k, fp4=True)
    torch.cuda.synchronize()
    cls = (np.arange(64) % 8) // 4                    # key class of each key of a tile
    for (i, t) in tiles:
        rows = np.arange(64 * i, 64 * i + 64)
        cols = np.arange(64 * t, 64 * t + 64)
        keep = (rows[:, None] < N) & (cols[None, :] < N)
        if w.causal:
            keep &= cols[None, :] <= rows[:, None]
        fr = rows < N
        live = keep.any(axis=1)
        fo, fl = torch.empty_like(tq), torch.empty(w.B, w.H, N, device="cuda")
        d = sb.debug_tile("fwd", bh, i, t, tq, tk, tv, fo, fl, None, w.causal, w.smooth_q, w.smooth_k,
                          fp4=True).numpy().tobytes()
        assert torch.equal(fo[b, h].view(torch.int16), po[b, h].view(torch.int16)), ("fp4 prod O", i, t)
        assert torch.equal(fl[b, h], plse[b, h]), ("fp4 prod LSE", i, t)
        r_s = _check_scores(_blk(d, A, np.float32), pp, rows, cols, keep, ("fp4 S", i, t))
        z = _blk(d, F2, np.float32)
        assert np.all(np.isneginf(z[fr][~keep[fr]])) and np.all(np.isfinite(z[keep])), ("fp4 z mask", i, t)
        zref = (_blk(d, A, np.float32).astype(np.float64) + pp.b[cols][None, :]) * (LOG2E / 8.0)
        assert np.all(np.abs(z[keep] - zref[keep]) <= 1e-6 * (1.0 + np.abs(zref[keep]))), ("fp4 z", i, t)
        M = np.frombuffer(d, np.float32, 64, SC)
        zmax = np.max(np.where(keep, z, -np.inf), axis=1)
        assert np.all(M[live] >= zmax[live]), ("fp4 running max", i, t)
        if t == 0:
            assert np.array_equal(M[live], zmax[live]), ("fp4 first-tile max", i, t)
        pt = _blk(d, F1, np.float32)
        arg = (z.astype(np.float32) + (-M[:, None]).astype(np.float32)).astype(np.float32)
        with np.errstate(invalid="ignore"):
            pref = np.where(keep, np.exp2(arg.astype(np.float64)), 0.0)
        assert np.all((np.abs(pt - pref) <= 2.0 ** -21 * pref + 2.0 ** -120)[fr]), ("fp4 P~", i, t)
        assert np.all((pt >= 0) & (pt <= 1)), ("fp4 P~ range", i, t)
        # Y2 per (query, key class): exponent, then E2M1 codes of P~ 2^-e
        ex = np.frombuffer(d, np.int32, 128, ACC1).reshape(64, 2)
        ptd = pt.astype(np.float64)
        e_ref = np.stack([Y.fp4_exponent(np.max(ptd[:, cls == c], axis=1)) for c in (0, 1)], axis=1)
        assert np.array_equal(ex, e_ref), ("fp4 exponents", i, t)
        codes = _blk(d, C1, np.uint8)
        scaled = ptd * np.ldexp(1.0, -ex[:, cls])
        assert np.array_equal(codes, Y.e2m1_encode(scaled)), ("fp4 codes", i, t)
        print(f"  tile ({i},{t}): exponents and E2M1 codes bit-exact, production outputs equal; "
              f"score error / sum|terms| {r_s:.1e}", flush=True)
