"""Replay checks of single tiles: bit-exact INT8 codes, block scales and i32
tile accumulators of the three attention kernels.

The P~, P and dS codes are functions of v_exp_f32 results and of float32
accumulation order, which a float64 oracle cannot reproduce bit for bit.  So
each kernel's debug instantiation dumps one 64x64 tile -- its integer score
accumulator, its float32 pre-quantization values, its codes and scales, and
its integer output products -- and the oracle's own quantizer and exact
integer products must reproduce every code, scale and accumulator from those
values exactly:
  A      = Q_code K_code^T                (oracle codes, exact integers)
  fwd    P~ codes = rne(127 P^) of the dumped values, P~V = codes V_code
  dkdv   s_P, P codes = F3 of the dumped P; P^T dO = codes^T dO_code;
         s_dS, dS codes = F3 of the dumped dS; dS^T Q = codes^T Q_code
  dq     A, the dS values, s_dS and the dS codes, recomputed in the
         forward's layout, bit for bit equal to the dK/dV kernel's;
         dS K = codes K_code
The codes the oracle forms from its own float64 P~, P and dS agree except at
rounding boundaries; that rate is reported and bounded.

The debug instantiations differ from the production kernels only by their
dump stores, which move instructions; so the production forward and
backward are also run on the same inputs and their outputs (O, LSE, dQ, dK,
dV of the dumped head) must equal the debug instantiations' outputs bit for
bit: the replayed codes and products are then those of the production
kernels.  (The library is built without floating-point contraction, so the
compiler cannot fuse a multiply and an add in one instantiation and not in
the other.)"""
import numpy as np
import pytest
import torch

import bit_trainable_attention_amd as sb
import workloads as W
from oracle import faithful as F
from tests import gpu_util as G

pytestmark = pytest.mark.gpu

A, F1, C1, ACC1, F2, C2, ACC2, SC = 0, 16384, 32768, 36864, 53248, 69632, 73728, 90112

CASES = [
    ("tiny", W.WORKLOADS["tiny"], 1, [(0, 0), (1, 1), (0, 1), (1, 0)], False),
    ("ragged_causal", W.custom(1, 2, 200, True, True, True, "kbias", 71), 1, [(3, 3), (3, 0), (2, 1)], False),
    ("pretrain", W.WORKLOADS["pretrain"], 100, [(5, 5), (31, 0), (17, 16)], False),
    ("video", W.WORKLOADS["video"], 33, [(277, 277), (0, 277), (277, 0), (150, 3)], False),
    ("llama16k", W.WORKLOADS["llama16k"], 5, [(255, 255), (255, 0), (100, 99)], False),
    # the all-INT8 ablation: dO V^T from INT8 codes (the dS tile must still be
    # bitwise the same in both backward kernels)
    ("ragged_causal_int8dp", W.custom(1, 2, 200, True, True, True, "kbias", 71), 1, [(3, 3), (3, 0), (2, 1)], True),
    ("video_int8dp", W.WORKLOADS["video"], 33, [(277, 277), (150, 3)], True),
]


def _blk(d, off, dtype):
    return np.frombuffer(d, dtype=dtype, count=4096, offset=off).reshape(64, 64)


@pytest.mark.parametrize("name,w,bh,tiles,int8_dp", CASES, ids=[c[0] for c in CASES])
def test_tile_replay_bitexact(name, w, bh, tiles, int8_dp):
    print(f"[replay] {name} B{w.B} H{w.H} N{w.N} causal={w.causal} head {bh} tiles {tiles}", flush=True)
    b, h = divmod(bh, w.H)
    x = W.make_inputs(w)
    tq, tk, tv, tdo = (G.dev(x[n]) for n in ("q", "k", "v", "do"))
    f = {n: W.bf16_bits_to_f32(x[n][b, h]) for n in x}
    del x
    N, T = w.N, (w.N + 63) // 64
    pp = F.prepare(f["q"], f["k"], f["v"], w.smooth_q, w.smooth_k)
    o_f, lse_f = F.fwd_head(pp, w.causal)
    # O and LSE handed to the backward: the oracle's for the checked head, benign values elsewhere
    o_all = np.zeros((w.B, w.H, N, 64), np.float32)
    lse_all = np.full((w.B, w.H, N), 50.0, np.float32)
    o_all[b, h] = o_f[:N]
    lse_all[b, h] = lse_f[:N]
    to = G.dev(W.f32_to_bf16_bits(o_all))
    tlse = torch.from_numpy(lse_all).cuda()
    o_b = W.bf16_bits_to_f32(W.f32_to_bf16_bits(o_all[b, h]))
    bp = F.prepare_bwd(pp, f["v"], o_b, lse_all[b, h], f["do"], int8_dp)
    fresh_total, fresh_diff = 0, 0
    fwd_total, fwd_diff = 0, 0
    # the production kernels on the same inputs (the backward re-quantizes, as
    # the debug path does)
    po, plse = sb.fwd(tq, tk, tv, w.causal, w.smooth_q, w.smooth_k)
    pgrads = sb.bwd(tq, tk, tv, to, tlse, tdo, w.causal, w.smooth_q, w.smooth_k, int8_dp=int8_dp)
    torch.cuda.synchronize()
    for (i, t) in tiles:
        rows = slice(64 * i, 64 * i + 64)
        cols = slice(64 * t, 64 * t + 64)
        a_ref = pp.qc[rows] @ pp.kc[cols].T
        # ---- forward
        fo, fl = torch.empty_like(tq), torch.empty(w.B, w.H, N, device="cuda")
        d = sb.debug_tile("fwd", bh, i, t, tq, tk, tv, fo, fl, None, w.causal, w.smooth_q, w.smooth_k).numpy().tobytes()
        assert np.array_equal(_blk(d, A, np.int32), a_ref.astype(np.int32)), ("fwd A", i, t)
        v = _blk(d, F1, np.float32)
        codes = _blk(d, C1, np.uint8)
        assert np.all(v >= 0) and np.all(v <= 127.5)
        assert np.array_equal(codes.astype(np.int64), np.rint(v.astype(np.float64)).astype(np.int64)), ("fwd codes", i, t)
        assert np.array_equal(_blk(d, ACC1, np.int32).astype(np.int64),
                              (codes.astype(np.float64) @ pp.vc[cols]).astype(np.int64)), ("fwd PV", i, t)
        assert torch.equal(fo[b, h].view(torch.int16), po[b, h].view(torch.int16)), ("fwd prod O", i, t)
        assert torch.equal(fl[b, h], plse[b, h]), ("fwd prod LSE", i, t)
        _, _, fc, _ = F.fwd_head(pp, w.causal, qblocks=[i], return_codes=True)
        fcode = fc[:, cols]
        keep = np.ones((64, 64), bool)
        if w.causal:
            keep &= (np.arange(64 * t, 64 * t + 64)[None, :] <= np.arange(64 * i, 64 * i + 64)[:, None])
        keep &= (np.arange(64 * i, 64 * i + 64)[:, None] < N) & (np.arange(64 * t, 64 * t + 64)[None, :] < N)
        nd = int(np.sum((fcode != codes) & keep))
        fwd_total += int(np.sum(keep))
        fwd_diff += nd
        # ---- dK/dV kernel
        d1, g1 = sb.debug_tile("dkdv", bh, i, t, tq, tk, tv, to, tlse, tdo, w.causal, w.smooth_q, w.smooth_k,
                               int8_dp, return_grads=True)
        d1 = d1.numpy().tobytes()
        for name, a, pr in (("dK", g1[1], pgrads[1]), ("dV", g1[2], pgrads[2])):
            assert torch.equal(a[b, h].view(torch.int16), pr[b, h].view(torch.int16)), (name + " prod", i, t)
        assert np.array_equal(_blk(d1, A, np.int32), a_ref.astype(np.int32)), ("dkdv A", i, t)
        P = _blk(d1, F1, np.float32)
        sP, invP = F.block_scale(np.max(np.abs(P)))
        sc1 = np.frombuffer(d1, np.float32, 2, SC)
        assert sc1[0].view(np.uint32) == np.float32(sP).view(np.uint32), ("s_P", i, t)
        cP = F.block_codes(P, invP)
        assert np.array_equal(_blk(d1, C1, np.uint8).astype(np.int64), cP.astype(np.int64)), ("P codes", i, t)
        assert np.array_equal(_blk(d1, ACC1, np.int32).astype(np.int64),
                              (cP.T @ bp.doc[rows]).astype(np.int64)), ("P^T dO", i, t)
        dS = _blk(d1, F2, np.float32)
        sdS, invdS = F.block_scale(np.max(np.abs(dS)))
        assert sc1[1].view(np.uint32) == np.float32(sdS).view(np.uint32), ("s_dS", i, t)
        cdS = F.block_codes(dS, invdS)
        assert np.array_equal(_blk(d1, C2, np.int8).astype(np.int64), cdS.astype(np.int64)), ("dS codes", i, t)
        assert np.array_equal(_blk(d1, ACC2, np.int32).astype(np.int64),
                              (cdS.T @ pp.qc[rows]).astype(np.int64)), ("dS^T Q", i, t)
        # ---- dQ kernel: it recomputes the tile in the forward's layout; its
        # score integers, dS values, scale and codes are bitwise the dK/dV
        # kernel's, and its dS K product is exact
        d2, g2 = sb.debug_tile("dq", bh, i, t, tq, tk, tv, to, tlse, tdo, w.causal, w.smooth_q, w.smooth_k,
                               int8_dp, return_grads=True)
        d2 = d2.numpy().tobytes()
        assert torch.equal(g2[0][b, h].view(torch.int16), pgrads[0][b, h].view(torch.int16)), ("dQ prod", i, t)
        assert np.array_equal(_blk(d2, A, np.int32), a_ref.astype(np.int32)), ("dq A", i, t)
        assert np.array_equal(_blk(d2, F2, np.uint32), _blk(d1, F2, np.uint32)), ("dq dS values", i, t)
        assert np.frombuffer(d2, np.float32, 1, SC)[0].view(np.uint32) == sc1[1].view(np.uint32), ("dq s_dS", i, t)
        assert np.array_equal(_blk(d2, C1, np.int8), _blk(d1, C2, np.int8)), ("dq codes", i, t)
        assert np.array_equal(_blk(d2, ACC1, np.int32).astype(np.int64),
                              (cdS @ pp.kc[cols]).astype(np.int64)), ("dS K", i, t)
        # ---- codes the oracle forms from its own float64 values
        tl = F.bwd_tiles(bp, [i], [t], w.causal)
        fresh_total += 2 * 4096
        fresh_diff += int(np.sum(tl["cP"] != cP)) + int(np.sum(tl["cdS"] != cdS))
        print(f"  tile ({i},{t}): bit-exact, production outputs equal; fresh-code differences P~ {nd} of "
              f"{int(np.sum(keep))}, P {int(np.sum(tl['cP'] != cP))} dS {int(np.sum(tl['cdS'] != cdS))} of 4096",
              flush=True)
    assert fresh_diff <= 0.02 * fresh_total, (fresh_diff, fresh_total)
    assert fwd_diff <= 0.02 * max(fwd_total, 1), (fwd_diff, fwd_total)
