"""Pins of the P~ code steps of the oracle's forward (faithful F6 and the
MXFP8 mode's X5) against codes derived independently of them.

A hand-built head of one 64-token block makes query row 0 see the scores
S_0j = (127 - j) / 8, so the tile-row maximum is S_00 and P~_0j = exp(-j/8)
for j = 0..63.  The expected codes are computed here with 40-digit decimal
arithmetic and rounded by hand (round half to even onto the integers for
INT8, onto the E4M3 grid written out from its bit layout for MXFP8), a route
that shares nothing with the oracle's numpy exp and rint.  Each fixture is
also checked to separate the plausible mistakes (floor for rint, 128 or 255
for the fixed scale), so a slip there would fail.

The same row also pins F8/X6 for this case: with V the identity (key j has
a single unit in channel j), O_0j = code_j / sum(codes)."""
from decimal import ROUND_FLOOR, ROUND_HALF_EVEN, Decimal, getcontext

import numpy as np

from oracle import faithful as F, mxfp8 as X

getcontext().prec = 40
NB = 64


def _p_hat():
    """exp(-j/8), j = 0..63, to 40 digits."""
    return [(Decimal(-j) / 8).exp() for j in range(NB)]


def _rne_int(d: Decimal) -> int:
    return int(d.to_integral_value(rounding=ROUND_HALF_EVEN))


def _e4m3_grid():
    """Finite non-negative E4M3 values (code, value), from the bit layout:
    exponent field e, mantissa m: (1 + m/8) 2^(e-7), subnormals m 2^-9."""
    out = []
    for c in range(0x7F):
        e, m = c >> 3, c & 7
        v = Decimal(m) * Decimal(2) ** -9 if e == 0 else (1 + Decimal(m) / 8) * Decimal(2) ** (e - 7)
        out.append((c, v))
    return out


def _e4m3_rne(d: Decimal) -> Decimal:
    grid = _e4m3_grid()
    best = min(abs(v - d) for _, v in grid)
    cands = [(c, v) for c, v in grid if abs(v - d) == best]
    if len(cands) > 1:
        cands = [cv for cv in cands if cv[0] % 2 == 0]
    return cands[0][1]


def _scores_head():
    """q codes: row 0 = unit in channel 0; k codes: key j has 127 - j in
    channel 0; scales 1, so A_0j = 127 - j and S_0j = (127 - j)/8."""
    qc = np.zeros((NB, 64))
    qc[0, 0] = 1.0
    kc = np.zeros((NB, 64))
    kc[:, 0] = 127.0 - np.arange(NB)
    vc = np.eye(NB)                   # key j: unit in channel j
    return qc, kc, vc


def test_faithful_f6_codes_hand_tile():
    qc, kc, vc = _scores_head()
    one = np.ones(1, np.float32)
    z = np.zeros(64, np.float32)
    pp = F.Prepared(NB, 1, z, z, qc, kc, vc, one, one, one, np.zeros(NB), np.zeros(NB), np.zeros((NB, 64)), True)
    o, lse, codes, m = F.fwd_head(pp, causal=False, return_codes=True)
    ph = _p_hat()
    want = [_rne_int(127 * p) for p in ph]
    assert codes[0].tolist() == want
    assert want[0] == 127 and want[-1] == 0
    # the fixture separates the plausible mistakes
    assert want != [int((127 * p).to_integral_value(rounding=ROUND_FLOOR)) for p in ph]
    assert want != [_rne_int(128 * p) for p in ph]
    # F8 on this row: O_0j = code_j / sum(codes), LSE = S_00 + ln(sum(codes)/127)
    tot = sum(want)
    assert np.allclose(o[0], np.array(want) / tot, rtol=0, atol=1e-15)
    assert abs(lse[0] - (127 / 8 + np.log(tot / 127))) < 1e-12


def test_mxfp8_x5_codes_hand_tile():
    qc, kc, vc = _scores_head()
    z = np.zeros(64)
    e0 = np.zeros((2, 2))
    pp = X.Prepared(NB, 1, z, z, qc, kc, vc, e0, e0, e0, np.zeros(NB), np.zeros(NB), np.zeros((NB, 64)), True)
    o, lse, codes, m = X.fwd_head(pp, causal=False, return_codes=True)
    ph = _p_hat()
    want = [_e4m3_rne(256 * p) for p in ph]
    assert [Decimal(float(c)) for c in codes[0]] == want
    assert want[0] == 256
    grid = [v for _, v in _e4m3_grid()]
    floor_grid = [max(v for v in grid if v <= 256 * p) for p in ph]
    assert want != floor_grid
    assert want != [_e4m3_rne(255 * p) for p in ph]
    tot = float(sum(want))
    assert np.allclose(o[0], np.array([float(w) for w in want]) / tot, rtol=0, atol=1e-15)
