"""Pins for oracle.exact (textbook attention, float64) against things other
than itself: an independent online formulation, closed forms, central finite
differences, translation invariances and torch's own CPU autograd."""
import numpy as np
import pytest
import torch

from oracle import exact, metrics as M


def _rand(n, d, seed, scale=1.0):
    r = np.random.default_rng(seed)
    return [r.standard_normal((n, d)) * scale for _ in range(4)]


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("n,d", [(7, 4), (33, 8), (70, 16)])
def test_online_matches_dense(causal, n, d):
    q, k, v, _ = _rand(n, d, n * 10 + d, 1.5)
    o1, l1 = exact.fwd(q, k, v, causal)
    o2, l2 = exact.fwd_online(q, k, v, causal, block=16)
    assert np.max(np.abs(o1 - o2)) < 1e-12
    assert np.max(np.abs(l1 - l2)) < 1e-12


@pytest.mark.parametrize("causal", [False, True])
def test_closed_forms(causal):
    n, d = 19, 8
    q, k, v, _ = _rand(n, d, 3)
    # Q = 0: uniform weights over the allowed keys
    o, lse = exact.fwd(np.zeros((n, d)), k, v, causal)
    for i in range(n):
        cnt = i + 1 if causal else n
        assert np.allclose(o[i], v[:cnt].mean(axis=0), atol=1e-13)
        assert abs(lse[i] - np.log(cnt)) < 1e-13
    # V constant: O constant
    vc = np.tile(np.arange(d, dtype=np.float64), (n, 1))
    o, _ = exact.fwd(q, k, vc, causal)
    assert np.allclose(o, vc, atol=1e-13)
    # linearity in V
    o1, _ = exact.fwd(q, k, v, causal)
    o2, _ = exact.fwd(q, k, 3.5 * v, causal)
    assert np.allclose(o2, 3.5 * o1, atol=1e-12)
    if causal:  # first row sees only key 0
        o, lse = exact.fwd(q, k, v, True)
        assert np.allclose(o[0], v[0], atol=1e-14)
        assert abs(lse[0] - q[0] @ k[0] / np.sqrt(d)) < 1e-13


@pytest.mark.parametrize("qk_norm", [False, True], ids=["plain", "qknorm"])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("n,d", [(5, 4), (8, 8), (13, 4)])
def test_finite_differences(causal, n, d, qk_norm):
    """Central differences of L = sum(dO * O) against the analytic backward
    (with QK-norm: through the row normalization of Q and K)."""
    q, k, v, do = _rand(n, d, 100 + n + d)
    if qk_norm:   # rows of different sizes, so the norm is not a no-op
        q = q * np.linspace(0.3, 3.0, n)[:, None]
        k = k * np.linspace(2.0, 0.5, n)[:, None]
    dq, dk, dv = exact.bwd(q, k, v, do, causal, qk_norm=qk_norm)
    h = 1e-6

    def loss(q_, k_, v_):
        return float(np.sum(do * exact.fwd(q_, k_, v_, causal, qk_norm)[0]))

    for which, grad in ((0, dq), (1, dk), (2, dv)):
        num = np.zeros((n, d))
        for i in range(n):
            for c in range(d):
                args_p = [q.copy(), k.copy(), v.copy()]
                args_m = [q.copy(), k.copy(), v.copy()]
                args_p[which][i, c] += h
                args_m[which][i, c] -= h
                num[i, c] = (loss(*args_p) - loss(*args_m)) / (2 * h)
        err = np.linalg.norm(num - grad) / max(np.linalg.norm(grad), 1e-30)
        assert err < 1e-6, (which, err)


@pytest.mark.parametrize("causal", [False, True])
def test_translation_invariances(causal):
    n, d = 40, 16
    q, k, v, do = _rand(n, d, 9)
    mu = np.random.default_rng(5).standard_normal(d) * 3
    o1, l1 = exact.fwd(q, k, v, causal)
    o2, l2 = exact.fwd(q, k - mu, v, causal)
    assert np.max(np.abs(o1 - o2)) < 1e-12
    assert np.max(np.abs((l1 - l2) - q @ mu / np.sqrt(d))) < 1e-11
    g1 = exact.bwd(q, k, v, do, causal)
    g2 = exact.bwd(q, k - mu, v, do, causal)
    for a, b in zip(g1, g2):
        assert np.max(np.abs(a - b)) < 1e-11
    assert np.max(np.abs(g1[1].sum(axis=0))) < 1e-11          # sum_j dK_j = 0
    ds = exact.dscores(q, k, v, do, causal)
    assert np.max(np.abs(ds.sum(axis=1))) < 1e-12              # rowsum dS = 0


@pytest.mark.parametrize("causal", [False, True])
def test_matches_torch_autograd(causal):
    n, d = 50, 64
    q, k, v, do = _rand(n, d, 21)
    o, lse = exact.fwd(q, k, v, causal)
    dq, dk, dv = exact.bwd(q, k, v, do, causal)
    tq, tk, tv = (torch.tensor(x, dtype=torch.float64, requires_grad=True) for x in (q, k, v))
    to = torch.nn.functional.scaled_dot_product_attention(tq[None, None], tk[None, None], tv[None, None],
                                                          is_causal=causal)[0, 0]
    to.backward(torch.tensor(do))
    assert np.max(np.abs(o - to.detach().numpy())) < 1e-12
    for a, t in ((dq, tq), (dk, tk), (dv, tv)):
        assert np.max(np.abs(a - t.grad.numpy())) < 1e-11
    s = (torch.tensor(q) @ torch.tensor(k).T) / 8.0
    if causal:
        s = s.masked_fill(torch.triu(torch.ones(n, n, dtype=torch.bool), 1), float("-inf"))
    assert np.max(np.abs(lse - torch.logsumexp(s, dim=1).numpy())) < 1e-12


@pytest.mark.parametrize("causal", [False, True])
def test_sampled_matches_dense(causal):
    q, k, v, do = _rand(300, 64, 41)
    o, lse = exact.fwd(q, k, v, causal)
    g = exact.bwd(q, k, v, do, causal)
    qr = np.array([0, 5, 299, 150])
    kr = np.array([1, 2, 250, 299])
    os_, ls, dq, dk, dv = exact.sampled(q, k, v, do, causal, qr, kr, chunk=64)
    assert np.max(np.abs(os_ - o[qr])) < 1e-13
    assert np.max(np.abs(ls - lse[qr])) < 1e-13
    assert np.max(np.abs(dq - g[0][qr])) < 1e-13
    assert np.max(np.abs(dk - g[1][kr])) < 1e-13
    assert np.max(np.abs(dv - g[2][kr])) < 1e-13


@pytest.mark.parametrize("causal", [False, True])
def test_qk_norm_matches_torch_autograd(causal):
    """QK-norm forward and its gradient against torch autograd of the same
    composition written directly (row RMS norm, eps 1e-6, then attention)."""
    n, d = 40, 64
    q, k, v, do = _rand(n, d, 23)
    q = q * np.linspace(0.2, 4.0, n)[:, None]
    o, _ = exact.fwd(q, k, v, causal, qk_norm=True)
    dq, dk, dv = exact.bwd(q, k, v, do, causal, qk_norm=True)
    tq, tk, tv = (torch.tensor(x, dtype=torch.float64, requires_grad=True) for x in (q, k, v))
    nq = tq / torch.sqrt((tq * tq).mean(dim=1, keepdim=True) + 1e-6)
    nk = tk / torch.sqrt((tk * tk).mean(dim=1, keepdim=True) + 1e-6)
    to = torch.nn.functional.scaled_dot_product_attention(nq[None, None], nk[None, None], tv[None, None],
                                                          is_causal=causal)[0, 0]
    to.backward(torch.tensor(do))
    assert np.max(np.abs(o - to.detach().numpy())) < 1e-12
    for a, t in ((dq, tq), (dk, tk), (dv, tv)):
        assert np.max(np.abs(a - t.grad.numpy())) < 1e-11


def test_qk_norm_radial_gradient_and_scale_invariance():
    """Scaling a row of Q or K leaves the normalized row unchanged (up to the
    1e-6 epsilon), so O barely moves and the gradient has no component along
    the row itself: |sum_c dQ_ic Q_ic| is at the epsilon level."""
    n, d = 30, 64
    q, k, v, do = _rand(n, d, 24)
    o1, _ = exact.fwd(q, k, v, True, qk_norm=True)
    c = np.linspace(0.5, 5.0, n)[:, None]
    o2, _ = exact.fwd(q * c, k / c, v, True, qk_norm=True)
    assert np.max(np.abs(o1 - o2)) < 1e-5
    dq, dk, _ = exact.bwd(q, k, v, do, True, qk_norm=True)
    for g, x in ((dq, q), (dk, k)):
        radial = np.abs(np.sum(g * x, axis=1))
        assert np.all(radial <= 1e-5 * np.linalg.norm(g, axis=1) * np.linalg.norm(x, axis=1) + 1e-15)


@pytest.mark.parametrize("causal", [False, True])
def test_sampled_matches_dense_qk_norm(causal):
    q, k, v, do = _rand(300, 64, 42)
    q = q * np.linspace(0.5, 2.0, 300)[:, None]
    o, lse = exact.fwd(q, k, v, causal, qk_norm=True)
    g = exact.bwd(q, k, v, do, causal, qk_norm=True)
    qr = np.array([0, 5, 299, 150])
    kr = np.array([1, 2, 250, 299])
    os_, ls, dq, dk, dv = exact.sampled(q, k, v, do, causal, qr, kr, chunk=64, qk_norm=True)
    assert np.max(np.abs(os_ - o[qr])) < 1e-13
    assert np.max(np.abs(ls - lse[qr])) < 1e-13
    assert np.max(np.abs(dq - g[0][qr])) < 1e-13
    assert np.max(np.abs(dk - g[1][kr])) < 1e-13
    assert np.max(np.abs(dv - g[2][kr])) < 1e-13


def test_worst_row_and_tile_metrics():
    """The local error metrics the GPU parity tests use next to rel-L2: one
    wrong row among many is invisible in a whole-tensor rel-L2 below 1e-2 but
    shows as a relative error of 1 in its row and at least 1/8 in its tile;
    rows that are zero in the reference are measured against the floor."""
    r = np.random.default_rng(5)
    ref = r.standard_normal((2, 3, 16384, 64))
    x = ref * (1 + 1e-3 * r.standard_normal(ref.shape))
    assert M.rel_l2(x, ref) < 2e-3 and M.worst_row_rel(x, ref) < 1e-2 and M.worst_tile_rel(x, ref) < 4e-3
    bad = x.copy()
    bad[1, 2, 777] = 0.0                              # one dropped row
    assert M.rel_l2(bad, ref) < 1e-2
    assert M.worst_row_rel(bad, ref) > 0.9 and M.worst_tile_rel(bad, ref) > 0.12
    z = ref.copy()
    z[0, 0, 5] = 0.0
    xz = z.copy()
    xz[0, 0, 5, 0] = 1e-3                            # residue on a zero reference row
    assert M.worst_row_rel(xz, z) < 1e-2
    # ragged tiles: the last tile of 48 rows is its own tile
    a = r.standard_normal((112, 64))
    b = a.copy()
    b[100:] += 1.0
    assert M.worst_tile_rel(b, a) > 0.45 and M.worst_tile_rel(b[:64], a[:64]) == 0.0
