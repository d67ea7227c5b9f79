"""The float64 oracle against closed forms, brute force, hand-derived examples,
an independent chunked algorithm and invariants (see ``oracle_pins.py``)."""
import pytest

import oracle
import oracle_pins


@pytest.fixture(scope="module")
def orc():
    oracle.build(force=False)
    return oracle._load()


@pytest.mark.parametrize("check", oracle_pins.ALL_CHECKS, ids=lambda f: f.__name__)
def test_pin(orc, check):
    check(orc)


def test_step_wrappers_match_the_definition():
    """oracle.scan_step / ssd_step take one token's slices; chained over L
    tokens they equal oracle.scan / ssd over L steps from the same state."""
    import numpy as np
    rng = np.random.default_rng(5)
    b, d, n, L = 2, 3, 4, 6
    u, z = rng.standard_normal((b, d, L)), rng.standard_normal((b, d, L))
    dl = np.exp(rng.uniform(-4, -1, (b, d, L)))
    A = -np.exp(rng.uniform(0, 1, (d, n)))
    B, C = rng.standard_normal((b, 2, n, L)), rng.standard_normal((b, 2, n, L))
    h0 = rng.standard_normal((b, d * 2 // 2, n))
    D = rng.standard_normal(d)
    A2 = np.concatenate([A, A]); D2 = np.concatenate([D, D])
    u2, z2, dl2 = (np.concatenate([a, a], axis=1) for a in (u, z, dl))
    h02 = np.concatenate([h0, h0], axis=1)
    y, h = oracle.scan(u2, dl2, A2, B, C, D2, z2, h02)
    st, ys = h02, []
    for t in range(L):
        yt, st = oracle.scan_step(u2[..., t], dl2[..., t], A2, B[..., t], C[..., t], D2, z2[..., t], st)
        ys.append(yt)
    assert np.array_equal(np.stack(ys, axis=-1), y) and np.array_equal(st, h)
    H, P, N = 2, 3, 4
    x, dt = rng.standard_normal((b, L, H, P)), np.exp(rng.uniform(-3, -1, (b, L, H)))
    Bs, Cs = rng.standard_normal((b, L, 1, N)), rng.standard_normal((b, L, 1, N))
    Ah, S0 = -np.exp(rng.uniform(0, 1, H)), rng.standard_normal((b, H, P, N))
    y, h = oracle.ssd(x, dt, Ah, Bs, Cs, None, None, S0)
    st, ys = S0, []
    for t in range(L):
        yt, st = oracle.ssd_step(x[:, t], dt[:, t], Ah, Bs[:, t], Cs[:, t], None, None, st)
        ys.append(yt)
    assert np.array_equal(np.stack(ys, axis=1), y) and np.array_equal(st, h)


def test_phase0_wrappers_chain_rule():
    """oracle.scan / scan_bwd with dt_softplus take raw delta: the gradient they
    return for it, and its sum over batch and steps for dt_bias, against
    central finite differences of the forward on raw delta and on dt_bias;
    oracle.ssd_trap with lam_sigmoid equals the plain call on expit(lam)."""
    import numpy as np
    from scipy.special import expit
    rng = np.random.default_rng(73)
    b, d, n, L = 2, 3, 4, 5
    u, z = rng.standard_normal((b, d, L)), rng.standard_normal((b, d, L))
    raw, bias = rng.uniform(-4, 1, (b, d, L)), rng.uniform(-1, 1, d)
    A = -np.exp(rng.uniform(-1, 1, (d, n)))
    B, C = rng.standard_normal((b, 1, n, L)), rng.standard_normal((b, 1, n, L))
    D, h0 = rng.standard_normal(d), rng.standard_normal((b, d, n))
    dy, dhl = rng.standard_normal((b, d, L)), rng.standard_normal((b, d, n))

    def loss(r, bb):
        y, h = oracle.scan(u, r, A, B, C, D, z, h0, dt_softplus=True, dt_bias=bb)
        return float(np.sum(dy * y) + np.sum(dhl * h))

    g = oracle.scan_bwd(u, raw, A, B, C, D, z, h0, dy, dhl, dt_softplus=True, dt_bias=bias)
    e = 1e-6
    fd = np.zeros_like(raw)
    for idx in np.ndindex(raw.shape):
        hi, lo = raw.copy(), raw.copy()
        hi[idx] += e
        lo[idx] -= e
        fd[idx] = (loss(hi, bias) - loss(lo, bias)) / (2 * e)
    assert np.max(np.abs(g["ddelta"] - fd)) <= 1e-7 * max(1.0, np.max(np.abs(fd)))
    fdb = np.zeros_like(bias)
    for k in range(d):
        hi, lo = bias.copy(), bias.copy()
        hi[k] += e
        lo[k] -= e
        fdb[k] = (loss(raw, hi) - loss(raw, lo)) / (2 * e)
    assert np.max(np.abs(g["ddelta"].sum(axis=(0, 2)) - fdb)) <= 1e-7 * max(1.0, np.max(np.abs(fdb)))
    H, P, N = 2, 3, 4
    x, dtr = rng.standard_normal((b, L, H, P)), rng.uniform(-4, 1, (b, L, H))
    lamr, hb = rng.standard_normal((b, L, H)), rng.uniform(-1, 1, H)
    Ah = -np.exp(rng.uniform(0, 1, H))
    Bs, Cs = rng.standard_normal((b, L, 1, N)), rng.standard_normal((b, L, 1, N))
    y1, h1 = oracle.ssd_trap(x, dtr, lamr, Ah, Bs, Cs, dt_softplus=True, dt_bias=hb, lam_sigmoid=True)
    y2, h2 = oracle.ssd_trap(x, np.logaddexp(0.0, dtr + hb), expit(lamr), Ah, Bs, Cs)
    assert np.allclose(y1, y2, rtol=1e-13, atol=1e-13) and np.allclose(h1, h2, rtol=1e-13, atol=1e-13)
