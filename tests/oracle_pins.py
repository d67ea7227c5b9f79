"""Pins for the float64 CPU oracle.

Each ``check_*`` function takes an ``Oracle``-like object (``.scan`` and
``.ssd``) and raises ``AssertionError`` if the oracle disagrees with something
fixed independently of it: a closed form, a brute-force materialised sum, a
hand-derived worked example, a different algorithm for the same quantity, or an
invariant of the recurrence.  ``test_oracle_pins.py`` runs them on the oracle;
``test_oracle_mutants.py`` runs them on copies of the oracle with planted
mistakes and requires every mistake to be caught.

Definitions followed (page titles and sections):
  * "We brought Mamba to Trainium", section "Mamba: bringing an unsupported
    model to the chip": h_t = Abar_t h_{t-1} + Bbar_t x_t, y_t = sum_n C_t h_t.
  * "Mamba-3 NKI Kernels for AWS Neuron", section "How it works": Phase 0
    alpha = exp(dt*A) and input weight dt (lam = 1); Phase 5 D skip then silu
    gate.  Section "Kernel details" (mamba3_siso_ssd_kernel): chunked SSD with
    the Mamba-2 structure; section "Repository layout": segsum and causal masks.
  * "We brought Mamba to Trainium", section "We built the parallel scan": the
    recurrence is associative, so it can be split and recombined.
  * "Mamba-3 NKI Kernels for AWS Neuron", section "How it works", Phase 0: the
    raw step goes through softplus(dt + dt_bias), the raw trapezoid weight
    through a sigmoid.
  * same page and section, Phase 1: the angles are the negated running sum of
    dt * theta and rotate B and C (the complex-valued state of its Mamba-3
    feature list).
"""
from __future__ import annotations

import json
import math
import os

import numpy as np

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")
RTOL = 1e-12


def _close(got, want, rtol=RTOL, what=""):
    got = np.asarray(got, dtype=np.float64)
    want = np.asarray(want, dtype=np.float64)
    assert got.shape == want.shape, f"{what}: shape {got.shape} != {want.shape}"
    scale = max(1.0, float(np.max(np.abs(want))) if want.size else 1.0)
    err = float(np.max(np.abs(got - want))) if want.size else 0.0
    assert err <= rtol * scale, f"{what}: max abs err {err:.3e} (scale {scale:.3e})"


def _silu(z):
    return z / (1.0 + np.exp(-z))


def _rand_scan(rng, batch, dim, N, L, G, a_scale=1.0):
    u = rng.standard_normal((batch, dim, L))
    delta = np.exp(rng.uniform(math.log(1e-2), math.log(0.5), (batch, dim, L)))
    A = -a_scale * np.exp(rng.uniform(math.log(0.3), math.log(3.0), (dim, N)))
    B = rng.standard_normal((batch, G, N, L))
    C = rng.standard_normal((batch, G, N, L))
    D = rng.standard_normal(dim)
    z = rng.standard_normal((batch, dim, L))
    return u, delta, A, B, C, D, z


def _rand_ssd(rng, batch, L, H, P, N, G):
    x = rng.standard_normal((batch, L, H, P))
    dt = np.exp(rng.uniform(math.log(1e-2), math.log(0.5), (batch, L, H)))
    A = -np.exp(rng.uniform(0.0, math.log(8.0), H))
    B = rng.standard_normal((batch, L, G, N))
    C = rng.standard_normal((batch, L, G, N))
    D = rng.standard_normal(H)
    z = rng.standard_normal((batch, L, H, P))
    return x, dt, A, B, C, D, z


# --------------------------------------------------------------------------
# Selective scan
# --------------------------------------------------------------------------

def check_scan_hand_example(orc):
    """Hand-derived worked example (tests/golden/scan_hand_example.json)."""
    g = json.load(open(os.path.join(GOLDEN, "scan_hand_example.json")))
    i, e = g["inputs"], g["expected"]
    arr = {k: np.array(v, dtype=np.float64) for k, v in i.items() if not k.endswith("exact")}
    y, h = orc.scan(arr["u"], arr["delta"], arr["A"], arr["B"], arr["C"], arr["D"])
    _close(y, e["y"], what="hand y")
    _close(h, e["h_last"], what="hand h_last")
    yg, hg = orc.scan(arr["u"], arr["delta"], arr["A"], arr["B"], arr["C"], arr["D"],
                      arr["z_gated_case"])
    _close(yg, e["y_gated"], what="hand gated y")
    _close(hg, e["h_last"], what="hand gated h_last (the gate does not touch the state)")


def check_scan_a_zero_prefix_sum(orc):
    """A = 0: no decay, so the state is a running (prefix) sum of dt*B*x."""
    rng = np.random.default_rng(11)
    batch, dim, N, L, G = 2, 4, 5, 37, 2
    u, delta, _, B, C, D, z = _rand_scan(rng, batch, dim, N, L, G)
    A = np.zeros((dim, N))
    y, h = orc.scan(u, delta, A, B, C, D, z)
    g_of_d = np.arange(dim) // (dim // G)
    Bd = B[:, g_of_d]                      # (batch, dim, N, L)
    Cd = C[:, g_of_d]
    contrib = delta[:, :, None, :] * Bd * u[:, :, None, :]
    hs = np.cumsum(contrib, axis=-1)       # (batch, dim, N, L)
    want = (np.sum(Cd * hs, axis=2) + D[None, :, None] * u) * _silu(z)
    _close(y, want, what="A=0 y")
    _close(h, hs[..., -1], what="A=0 h_last")


def check_scan_constant_coeff_geometric(orc):
    """Constant dt, x, B, C: geometric series h_t = dt B x (1 - r^(t+1)) / (1 - r)."""
    dim, N, L = 3, 4, 50
    dl, xi = 0.07, 1.3
    A = np.array([[-0.5, -1.0, -2.0, -4.0],
                  [-0.1, -0.2, -3.0, -0.7],
                  [-1.5, -0.05, -0.9, -6.0]])
    beta = np.array([0.9, -0.4, 1.7, 0.3])
    gam = np.array([1.1, 0.6, -0.8, 2.0])
    Dk = np.array([0.3, -1.2, 0.0])
    u = np.full((1, dim, L), xi)
    delta = np.full((1, dim, L), dl)
    B = np.broadcast_to(beta[None, None, :, None], (1, 1, N, L)).copy()
    C = np.broadcast_to(gam[None, None, :, None], (1, 1, N, L)).copy()
    y, h = orc.scan(u, delta, A, B, C, Dk)
    t = np.arange(L)
    r = np.exp(dl * A)                                     # (dim, N)
    geo = (1.0 - r[:, :, None] ** (t + 1)) / (1.0 - r[:, :, None])
    hs = dl * beta[None, :, None] * xi * geo               # (dim, N, L)
    want = np.einsum("n,dnt->dt", gam, hs) + Dk[:, None] * xi
    _close(y[0], want, what="geometric y")
    _close(h[0], hs[..., -1], what="geometric h_last")


def check_scan_l1(orc):
    """L = 1 from a zero state: y0 = dt0 x0 sum_n C0 B0 + D x0, h = dt0 B0 x0."""
    rng = np.random.default_rng(12)
    batch, dim, N, G = 3, 4, 6, 1
    u, delta, A, B, C, D, z = _rand_scan(rng, batch, dim, N, 1, G)
    y, h = orc.scan(u, delta, A, B, C, D, z)
    cb = np.sum(C[:, 0, :, 0] * B[:, 0, :, 0], axis=1)   # (batch,)
    want = (delta[..., 0] * u[..., 0] * cb[:, None] + D[None, :] * u[..., 0]) * _silu(z[..., 0])
    _close(y[..., 0], want, what="L=1 y")
    _close(h, delta[..., 0, None] * B[:, 0, None, :, 0] * u[..., 0, None], what="L=1 h_last")


def check_scan_bruteforce(orc):
    """Materialised quadratic form on tiny inputs, pure Python loops:
    y_t = sum_{s<=t} sum_n C_t[n] (prod_{k=s+1..t} exp(dt_k A[n])) dt_s B_s[n] x_s + D x_t,
    then the gate; h_last[n] is the same sum at t = L-1 without C."""
    rng = np.random.default_rng(13)
    for (batch, dim, N, L, G) in [(2, 3, 4, 9, 1), (1, 2, 3, 13, 2), (1, 1, 2, 24, 1)]:
        u, delta, A, B, C, D, z = _rand_scan(rng, batch, dim, N, L, G)
        y, h = orc.scan(u, delta, A, B, C, D, z)
        dpg = dim // G
        want_y = np.zeros((batch, dim, L))
        want_h = np.zeros((batch, dim, N))
        for b in range(batch):
            for d in range(dim):
                g = d // dpg
                for t in range(L):
                    acc = 0.0
                    for s in range(t + 1):
                        for n in range(N):
                            prod = 1.0
                            for k in range(s + 1, t + 1):
                                prod *= math.exp(delta[b, d, k] * A[d, n])
                            acc += C[b, g, n, t] * prod * delta[b, d, s] * B[b, g, n, s] * u[b, d, s]
                    acc += D[d] * u[b, d, t]
                    want_y[b, d, t] = acc * z[b, d, t] / (1.0 + math.exp(-z[b, d, t]))
                for n in range(N):
                    acc = 0.0
                    for s in range(L):
                        prod = 1.0
                        for k in range(s + 1, L):
                            prod *= math.exp(delta[b, d, k] * A[d, n])
                        acc += prod * delta[b, d, s] * B[b, g, n, s] * u[b, d, s]
                    want_h[b, d, n] = acc
        _close(y, want_y, rtol=1e-11, what=f"brute y {(batch, dim, N, L, G)}")
        _close(h, want_h, rtol=1e-11, what=f"brute h {(batch, dim, N, L, G)}")


def check_scan_invariants(orc):
    """Causality, linearity in x (no gate) and split continuation through h0."""
    rng = np.random.default_rng(14)
    batch, dim, N, L, G = 2, 3, 5, 41, 1
    u, delta, A, B, C, D, z = _rand_scan(rng, batch, dim, N, L, G)
    y, h = orc.scan(u, delta, A, B, C, D, z)
    # causality: changing x at t0 leaves y_{<t0} unchanged and changes y_{t0}
    t0 = 17
    u2 = u.copy()
    u2[:, :, t0] += 1.0
    y2, _ = orc.scan(u2, delta, A, B, C, D, z)
    assert np.array_equal(y2[..., :t0], y[..., :t0]), "causality"
    assert np.all(y2[..., t0] != y[..., t0]), "x_t0 must reach y_t0"
    # linearity in x without the gate
    v = rng.standard_normal(u.shape)
    ya, ha = orc.scan(u, delta, A, B, C, D)
    yb, hb = orc.scan(v, delta, A, B, C, D)
    yc, hc = orc.scan(2.0 * u - 3.0 * v, delta, A, B, C, D)
    _close(yc, 2.0 * ya - 3.0 * yb, rtol=1e-11, what="linearity y")
    _close(hc, 2.0 * ha - 3.0 * hb, rtol=1e-11, what="linearity h")
    # split continuation: [0, L1) then [L1, L) from the first part's h_last
    for L1 in (1, 20, L - 1):
        yl, hl = orc.scan(u[..., :L1], delta[..., :L1], A, B[..., :L1], C[..., :L1], D, z[..., :L1])
        yr, hr = orc.scan(u[..., L1:], delta[..., L1:], A, B[..., L1:], C[..., L1:], D,
                          z[..., L1:], h0=hl)
        _close(np.concatenate([yl, yr], axis=-1), y, what=f"split y at {L1}")
        _close(hr, h, what=f"split h_last at {L1}")
    # the gate: z = 0 zeroes y, and never touches the state
    y0, h0 = orc.scan(u, delta, A, B, C, D, np.zeros_like(z))
    assert np.all(y0 == 0.0), "silu(0) = 0"
    _close(h0, h, rtol=0.0, what="gate leaves the state alone")


# --------------------------------------------------------------------------
# Scalar-decay SSD
# --------------------------------------------------------------------------

def check_ssd_hand_example(orc):
    """Hand-derived worked example (tests/golden/ssd_hand_example.json)."""
    g = json.load(open(os.path.join(GOLDEN, "ssd_hand_example.json")))
    i, e = g["inputs"], g["expected"]
    arr = {k: np.array(v, dtype=np.float64) for k, v in i.items() if not k.endswith("exact")}
    y, h = orc.ssd(arr["x"], arr["dt"], arr["A"], arr["B"], arr["C"], arr["D"])
    _close(y, e["y"], what="hand ssd y")
    _close(h, e["h_last"], what="hand ssd h_last")


def chunked_ssd_numpy(x, dt, A, B, C, D, z, Q):
    """The chunked (Mamba-2 structured) SSD written with matrices in float64.

    Per chunk of Q steps (the last chunk may be shorter), with a_t the inclusive
    cumulative sum of dt*A inside the chunk:
      intra-chunk  Y_diag[t] = sum_{s<=t} (C_t . B_s) exp(a_t - a_s) dt_s x_s
      state in     Y_off[t]  = exp(a_t) C_t . H_prev
      state out    H_new     = exp(a_last) H_prev + sum_s exp(a_last - a_s) dt_s x_s B_s^T
    This is a different algorithm from the step-by-step recurrence; both must
    give the same numbers.
    """
    batch, L, H, P = x.shape
    G, N = B.shape[2], B.shape[3]
    hpg = H // G
    y = np.zeros_like(x)
    hl = np.zeros((batch, H, P, N))
    for b in range(batch):
        for hd in range(H):
            g = hd // hpg
            Hs = np.zeros((P, N))
            for c0 in range(0, L, Q):
                c1 = min(L, c0 + Q)
                Xc = x[b, c0:c1, hd, :]                 # (q, P)
                dtc = dt[b, c0:c1, hd]                  # (q,)
                Bc = B[b, c0:c1, g, :]                  # (q, N)
                Cc = C[b, c0:c1, g, :]
                a = np.cumsum(dtc * A[hd])              # (q,)
                seg = a[:, None] - a[None, :]           # segsum a_t - a_s
                q = c1 - c0
                causal = np.tril(np.ones((q, q), dtype=bool))
                Lmat = np.where(causal, np.exp(np.where(causal, seg, 0.0)), 0.0)
                G_cb = Cc @ Bc.T                        # (q, q)
                Ydiag = (G_cb * Lmat * dtc[None, :]) @ Xc
                Yoff = np.exp(a)[:, None] * (Cc @ Hs.T)
                decay_end = np.exp(a[-1] - a)           # (q,)
                Hs = np.exp(a[-1]) * Hs + (Xc * (decay_end * dtc)[:, None]).T @ Bc
                yc = Ydiag + Yoff
                if D is not None:
                    yc = yc + D[hd] * Xc
                if z is not None:
                    yc = yc * _silu(z[b, c0:c1, hd, :])
                y[b, c0:c1, hd, :] = yc
            hl[b, hd] = Hs
    return y, hl


def check_ssd_chunked_equals_recurrence(orc):
    """The chunked matrix form (chunk 1, 3, 16, 64; ragged tails) equals the oracle."""
    rng = np.random.default_rng(21)
    for (batch, L, H, P, N, G) in [(2, 70, 4, 3, 5, 2), (1, 64, 2, 4, 8, 1), (1, 5, 1, 2, 3, 1)]:
        x, dt, A, B, C, D, z = _rand_ssd(rng, batch, L, H, P, N, G)
        y, h = orc.ssd(x, dt, A, B, C, D, z)
        for Q in (1, 3, 16, 64):
            yc, hc = chunked_ssd_numpy(x, dt, A, B, C, D, z, Q)
            _close(y, yc, rtol=1e-11, what=f"chunked y Q={Q} {(batch, L, H, P, N, G)}")
            _close(h, hc, rtol=1e-11, what=f"chunked h Q={Q} {(batch, L, H, P, N, G)}")


def check_ssd_equals_scan_broadcast(orc):
    """SSD is the selective scan with A[d=(h,p), n] = A_h and dt broadcast over p."""
    rng = np.random.default_rng(22)
    batch, L, H, P, N, G = 2, 29, 4, 3, 5, 2
    x, dt, A, B, C, D, z = _rand_ssd(rng, batch, L, H, P, N, G)
    y, h = orc.ssd(x, dt, A, B, C, D, z)
    dim = H * P
    u = x.reshape(batch, L, dim).transpose(0, 2, 1).copy()
    delta = np.repeat(dt, P, axis=2).transpose(0, 2, 1).copy()
    Asc = np.repeat(A, P)[:, None] * np.ones((1, N))
    Bsc = B.transpose(0, 2, 3, 1).copy()
    Csc = C.transpose(0, 2, 3, 1).copy()
    zsc = z.reshape(batch, L, dim).transpose(0, 2, 1).copy()
    ys, hs = orc.scan(u, delta, Asc, Bsc, Csc, np.repeat(D, P), zsc)
    _close(y, ys.transpose(0, 2, 1).reshape(batch, L, H, P), what="ssd vs scan y")
    _close(h, hs.reshape(batch, H, P, N), what="ssd vs scan h")


def check_ssd_invariants(orc):
    """Split continuation through h0, causality, and the zero-dt identity."""
    rng = np.random.default_rng(23)
    batch, L, H, P, N, G = 2, 33, 2, 3, 4, 1
    x, dt, A, B, C, D, z = _rand_ssd(rng, batch, L, H, P, N, G)
    y, h = orc.ssd(x, dt, A, B, C, D, z)
    for L1 in (1, 16, 32):
        yl, hl = orc.ssd(x[:, :L1], dt[:, :L1], A, B[:, :L1], C[:, :L1], D, z[:, :L1])
        yr, hr = orc.ssd(x[:, L1:], dt[:, L1:], A, B[:, L1:], C[:, L1:], D, z[:, L1:], h0=hl)
        _close(np.concatenate([yl, yr], axis=1), y, what=f"ssd split y at {L1}")
        _close(hr, h, what=f"ssd split h at {L1}")
    x2 = x.copy()
    x2[:, 10] += 1.0
    y2, _ = orc.ssd(x2, dt, A, B, C, D, z)
    assert np.array_equal(y2[:, :10], y[:, :10]), "ssd causality"
    # dt = 0 everywhere: no decay and no input, so the state stays h0 and y = C.h0 + D x
    h0 = rng.standard_normal((batch, H, P, N))
    y3, h3 = orc.ssd(x, np.zeros_like(dt), A, B, C, D, None, h0=h0)
    want = np.einsum("blgn,bhpn->blhp", C[:, :, [0]], h0) + D[None, None, :, None] * x
    _close(y3, want, what="dt=0 y")
    _close(h3, h0, rtol=0.0, what="dt=0 h")


def check_decode_steps_chain(orc):
    """A decode step is the recurrence at one token from a cached state: L
    steps chained through the state reproduce one run over L steps exactly
    (same float64 operations in the same order), for the scan and the SSD."""
    rng = np.random.default_rng(77)
    b, d, n, L = 2, 5, 4, 9
    u = rng.standard_normal((b, d, L))
    dl = np.exp(rng.uniform(-5, -1, (b, d, L)))
    A = -np.exp(rng.uniform(0, 1.5, (d, n)))
    B = rng.standard_normal((b, 1, n, L))
    C = rng.standard_normal((b, 1, n, L))
    D = rng.standard_normal(d)
    z = rng.standard_normal((b, d, L))
    h0 = rng.standard_normal((b, d, n))
    y, h = orc.scan(u, dl, A, B, C, D, z, h0)
    st, ys = h0, []
    for t in range(L):
        yt, st = orc.scan(u[..., t:t + 1], dl[..., t:t + 1], A, B[..., t:t + 1], C[..., t:t + 1], D,
                          z[..., t:t + 1], st)
        ys.append(yt)
    _close(np.concatenate(ys, axis=-1), y, rtol=0.0, what="scan steps chained")
    _close(st, h, rtol=0.0, what="scan state after chained steps")
    H, P, N = 3, 4, 8
    x = rng.standard_normal((b, L, H, P))
    dt = np.exp(rng.uniform(-4, -1, (b, L, H)))
    Ah = -np.exp(rng.uniform(0, 2, H))
    Bs = rng.standard_normal((b, L, 1, N))
    Cs = rng.standard_normal((b, L, 1, N))
    Dh = rng.standard_normal(H)
    S0 = rng.standard_normal((b, H, P, N))
    y, h = orc.ssd(x, dt, Ah, Bs, Cs, Dh, None, S0)
    st, ys = S0, []
    for t in range(L):
        yt, st = orc.ssd(x[:, t:t + 1], dt[:, t:t + 1], Ah, Bs[:, t:t + 1], Cs[:, t:t + 1], Dh, None, st)
        ys.append(yt)
    _close(np.concatenate(ys, axis=1), y, rtol=0.0, what="ssd steps chained")
    _close(st, h, rtol=0.0, what="ssd state after chained steps")


def check_scan_bwd_finite_differences(orc):
    """The backward against central finite differences of the forward, on tiny
    problems with every optional input present: the gradient of
    L = sum(dy * y) + sum(dh_last * h_last) with respect to each element of
    u, delta, A, B, C, D, z and h0 (two group counts)."""
    names = {"u": "du", "delta": "ddelta", "A": "dA", "B": "dB", "C": "dC", "D": "dD", "z": "dz",
             "h0": "dh0"}
    for seed, (b, d, n, L, G) in ((11, (2, 3, 4, 6, 1)), (12, (1, 4, 2, 5, 2))):
        rng = np.random.default_rng(seed)
        inp = {"u": rng.standard_normal((b, d, L)), "delta": np.exp(rng.uniform(-3, 0, (b, d, L))),
               "A": -np.exp(rng.uniform(-1, 1, (d, n))), "B": rng.standard_normal((b, G, n, L)),
               "C": rng.standard_normal((b, G, n, L)), "D": rng.standard_normal(d),
               "z": rng.standard_normal((b, d, L)), "h0": rng.standard_normal((b, d, n))}
        dy, dhl = rng.standard_normal((b, d, L)), rng.standard_normal((b, d, n))

        def loss(v):
            y, h = orc.scan(v["u"], v["delta"], v["A"], v["B"], v["C"], v["D"], v["z"], v["h0"])
            return float(np.sum(dy * y) + np.sum(dhl * h))

        g = orc.scan_bwd(inp["u"], inp["delta"], inp["A"], inp["B"], inp["C"], inp["D"], inp["z"],
                         inp["h0"], dy, dhl)
        for k, gk in names.items():
            fd = np.zeros_like(inp[k])
            for idx in np.ndindex(inp[k].shape):
                e = 1e-6 * max(1.0, abs(inp[k][idx]))
                lo, hi = dict(inp), dict(inp)
                lo[k], hi[k] = inp[k].copy(), inp[k].copy()
                lo[k][idx] -= e
                hi[k][idx] += e
                fd[idx] = (loss(hi) - loss(lo)) / (2 * e)
            _close(g[gk], fd, rtol=1e-7, what=f"d{k} against finite differences (seed {seed})")


def check_ssd_bwd_finite_differences(orc):
    """The SSD backward against central finite differences of the SSD forward,
    with every optional input present (two group counts): the gradient of
    L = sum(dy * y) + sum(dh_last * h_last) with respect to each element of
    x, dt, A, B, C, D, z and h0."""
    names = {"x": "dx", "dt": "ddt", "A": "dA", "B": "dB", "C": "dC", "D": "dD", "z": "dz", "h0": "dh0"}
    for seed, (b, L, H, P, N, G) in ((13, (2, 5, 2, 3, 4, 1)), (14, (1, 4, 4, 2, 3, 2))):
        rng = np.random.default_rng(seed)
        inp = {"x": rng.standard_normal((b, L, H, P)), "dt": np.exp(rng.uniform(-3, 0, (b, L, H))),
               "A": -np.exp(rng.uniform(-1, 1, H)), "B": rng.standard_normal((b, L, G, N)),
               "C": rng.standard_normal((b, L, G, N)), "D": rng.standard_normal(H),
               "z": rng.standard_normal((b, L, H, P)), "h0": rng.standard_normal((b, H, P, N))}
        dy, dhl = rng.standard_normal((b, L, H, P)), rng.standard_normal((b, H, P, N))

        def loss(v):
            y, h = orc.ssd(v["x"], v["dt"], v["A"], v["B"], v["C"], v["D"], v["z"], v["h0"])
            return float(np.sum(dy * y) + np.sum(dhl * h))

        g = orc.ssd_bwd(inp["x"], inp["dt"], inp["A"], inp["B"], inp["C"], inp["D"], inp["z"], inp["h0"],
                        dy, dhl)
        for k, gk in names.items():
            fd = np.zeros_like(inp[k])
            for idx in np.ndindex(inp[k].shape):
                e = 1e-6 * max(1.0, abs(inp[k][idx]))
                lo, hi = dict(inp), dict(inp)
                lo[k], hi[k] = inp[k].copy(), inp[k].copy()
                lo[k][idx] -= e
                hi[k][idx] += e
                fd[idx] = (loss(hi) - loss(lo)) / (2 * e)
            _close(g[gk], fd, rtol=1e-7, what=f"ssd d{k} against finite differences (seed {seed})")


def check_ssd_bwd_equals_scan_bwd_broadcast(orc):
    """The SSD backward is the selective-scan backward with A[d=(h,p), n] = A_h
    and dt broadcast over p: dx, dz, dB, dC, dh0 equal the scan's, and dA, dD,
    ddt are the scan's summed over the head's p (and n for dA)."""
    rng = np.random.default_rng(23)
    batch, L, H, P, N, G = 2, 9, 4, 3, 5, 2
    x, dt, A, B, C, D, z = _rand_ssd(rng, batch, L, H, P, N, G)
    h0 = rng.standard_normal((batch, H, P, N))
    dy, dhl = rng.standard_normal((batch, L, H, P)), rng.standard_normal((batch, H, P, N))
    g = orc.ssd_bwd(x, dt, A, B, C, D, z, h0, dy, dhl)
    dim = H * P
    tr = lambda a: a.reshape(batch, L, dim).transpose(0, 2, 1).copy()
    gs = orc.scan_bwd(tr(x), np.repeat(dt, P, axis=2).transpose(0, 2, 1).copy(),
                      np.repeat(A, P)[:, None] * np.ones((1, N)), B.transpose(0, 2, 3, 1).copy(),
                      C.transpose(0, 2, 3, 1).copy(), np.repeat(D, P), tr(z), h0.reshape(batch, dim, N),
                      tr(dy), dhl.reshape(batch, dim, N))
    back = lambda a: a.transpose(0, 2, 1).reshape(batch, L, H, P)
    _close(g["dx"], back(gs["du"]), what="ssd dx vs scan du")
    _close(g["dz"], back(gs["dz"]), what="ssd dz vs scan dz")
    _close(g["dB"], gs["dB"].transpose(0, 3, 1, 2), what="ssd dB vs scan dB")
    _close(g["dC"], gs["dC"].transpose(0, 3, 1, 2), what="ssd dC vs scan dC")
    _close(g["dh0"], gs["dh0"].reshape(batch, H, P, N), what="ssd dh0 vs scan dh0")
    _close(g["dA"], gs["dA"].reshape(H, P, N).sum(axis=(1, 2)), what="ssd dA vs scan dA summed")
    _close(g["dD"], gs["dD"].reshape(H, P).sum(axis=1), what="ssd dD vs scan dD summed")
    _close(g["ddt"], gs["ddelta"].reshape(batch, H, P, L).sum(axis=2).transpose(0, 2, 1),
           what="ssd ddt vs scan ddelta summed")


def _trap_inputs(rng, b, L, H, P, N, G):
    return {"x": rng.standard_normal((b, L, H, P)), "dt": np.exp(rng.uniform(-3, 0, (b, L, H))),
            "lam": rng.uniform(0, 1, (b, L, H)), "A": -np.exp(rng.uniform(-1, 1, H)),
            "B": rng.standard_normal((b, L, G, N)), "C": rng.standard_normal((b, L, G, N)),
            "D": rng.standard_normal(H), "z": rng.standard_normal((b, L, H, P)),
            "h0": rng.standard_normal((b, H, P, N))}


def check_ssd_trap_bwd_finite_differences(orc):
    """The trapezoidal SSD backward against central finite differences of the
    trapezoidal forward, every optional input present, the token before the
    sequence given (two group counts): the gradient of L = sum(dy * y) +
    sum(dh_last * h_last) with respect to each element of x, dt, lam, A, B, C,
    D, z, h0, x_prev and B_prev."""
    names = {"x": "dx", "dt": "ddt", "lam": "dlam", "A": "dA", "B": "dB", "C": "dC", "D": "dD", "z": "dz",
             "h0": "dh0", "x_prev": "dx_prev", "B_prev": "dB_prev"}
    for seed, (b, L, H, P, N, G) in ((71, (2, 5, 2, 3, 4, 1)), (72, (1, 4, 4, 2, 3, 2))):
        rng = np.random.default_rng(seed)
        inp = _trap_inputs(rng, b, L, H, P, N, G)
        inp["x_prev"], inp["B_prev"] = rng.standard_normal((b, H, P)), rng.standard_normal((b, G, N))
        dy, dhl = rng.standard_normal((b, L, H, P)), rng.standard_normal((b, H, P, N))

        def loss(v):
            y, h = orc.ssd_trap(v["x"], v["dt"], v["lam"], v["A"], v["B"], v["C"], v["D"], v["z"], v["h0"],
                                v["x_prev"], v["B_prev"])
            return float(np.sum(dy * y) + np.sum(dhl * h))

        g = orc.ssd_trap_bwd(inp["x"], inp["dt"], inp["lam"], inp["A"], inp["B"], inp["C"], inp["D"], inp["z"],
                             inp["h0"], inp["x_prev"], inp["B_prev"], dy, dhl)
        for k, gk in names.items():
            fd = np.zeros_like(inp[k])
            for idx in np.ndindex(inp[k].shape):
                e = 1e-6 * max(1.0, abs(inp[k][idx]))
                lo, hi = dict(inp), dict(inp)
                lo[k], hi[k] = inp[k].copy(), inp[k].copy()
                lo[k][idx] -= e
                hi[k][idx] += e
                fd[idx] = (loss(hi) - loss(lo)) / (2 * e)
            _close(g[gk], fd, rtol=1e-7, what=f"trapezoidal d{k} against finite differences (seed {seed})")


def check_ssd_trap_bwd_lam_one_is_ssd_bwd(orc):
    """lam = 1 and no previous token: the trapezoid is the plain SSD, so every
    gradient but dlam equals the SSD backward's."""
    rng = np.random.default_rng(73)
    v = _trap_inputs(rng, 2, 9, 3, 4, 5, 1)
    one = np.ones_like(v["lam"])
    dy, dhl = rng.standard_normal(v["x"].shape), rng.standard_normal(v["h0"].shape)
    g = orc.ssd_trap_bwd(v["x"], v["dt"], one, v["A"], v["B"], v["C"], v["D"], v["z"], v["h0"], None, None,
                         dy, dhl)
    r = orc.ssd_bwd(v["x"], v["dt"], v["A"], v["B"], v["C"], v["D"], v["z"], v["h0"], dy, dhl)
    for k in ("dx", "ddt", "dA", "dB", "dC", "dD", "dz", "dh0"):
        _close(g[k], r[k], rtol=1e-12, what=f"trapezoidal {k} at lam = 1 vs SSD backward")


def check_ssd_trap_lam_one_is_ssd(orc):
    """lam = 1: gamma = dt and beta = 0, so the three-term recurrence is the
    plain scalar-decay SSD (equal up to the order of one product's rounding)."""
    rng = np.random.default_rng(61)
    v = _trap_inputs(rng, 2, 9, 3, 4, 5, 1)
    one = np.ones_like(v["lam"])
    y, h = orc.ssd_trap(v["x"], v["dt"], one, v["A"], v["B"], v["C"], v["D"], v["z"], v["h0"])
    yr, hr = orc.ssd(v["x"], v["dt"], v["A"], v["B"], v["C"], v["D"], v["z"], v["h0"])
    _close(y, yr, rtol=1e-13, what="trapezoidal at lam = 1 vs SSD")
    _close(h, hr, rtol=1e-13, what="trapezoidal h_last at lam = 1 vs SSD")


def check_ssd_trap_single_ssd_form(orc):
    """Against the single-SSD form written out independently: the input of
    step s reaches step t > s with weight scale_s = gamma_s + dt_{s+1} (1 -
    lam_{s+1}) times the decay exp(sum_{k=s+1..t} dt_k A), and its own step
    with gamma_t (the diagonal correction); h0 decays from before step 0."""
    rng = np.random.default_rng(62)
    b, L, H, P, N, G = 2, 11, 4, 3, 5, 2
    v = _trap_inputs(rng, b, L, H, P, N, G)
    y, h = orc.ssd_trap(v["x"], v["dt"], v["lam"], v["A"], v["B"], v["C"], v["D"], v["z"], v["h0"])
    hpg = H // G
    for bb in range(b):
        for hd in range(H):
            g = hd // hpg
            dt, lam = v["dt"][bb, :, hd], v["lam"][bb, :, hd]
            la = dt * v["A"][hd]                                  # log decay of each step
            gam = lam * dt
            nxt = np.append(dt[1:] * (1 - lam[1:]), 0.0)
            scale = gam + nxt
            for t in range(L):
                state = np.exp(np.sum(la[:t + 1])) * v["h0"][bb, hd]     # (P, N)
                for s in range(t + 1):
                    w = gam[s] if s == t else scale[s] * np.exp(np.sum(la[s + 1:t + 1]))
                    state = state + w * np.outer(v["x"][bb, s, hd], v["B"][bb, s, g])
                yt = state @ v["C"][bb, t, g] + v["D"][hd] * v["x"][bb, t, hd]
                zt = v["z"][bb, t, hd]
                yt = yt * zt / (1 + np.exp(-zt))
                _close(y[bb, t, hd], yt, what=f"single-SSD form y (b{bb} h{hd} t{t})")
                if t == L - 1:
                    _close(h[bb, hd], state, what=f"single-SSD form h_last (b{bb} h{hd})")


def check_ssd_trap_previous_token(orc):
    """The previous-token term carried across a split.  (1) A sequence run in
    two pieces, the second starting from the first's h_last and its last
    token's x and B (x_prev, B_prev), equals one run over the whole, at every
    split point, and token-by-token calls chained the same way equal it too
    ("Mamba-3 NKI Kernels for AWS Neuron", section "How it works": the step()
    recurrence carries beta * prev_Bx from token to token).  (2) One token
    with h0 and a previous token, written out:
    S = alpha h0 + beta x_prev B_prev^T + gamma x_0 B_0^T, y = (S C_0 + D x_0) silu(z_0),
    with alpha = exp(dt A), gamma = lam dt, beta = (dt - gamma) alpha."""
    rng = np.random.default_rng(63)
    b, L, H, P, N, G = 2, 10, 4, 3, 5, 2
    v = _trap_inputs(rng, b, L, H, P, N, G)
    args = lambda t0, t1: [v[k][:, t0:t1] for k in ("x", "dt", "lam")] + [v["A"]] + \
        [v[k][:, t0:t1] for k in ("B", "C")] + [v["D"], v["z"][:, t0:t1]]
    y, h = orc.ssd_trap(*args(0, L), v["h0"])
    for L1 in (1, 4, 9):
        y1, h1 = orc.ssd_trap(*args(0, L1), v["h0"])
        y2, h2 = orc.ssd_trap(*args(L1, L), h1, v["x"][:, L1 - 1], v["B"][:, L1 - 1])
        _close(np.concatenate([y1, y2], axis=1), y, rtol=1e-12, what=f"split at {L1}: y")
        _close(h2, h, rtol=1e-12, what=f"split at {L1}: h_last")
    st, ys, xp, bp = v["h0"], [], None, None
    for t in range(L):
        yt, st = orc.ssd_trap(*args(t, t + 1), st, xp, bp)
        ys.append(yt)
        xp, bp = v["x"][:, t], v["B"][:, t]
    _close(np.concatenate(ys, axis=1), y, rtol=1e-12, what="token-by-token chain: y")
    _close(st, h, rtol=1e-12, what="token-by-token chain: h_last")
    xp, bp = rng.standard_normal((b, H, P)), rng.standard_normal((b, G, N))
    y1, h1 = orc.ssd_trap(*args(0, 1), v["h0"], xp, bp)
    for bb in range(b):
        for hd in range(H):
            g = hd // (H // G)
            dt, lam = v["dt"][bb, 0, hd], v["lam"][bb, 0, hd]
            alpha = np.exp(dt * v["A"][hd])
            gamma = lam * dt
            beta = (dt - gamma) * alpha
            S = alpha * v["h0"][bb, hd] + beta * np.outer(xp[bb, hd], bp[bb, g]) + \
                gamma * np.outer(v["x"][bb, 0, hd], v["B"][bb, 0, g])
            zt = v["z"][bb, 0, hd]
            yt = (S @ v["C"][bb, 0, g] + v["D"][hd] * v["x"][bb, 0, hd]) * zt / (1 + np.exp(-zt))
            _close(y1[bb, 0, hd], yt, what=f"one token with a previous token: y (b{bb} h{hd})")
            _close(h1[bb, hd], S, what=f"one token with a previous token: h_last (b{bb} h{hd})")


def _rel_close(got, want, rtol, what):
    got, want = np.asarray(got, dtype=np.float64), np.asarray(want, dtype=np.float64)
    assert got.shape == want.shape, f"{what}: shape {got.shape} != {want.shape}"
    err = np.abs(got - want) / np.maximum(np.abs(want), 1e-300)
    assert float(np.max(err)) <= rtol, f"{what}: max rel err {float(np.max(err)):.3e}"


def check_phase0_softplus(orc):
    """The Phase-0 step map ("Mamba-3 NKI Kernels for AWS Neuron", section "How
    it works", Phase 0) against numpy's log(exp(0) + exp(v)) on [-700, 750]
    (no overflow at the ends), softplus(v) - softplus(-v) = v, softplus(0) =
    log 2, and the bias index of both layouts: element (b, d, t) of a
    (batch, dim, L) array adds bias[d], element (b, t, h) of a (batch, L, H)
    array adds bias[h]."""
    rng = np.random.default_rng(71)
    v = np.concatenate([rng.uniform(-40, 40, 300), [-700.0, -30.0, 0.0, 30.0, 750.0]])
    _rel_close(orc.softplus(v, None, 1), np.logaddexp(0.0, v), 1e-14, "softplus vs logaddexp")
    w = rng.uniform(-30, 30, 200)
    _close(orc.softplus(w, None, 1) - orc.softplus(-w, None, 1), w, rtol=1e-14, what="softplus odd part")
    _close(orc.softplus(np.zeros(1), None, 1), [math.log(2.0)], rtol=1e-15, what="softplus(0)")
    raw, bias = rng.uniform(-6, 6, (2, 3, 5)), rng.uniform(-3, 3, 3)
    _rel_close(orc.softplus(raw, bias, 5).reshape(raw.shape), np.logaddexp(0.0, raw + bias[None, :, None]),
               1e-14, "softplus bias per channel (batch, dim, L)")
    raw2 = rng.uniform(-6, 6, (2, 5, 3))
    _rel_close(orc.softplus(raw2, bias, 1).reshape(raw2.shape), np.logaddexp(0.0, raw2 + bias[None, None, :]),
               1e-14, "softplus bias per head (batch, L, H)")


def check_phase0_sigmoid_and_softplus_grad(orc):
    """sigmoid against scipy's expit, sigmoid(v) + sigmoid(-v) = 1 and
    sigmoid(0) = 1/2; the chain rule through the biased softplus against
    central finite differences of the softplus itself (its derivative is the
    sigmoid), in the (batch, dim, L) layout."""
    from scipy.special import expit
    rng = np.random.default_rng(72)
    v = np.concatenate([rng.uniform(-40, 40, 300), [-700.0, 0.0, 700.0]])
    _rel_close(orc.sigmoid(v), expit(v), 1e-14, "sigmoid vs expit")
    _close(orc.sigmoid(v) + orc.sigmoid(-v), np.ones_like(v), rtol=1e-15, what="sigmoid symmetry")
    _close(orc.sigmoid(np.zeros(1)), [0.5], rtol=0.0, what="sigmoid(0)")
    raw, bias = rng.uniform(-6, 6, (2, 3, 4)), rng.uniform(-2, 2, 3)
    g = rng.standard_normal(raw.shape)
    got = orc.softplus_grad(raw, bias, 4, g).reshape(raw.shape)
    e = 1e-6
    fd = (orc.softplus(raw + e, bias, 4) - orc.softplus(raw - e, bias, 4)).reshape(raw.shape) / (2 * e)
    _close(got, g * fd, rtol=1e-8, what="softplus chain rule vs finite differences")


# --------------------------------------------------------------------------
# Rotary step on B and C (Mamba-3 complex-valued state)
# --------------------------------------------------------------------------

def check_rope_closed_form(orc):
    """Constant step c and a constant theta w per (head, pair): after step t
    the angle is a0 - (t + 1) c w, so a unit vector on the first member of
    pair k (k and k + N/2) turns into (cos phi, sin phi) on the pair and one
    on the second member into (-sin phi, cos phi); C (here 3 B) the same, and
    angle_last = a0 - L c w.  Per-head thetas, two groups with distinct
    amplitudes (head h reads group h / (H / G))."""
    batch, L, H, G, N = 1, 7, 4, 2, 6
    half = N // 2
    c = 0.3
    rng = np.random.default_rng(81)
    w = rng.uniform(-2.0, 2.0, (H, half))
    a0 = rng.uniform(-1.0, 1.0, (batch, H, half))
    dt = np.full((batch, L, H), c)
    theta = np.broadcast_to(w[None, None], (batch, L, H, half)).copy()
    for k in range(half):
        for second in (False, True):
            B = np.zeros((batch, L, G, N))
            for g in range(G):
                B[:, :, g, k + (half if second else 0)] = g + 1.0
            br, cr, last = orc.rope_bc(dt, theta, B, 3.0 * B, a0)
            for h in range(H):
                amp = h // (H // G) + 1.0
                for t in range(L):
                    phi = a0[0, h, k] - (t + 1) * c * w[h, k]
                    want = np.zeros(N)
                    if second:
                        want[k], want[k + half] = -math.sin(phi), math.cos(phi)
                    else:
                        want[k], want[k + half] = math.cos(phi), math.sin(phi)
                    _close(br[0, t, h], amp * want, what=f"rope B (k{k} second={second} h{h} t{t})")
                    _close(cr[0, t, h], 3.0 * amp * want, what=f"rope C (k{k} second={second} h{h} t{t})")
            _close(last, a0 - L * c * w[None], what="rope angle_last")


def check_rope_complex_state(orc):
    """Rotating B and C turns the real SSD into the complex-state recurrence of
    Mamba-3.  With each pair (k, k + N/2) of B and C read as a complex number
    b, c:  h_t = exp(dt_t A) exp(i dt_t theta_t) h_{t-1} + dt_t x_t b_t and
    y_t = Re(sum_k conj(c_t,k) h_t,k).  That loop, on the unrotated B and C,
    must equal the oracle's SSD (one group per head) on the oracle's rotated
    B and C."""
    rng = np.random.default_rng(82)
    batch, L, H, P, N = 2, 9, 3, 2, 4
    half = N // 2
    x, dt, A, B, C, _, _ = _rand_ssd(rng, batch, L, H, P, N, 1)
    theta = rng.uniform(-3.0, 3.0, (batch, L, H, half))
    br, cr, _ = orc.rope_bc(dt, theta, B, C)
    y, _ = orc.ssd(x, dt, A, br, cr)
    for b in range(batch):
        for h in range(H):
            hc = np.zeros((P, half), dtype=complex)
            for t in range(L):
                bz = B[b, t, 0, :half] + 1j * B[b, t, 0, half:]
                cz = C[b, t, 0, :half] + 1j * C[b, t, 0, half:]
                rot = np.exp(dt[b, t, h] * A[h]) * np.exp(1j * dt[b, t, h] * theta[b, t, h])
                hc = rot[None, :] * hc + dt[b, t, h] * x[b, t, h][:, None] * bz[None, :]
                _close(y[b, t, h], np.real(hc @ np.conj(cz)), rtol=1e-11, what=f"complex state (b{b} h{h} t{t})")


def check_rope_chaining_and_identities(orc):
    """Two calls, the second starting from the first's angle_last, equal one
    call over the whole sequence; one set of angles for all heads
    (theta_heads = 1) equals the same angles given to every head; theta = 0
    copies B and C to every head of their group unchanged."""
    rng = np.random.default_rng(83)
    batch, L, H, G, N = 2, 11, 4, 2, 8
    half = N // 2
    dt = np.exp(rng.uniform(math.log(1e-2), math.log(0.5), (batch, L, H)))
    theta = rng.uniform(-3.0, 3.0, (batch, L, H, half))
    B = rng.standard_normal((batch, L, G, N))
    C = rng.standard_normal((batch, L, G, N))
    a0 = rng.uniform(-2.0, 2.0, (batch, H, half))
    full = orc.rope_bc(dt, theta, B, C, a0)
    m = 5
    first = orc.rope_bc(dt[:, :m], theta[:, :m], B[:, :m], C[:, :m], a0)
    second = orc.rope_bc(dt[:, m:], theta[:, m:], B[:, m:], C[:, m:], first[2])
    _close(np.concatenate([first[0], second[0]], axis=1), full[0], what="rope chained B")
    _close(np.concatenate([first[1], second[1]], axis=1), full[1], what="rope chained C")
    _close(second[2], full[2], what="rope chained angle_last")
    shared = theta[:, :, :1]
    one = orc.rope_bc(dt, shared, B, C, a0)
    every = orc.rope_bc(dt, np.repeat(shared, H, axis=2), B, C, a0)
    for a, b_, what in zip(one, every, ("B", "C", "angle_last")):
        _close(a, b_, rtol=0.0, what=f"rope shared theta {what}")
    br, cr, last = orc.rope_bc(dt, np.zeros_like(theta), B, C, a0 * 0.0)
    _close(br, np.repeat(B, H // G, axis=2), rtol=0.0, what="rope theta = 0, B")
    _close(cr, np.repeat(C, H // G, axis=2), rtol=0.0, what="rope theta = 0, C")
    _close(last, np.zeros_like(last), rtol=0.0, what="rope theta = 0, angle_last")


def check_rope_bwd_finite_differences(orc):
    """The rotary step's backward against central finite differences of the
    forward: the gradient of L = sum(wB * B_rot) + sum(wC * C_rot) +
    sum(wA * angle_last) with respect to each element of dt, theta, B, C and
    angle0; shared and per-head theta, two group counts."""
    for seed, (b, L, H, G, N, TH) in ((31, (2, 5, 4, 2, 6, 1)), (32, (1, 6, 2, 1, 4, 2)), (33, (1, 4, 3, 3, 8, 3))):
        rng = np.random.default_rng(seed)
        inp = {"dt": np.exp(rng.uniform(-3, 0, (b, L, H))), "theta": rng.standard_normal((b, L, TH, N // 2)),
               "B": rng.standard_normal((b, L, G, N)), "C": rng.standard_normal((b, L, G, N)),
               "angle0": rng.uniform(-3, 3, (b, H, N // 2))}
        wb, wc = rng.standard_normal((b, L, H, N)), rng.standard_normal((b, L, H, N))
        wa = rng.standard_normal((b, H, N // 2))

        def loss(v):
            br, cr, last = orc.rope_bc(v["dt"], v["theta"], v["B"], v["C"], v["angle0"])
            return float(np.sum(wb * br) + np.sum(wc * cr) + np.sum(wa * last))

        g = orc.rope_bc_bwd(inp["dt"], inp["theta"], inp["B"], inp["C"], inp["angle0"], wb, wc, wa)
        for k, gk in (("dt", "ddt"), ("theta", "dtheta"), ("B", "dB"), ("C", "dC"), ("angle0", "dangle0")):
            fd = np.zeros_like(inp[k])
            for idx in np.ndindex(inp[k].shape):
                e = 1e-6 * max(1.0, abs(inp[k][idx]))
                lo, hi = dict(inp), dict(inp)
                lo[k], hi[k] = inp[k].copy(), inp[k].copy()
                lo[k][idx] -= e
                hi[k][idx] += e
                fd[idx] = (loss(hi) - loss(lo)) / (2 * e)
            _close(g[gk], fd, rtol=1e-7, what=f"rope d{k} against finite differences (seed {seed})")


def check_rope_bwd_orthogonality(orc):
    """With one group per head the rotation of B (and of C) at fixed angles is
    orthogonal, so its transpose preserves inner products:
    <dB, B> = <dB_rot, B_rot> and <dC, C> = <dC_rot, C_rot>; and with theta = 0
    and no starting angle nothing turns: dB = dB_rot, dC = dC_rot, ddt = 0."""
    rng = np.random.default_rng(34)
    b, L, H, N = 2, 9, 3, 10
    dt = np.exp(rng.uniform(-3, 0, (b, L, H)))
    theta = rng.standard_normal((b, L, H, N // 2))
    B, C = rng.standard_normal((b, L, H, N)), rng.standard_normal((b, L, H, N))
    a0 = rng.uniform(-3, 3, (b, H, N // 2))
    wb, wc = rng.standard_normal((b, L, H, N)), rng.standard_normal((b, L, H, N))
    br, cr, _ = orc.rope_bc(dt, theta, B, C, a0)
    g = orc.rope_bc_bwd(dt, theta, B, C, a0, wb, wc, None)
    _close(np.sum(g["dB"] * B), np.sum(wb * br), what="rope <dB, B> = <dB_rot, B_rot>")
    _close(np.sum(g["dC"] * C), np.sum(wc * cr), what="rope <dC, C> = <dC_rot, C_rot>")
    g0 = orc.rope_bc_bwd(dt, np.zeros_like(theta), B, C, None, wb, wc, None)
    _close(g0["dB"], wb, rtol=0.0, what="rope theta = 0: dB = dB_rot")
    _close(g0["dC"], wc, rtol=0.0, what="rope theta = 0: dC = dC_rot")
    _close(g0["ddt"], np.zeros_like(dt), rtol=0.0, what="rope theta = 0: ddt = 0")


ALL_CHECKS = [
    check_scan_hand_example,
    check_scan_a_zero_prefix_sum,
    check_scan_constant_coeff_geometric,
    check_scan_l1,
    check_scan_bruteforce,
    check_scan_invariants,
    check_ssd_hand_example,
    check_ssd_chunked_equals_recurrence,
    check_ssd_equals_scan_broadcast,
    check_ssd_invariants,
    check_decode_steps_chain,
    check_scan_bwd_finite_differences,
    check_ssd_bwd_finite_differences,
    check_ssd_bwd_equals_scan_bwd_broadcast,
    check_ssd_trap_lam_one_is_ssd,
    check_ssd_trap_single_ssd_form,
    check_ssd_trap_previous_token,
    check_ssd_trap_bwd_finite_differences,
    check_ssd_trap_bwd_lam_one_is_ssd_bwd,
    check_phase0_softplus,
    check_phase0_sigmoid_and_softplus_grad,
    check_rope_closed_form,
    check_rope_complex_state,
    check_rope_chaining_and_identities,
    check_rope_bwd_finite_differences,
    check_rope_bwd_orthogonality,
]
