"""Parity of the rotary step on B and C (``ssm_rope_bc``) with the float64
CPU oracle, alone and feeding the chunked SSD.

Bar: max|out - ref| / max|ref| <= 1e-5 when every stored tensor is float32,
<= 2e-2 when any is bfloat16, for B_rot, C_rot, angle_last and the SSD's y
and h_last.  Outputs are NaN-poisoned before each call.
"""
import numpy as np
import pytest
import torch

import oracle
import state_space_model_ssm_amd as ssm
from state_space_model_ssm_amd.synth import (WORKLOADS, SsdShape, make_lam, make_raw_step, make_ssd_inputs,
                                             make_state, make_theta)

pytestmark = pytest.mark.gpu

TOL_F32, TOL_BF16 = 1e-5, 2e-2
DT = {"f32": torch.float32, "bf16": torch.bfloat16}


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    torch.cuda.init()


def rel_err(got, want) -> float:
    got = np.asarray(got, dtype=np.float64)
    want = np.asarray(want, dtype=np.float64)
    if want.size == 0:
        return 0.0
    diff = np.abs(got - want)
    if np.isnan(diff).any():
        return float("inf")
    scale = float(np.max(np.abs(want)))
    return float(np.max(diff)) / (scale if scale > 0 else 1.0)


def angle_err(got, want) -> float:
    """Largest difference of two angle arrays modulo 2 pi, over pi (the
    library returns the angle reduced to [-pi, pi]; only its value modulo
    2 pi matters), and inf if any returned angle is outside [-pi, pi]."""
    got = np.asarray(got, dtype=np.float64)
    want = np.asarray(want, dtype=np.float64)
    if got.size == 0:
        return 0.0
    if np.isnan(got).any() or np.abs(got).max() > np.pi * (1 + 1e-6):
        return float("inf")
    d = np.remainder(got - want + np.pi, 2 * np.pi) - np.pi
    return float(np.abs(d).max()) / np.pi


def _inputs(batch, L, H, G, N, TH, dtype, seed, theta_scale):
    rng = np.random.default_rng(seed)
    dt = np.logaddexp(0.0, rng.standard_normal((batch, L, H)) - 4.6)  # softplus: steps around 0.01
    B = rng.standard_normal((batch, L, G, N)) / np.sqrt(N)
    C = rng.standard_normal((batch, L, G, N)) / np.sqrt(N)
    cast = lambda a: torch.from_numpy(a).to(DT[dtype])
    theta = make_theta((batch, L, TH, N // 2), seed + 1, dtype, theta_scale)
    angle0 = torch.from_numpy(rng.uniform(-4.0, 4.0, (batch, H, N // 2)).astype(np.float32))
    return cast(dt), theta, cast(B), cast(C), angle0


def _run(dt, theta, B, C, angle0, out_dtype, **kw):
    batch, L, G, N = B.shape
    H = dt.shape[2]
    br = torch.full((batch, L, H, N), float("nan"), dtype=out_dtype, device="cuda")
    cr = torch.full_like(br, float("nan"))
    al = torch.full((batch, H, N // 2), float("nan"), dtype=torch.float32, device="cuda")
    a0 = None if angle0 is None else angle0.cuda()
    ssm.rope_bc(dt.cuda(), theta.cuda(), B.cuda(), C.cuda(), angle0=a0, out_dtype=out_dtype, B_rot=br,
                C_rot=cr, angle_last=al, **kw)
    torch.cuda.synchronize()
    return br.float().cpu(), cr.float().cpu(), al.cpu()


# (batch, L, H, G, N, theta_heads, in dtype, out dtype, angle0, theta scale, seed)
CASES = [
    (2, 100, 4, 2, 16, 4, "f32", "f32", True, 20.0, 1),     # 64 time segments of 2 steps, ragged
    (1, 1000, 2, 1, 128, 1, "f32", "f32", False, 20.0, 2),  # 8 segments of 125 steps
    (2, 37, 3, 3, 2, 3, "f32", "f32", True, 5.0, 3),        # one pair, most segments empty
    (1, 5, 2, 1, 256, 2, "f32", "bf16", True, 5.0, 4),      # 128 pairs, 4 segments
    (2, 256, 8, 1, 64, 1, "bf16", "bf16", False, 1.0, 5),
    (1, 300, 4, 2, 32, 4, "bf16", "f32", True, 10.0, 6),
    (1, 0, 2, 1, 16, 1, "f32", "f32", True, 1.0, 7),        # empty sequence: angle_last = angle0
    (1, 4096, 2, 1, 16, 2, "f32", "f32", True, 30.0, 8),    # angles reach ~10^3 rad
]


@pytest.mark.parametrize("case", CASES, ids=lambda c: "b{}l{}h{}g{}n{}th{}_{}_{}_a0{}".format(*c[:9]))
def test_rope_matches_oracle(case):
    batch, L, H, G, N, TH, din, dout, with_a0, scale, seed = case
    dt, theta, B, C, angle0 = _inputs(batch, L, H, G, N, TH, din, seed, scale)
    a0 = angle0 if with_a0 else None
    br, cr, al = _run(dt, theta, B, C, a0, DT[dout])
    rb, rc, ra = oracle.rope_bc(dt, theta, B, C, a0)
    tol = TOL_F32 if din == dout == "f32" else TOL_BF16
    assert rel_err(br, rb) <= tol and rel_err(cr, rc) <= tol, (rel_err(br, rb), rel_err(cr, rc))
    assert angle_err(al, ra) <= TOL_F32, angle_err(al, ra)


@pytest.mark.parametrize("with_bias", [True, False])
def test_rope_dt_softplus(with_bias):
    batch, L, H, N = 2, 130, 4, 32
    raw, bias = make_raw_step((batch, L, H), H, seed=41, dtype="f32")
    _, theta, B, C, angle0 = _inputs(batch, L, H, 1, N, H, "f32", 42, 10.0)
    bias = bias if with_bias else None
    br, cr, al = _run(raw, theta, B, C, angle0, torch.float32, dt_softplus=True,
                      dt_bias=None if bias is None else bias.cuda())
    rb, rc, ra = oracle.rope_bc(raw, theta, B, C, angle0, dt_softplus=True, dt_bias=bias)
    assert max(rel_err(br, rb), rel_err(cr, rc), angle_err(al, ra)) <= TOL_F32


def test_rope_chained_in_place():
    """A sequence rotated in three pieces, each call taking the angle its
    predecessor left in the same buffer, equals one call over the whole."""
    batch, L, H, G, N = 2, 200, 4, 1, 64
    dt, theta, B, C, angle0 = _inputs(batch, L, H, G, N, 1, "f32", 51, 20.0)
    rb, rc, ra = oracle.rope_bc(dt, theta, B, C, angle0)
    ang = angle0.cuda().clone()
    outs = []
    for lo, hi in ((0, 70), (70, 71), (71, 200)):
        sl = lambda t: t[:, lo:hi].contiguous().cuda()
        b_rot, c_rot, _ = ssm.rope_bc(sl(dt), sl(theta), sl(B), sl(C), angle0=ang, angle_last=ang)
        outs.append((b_rot, c_rot))
    torch.cuda.synchronize()
    got_b = torch.cat([o[0] for o in outs], dim=1).float().cpu()
    got_c = torch.cat([o[1] for o in outs], dim=1).float().cpu()
    assert max(rel_err(got_b, rb), rel_err(got_c, rc), angle_err(ang.cpu(), ra)) <= TOL_F32


def test_rope_chained_large_angles():
    """Four chained calls whose running angle grows past 10^4 rad (theta with
    a mean of 400, steps around 0.01: ~4 rad per step over 3000 steps).  The
    angle handed from call to call is reduced modulo 2 pi before its float32
    store, so every piece rotates as one float64 call over the whole sequence
    would (float32 bar)."""
    batch, L, H, G, N = 1, 3000, 2, 1, 32
    rng = np.random.default_rng(71)
    dt = torch.from_numpy(np.logaddexp(0.0, rng.standard_normal((batch, L, H)) - 4.6)).float()
    theta = torch.from_numpy(400.0 + 5.0 * rng.standard_normal((batch, L, H, N // 2))).float()
    B = torch.from_numpy(rng.standard_normal((batch, L, G, N)) / np.sqrt(N)).float()
    C = torch.from_numpy(rng.standard_normal((batch, L, G, N)) / np.sqrt(N)).float()
    angle0 = torch.from_numpy(rng.uniform(-3.0, 3.0, (batch, H, N // 2))).float()
    rb, rc, ra = oracle.rope_bc(dt, theta, B, C, angle0)
    assert np.abs(ra).max() > 1e4
    ang = angle0.cuda().clone()
    outs = []
    for lo, hi in ((0, 700), (700, 1500), (1500, 1501), (1501, 3000)):
        sl = lambda t: t[:, lo:hi].contiguous().cuda()
        b_rot, c_rot, _ = ssm.rope_bc(sl(dt), sl(theta), sl(B), sl(C), angle0=ang, angle_last=ang)
        outs.append((b_rot, c_rot))
    torch.cuda.synchronize()
    got_b = torch.cat([o[0] for o in outs], dim=1).cpu()
    got_c = torch.cat([o[1] for o in outs], dim=1).cpu()
    errs = (rel_err(got_b, rb), rel_err(got_c, rc), angle_err(ang.cpu(), ra))
    assert max(errs) <= TOL_F32, errs


@pytest.mark.parametrize("trap", [False, True])
def test_rope_feeds_ssd(trap):
    """Rotary step, then the chunked SSD with one group per head (bf16, so one
    head per workgroup), against the oracle's rotary step and SSD."""
    s = SsdShape(8, 192, 32, 64, 128, 1, 64, "bf16", has_z=True, dskip="normal", seed=61)
    inp = make_ssd_inputs(s)
    theta = make_theta((s.batch, s.seqlen, 1, s.dstate // 2), 62, "bf16", 20.0)
    lam = make_lam((s.batch, s.seqlen, s.nheads), 63)
    h0 = make_state((s.batch, s.nheads, s.headdim, s.dstate), 64, 0.5)
    d = {k: (None if v is None else v.cuda()) for k, v in inp.items()}
    br, cr, _ = ssm.rope_bc(d["dt"], theta.cuda(), d["B"], d["C"])
    if trap:
        y, hl = ssm.ssd_trap_chunked_fwd(d["x"], d["dt"], lam.cuda(), d["A"], br, cr, d["D"], d["z"], h0=h0.cuda())
    else:
        y, hl = ssm.ssd_chunked_fwd(d["x"], d["dt"], d["A"], br, cr, d["D"], d["z"], h0=h0.cuda())
    torch.cuda.synchronize()
    rb, rc, _ = oracle.rope_bc(inp["dt"], theta, inp["B"], inp["C"])
    # The SSD reads B and C as bf16: the oracle SSD takes the oracle's rotated
    # B and C rounded the same way.
    rb16 = torch.from_numpy(rb).to(torch.bfloat16)
    rc16 = torch.from_numpy(rc).to(torch.bfloat16)
    if trap:
        ry, rh = oracle.ssd_trap(inp["x"], inp["dt"], lam, inp["A"], rb16, rc16, inp["D"], inp["z"], h0)
    else:
        ry, rh = oracle.ssd(inp["x"], inp["dt"], inp["A"], rb16, rc16, inp["D"], inp["z"], h0)
    assert rel_err(y.float().cpu(), ry) <= TOL_BF16 and rel_err(hl.cpu(), rh) <= TOL_BF16


def test_rope_named_workload_full_size():
    """The rotary step at the SSD workload's full size (32 x 256, 32 heads,
    dstate 128, bf16, one set of angles for all heads), every output."""
    s = WORKLOADS["ssd_32x256_h32p64n128_bf16"]
    inp = make_ssd_inputs(s)
    theta = make_theta((s.batch, s.seqlen, 1, s.dstate // 2), 71, "bf16", 1.0)
    br, cr, al = _run(inp["dt"], theta, inp["B"], inp["C"], None, torch.bfloat16)
    rb, rc, ra = oracle.rope_bc(inp["dt"], theta, inp["B"], inp["C"])
    assert max(rel_err(br, rb), rel_err(cr, rc)) <= TOL_BF16
    assert angle_err(al, ra) <= TOL_F32


def test_rope_prefill_then_decode_steps():
    """Mamba-3 serving order: a 64-token prefill (rotary step, then the SSD on
    the per-head B and C), then 16 decode tokens, each a one-token rotary step
    from the cached angle (updated in place) and an SSD decode step on the
    cached state; every output against the oracle over all 80 tokens."""
    s = SsdShape(2, 80, 8, 64, 64, 1, 64, "bf16", has_z=True, dskip="normal", seed=91)
    inp = make_ssd_inputs(s)
    theta = make_theta((s.batch, s.seqlen, s.nheads, s.dstate // 2), 92, "bf16", 10.0)
    rb, rc, _ = oracle.rope_bc(inp["dt"], theta, inp["B"], inp["C"])
    rb16 = torch.from_numpy(rb).to(torch.bfloat16)
    rc16 = torch.from_numpy(rc).to(torch.bfloat16)
    ry, rh = oracle.ssd(inp["x"], inp["dt"], inp["A"], rb16, rc16, inp["D"], inp["z"])
    d = {k: (None if v is None else v.cuda()) for k, v in inp.items()}
    th = theta.cuda()
    T = 64
    pre = lambda t: t[:, :T].contiguous()
    br, cr, ang = ssm.rope_bc(pre(d["dt"]), pre(th), pre(d["B"]), pre(d["C"]))
    y0, state = ssm.ssd_chunked_fwd(pre(d["x"]), pre(d["dt"]), d["A"], br, cr, d["D"], pre(d["z"]))
    ys = [y0.float()]
    for t in range(T, s.seqlen):
        one = lambda a: a[:, t:t + 1].contiguous()
        b1, c1, _ = ssm.rope_bc(one(d["dt"]), one(th), one(d["B"]), one(d["C"]), angle0=ang, angle_last=ang)
        y = ssm.ssd_step(d["x"][:, t].contiguous(), d["dt"][:, t].contiguous(), d["A"], b1[:, 0].contiguous(),
                         c1[:, 0].contiguous(), d["D"], d["z"][:, t].contiguous(), state=state)
        ys.append(y.float()[:, None])
    torch.cuda.synchronize()
    got = torch.cat(ys, dim=1).cpu()
    assert rel_err(got, ry) <= TOL_BF16, rel_err(got, ry)
    assert rel_err(state.cpu(), rh) <= TOL_BF16, rel_err(state.cpu(), rh)


def test_rope_trap_prefill_then_128_decode_steps():
    """Mamba-3 SISO serving order with the trapezoid: a 64-token prefill
    (rotary step, then the trapezoidal chunked SSD on the per-head B and C),
    then 128 decode tokens, each a one-token rotary step from the cached angle
    and an ssd_trap_step on the cached state that passes the previous token's
    x and rotated B.  Every output against the oracle (rotary step, then the
    trapezoidal SSD) over all 192 tokens."""
    s = SsdShape(1, 192, 32, 64, 128, 1, 64, "bf16", has_z=True, dskip="ones", seed=95)
    inp = make_ssd_inputs(s)
    lam = make_lam((1, 192, 32), seed=96)
    theta = make_theta((1, 192, 1, 64), 97, "bf16", 5.0)
    rb, rc, _ = oracle.rope_bc(inp["dt"], theta, inp["B"], inp["C"])
    rb16 = torch.from_numpy(rb).to(torch.bfloat16)
    rc16 = torch.from_numpy(rc).to(torch.bfloat16)
    ry, rh = oracle.ssd_trap(inp["x"], inp["dt"], lam, inp["A"], rb16, rc16, inp["D"], inp["z"])
    d = {k: (None if v is None else v.cuda()) for k, v in inp.items()}
    th, lamd = theta.cuda(), lam.cuda()
    T = 64
    pre = lambda t: t[:, :T].contiguous()
    br, cr, ang = ssm.rope_bc(pre(d["dt"]), pre(th), pre(d["B"]), pre(d["C"]))
    y0, state = ssm.ssd_trap_chunked_fwd(pre(d["x"]), pre(d["dt"]), pre(lamd), d["A"], br, cr, d["D"], pre(d["z"]))
    ys = [y0.float()]
    xp, bp = d["x"][:, T - 1].contiguous(), br[:, T - 1].contiguous()
    for t in range(T, s.seqlen):
        one = lambda a: a[:, t:t + 1].contiguous()
        b1, c1, _ = ssm.rope_bc(one(d["dt"]), one(th), one(d["B"]), one(d["C"]), angle0=ang, angle_last=ang)
        xt = d["x"][:, t].contiguous()
        y = ssm.ssd_trap_step(xt, d["dt"][:, t].contiguous(), lamd[:, t].contiguous(), d["A"],
                              b1[:, 0].contiguous(), c1[:, 0].contiguous(), d["D"], d["z"][:, t].contiguous(),
                              state=state, x_prev=xp, B_prev=bp)
        ys.append(y.float()[:, None])
        xp, bp = xt, b1[:, 0].contiguous()
    torch.cuda.synchronize()
    got = torch.cat(ys, dim=1).cpu()
    assert rel_err(got, ry) <= TOL_BF16, rel_err(got, ry)
    assert rel_err(state.cpu(), rh) <= TOL_BF16, rel_err(state.cpu(), rh)


# ---------------------------------------------------------------------------
# The fused forms: ssd_rope_chunked_fwd / ssd_rope_trap_chunked_fwd against
# the oracle's rotary step followed by the oracle's SSD on the rotated B and
# C (rounded to bf16, as the SSD reads them).
# ---------------------------------------------------------------------------

# (batch, L, H, G, N, theta_heads, has_z, out dtype, trap, angle0, theta scale, seed)
FUSED_CASES = [
    (2, 192, 8, 1, 128, 1, True, "bf16", False, False, 20.0, 201),   # three whole chunks
    (2, 130, 4, 2, 128, 4, False, "f32", False, True, 20.0, 202),    # ragged tail of 2 steps, per-head theta
    (3, 100, 6, 3, 64, 1, True, "bf16", False, True, 5.0, 203),      # dstate 64, ragged
    (1, 64, 2, 1, 64, 2, False, "f32", False, False, 50.0, 204),     # one whole chunk
    (2, 1, 4, 1, 128, 1, True, "bf16", False, True, 20.0, 205),      # a single step
    (2, 192, 8, 1, 128, 1, True, "bf16", True, False, 20.0, 206),    # trapezoidal
    (2, 77, 4, 2, 64, 4, False, "f32", True, True, 10.0, 207),       # trapezoidal, ragged, dstate 64
    (1, 2048, 2, 1, 128, 1, False, "f32", False, True, 30.0, 208),   # 32 chunks: the angle carry
]


def _fused_inputs(batch, L, H, G, N, TH, has_z, trap, a0, scale, seed):
    s = SsdShape(batch, L, H, 64, N, G, 64, "bf16", has_z=has_z, dskip="normal", seed=seed)
    inp = make_ssd_inputs(s)
    inp["theta"] = make_theta((batch, L, TH, N // 2), seed + 1000, "bf16", scale)
    inp["lam"] = make_lam((batch, L, H), seed + 2000) if trap else None
    inp["h0"] = make_state((batch, H, 64, N), seed + 3000, 0.5)
    rng = np.random.default_rng(seed + 4000)
    inp["angle0"] = torch.from_numpy(rng.uniform(-4.0, 4.0, (batch, H, N // 2)).astype(np.float32)) if a0 else None
    return inp


def _fused_oracle(inp, trap, dt_bias=None, lam_sigmoid=False):
    """The oracle's rotary step, then its SSD on the rotated B and C rounded to
    bf16; dt_bias given: dt holds raw values (the step is softplus(dt + bias))."""
    sp = dict(dt_softplus=dt_bias is not None, dt_bias=dt_bias)
    rb, rc, ra = oracle.rope_bc(inp["dt"], inp["theta"], inp["B"], inp["C"], inp["angle0"], **sp)
    rb16 = torch.from_numpy(rb).to(torch.bfloat16)
    rc16 = torch.from_numpy(rc).to(torch.bfloat16)
    if trap:
        ry, rh = oracle.ssd_trap(inp["x"], inp["dt"], inp["lam"], inp["A"], rb16, rc16, inp["D"], inp["z"],
                                 inp["h0"], lam_sigmoid=lam_sigmoid, **sp)
    else:
        ry, rh = oracle.ssd(inp["x"], inp["dt"], inp["A"], rb16, rc16, inp["D"], inp["z"], inp["h0"], **sp)
    return ry, rh, ra, rb16


def _fused_run(inp, trap, out_dtype, **kw):
    d = {k: (None if v is None else v.cuda()) for k, v in inp.items()}
    batch, L, H, P = inp["x"].shape
    N = inp["B"].shape[3]
    y = torch.full((batch, L, H, P), float("nan"), dtype=out_dtype, device="cuda")
    hl = torch.full((batch, H, P, N), float("nan"), dtype=torch.float32, device="cuda")
    al = torch.full((batch, H, N // 2), float("nan"), dtype=torch.float32, device="cuda")
    bl = torch.full((batch, H, N), float("nan"), dtype=torch.bfloat16, device="cuda")
    common = dict(angle0=d["angle0"], angle_last=al, B_last=bl, h0=d["h0"], y=y, h_last=hl, out_dtype=out_dtype)
    common.update(kw)
    if trap:
        out = ssm.ssd_rope_trap_chunked_fwd(d["x"], d["dt"], d["lam"], d["A"], d["B"], d["C"], d["theta"], d["D"],
                                            d["z"], **common)
    else:
        out = ssm.ssd_rope_chunked_fwd(d["x"], d["dt"], d["A"], d["B"], d["C"], d["theta"], d["D"], d["z"], **common)
    torch.cuda.synchronize()
    return [None if t is None else t.float().cpu() for t in out]


@pytest.mark.parametrize("case", FUSED_CASES, ids=lambda c: "b{}l{}h{}g{}n{}th{}_z{}_{}_trap{}_a0{}".format(*c[:10]))
def test_fused_rope_ssd_matches_oracle(case):
    batch, L, H, G, N, TH, has_z, out, trap, a0, scale, seed = case
    print(f"fused rope ssd case {case}", flush=True)
    inp = _fused_inputs(batch, L, H, G, N, TH, has_z, trap, a0, scale, seed)
    y, hl, al, bl = _fused_run(inp, trap, DT[out])
    ry, rh, ra, rb16 = _fused_oracle(inp, trap)
    errs = (rel_err(y, ry), rel_err(hl, rh), angle_err(al, ra))
    assert errs[0] <= TOL_BF16 and errs[1] <= TOL_BF16 and errs[2] <= TOL_F32, errs
    # The last step's rotated B (bf16): within one bf16 rounding of the oracle's.
    assert rel_err(bl, rb16[:, L - 1].float()) <= 1e-2


def test_fused_rope_ssd_empty_sequence():
    """seqlen 0: h_last is h0, angle_last is angle0 reduced to [-pi, pi], and
    B_last is left untouched."""
    inp = _fused_inputs(2, 0, 4, 1, 128, 1, False, False, True, 1.0, 209)
    inp["angle0"] = inp["angle0"] * 3.0  # beyond [-pi, pi]
    y, hl, al, bl = _fused_run(inp, False, torch.bfloat16)
    assert y.numel() == 0 and torch.isnan(bl).all()
    assert torch.equal(hl, inp["h0"])
    assert angle_err(al, inp["angle0"].double().numpy()) <= TOL_F32


@pytest.mark.parametrize("trap", [False, True])
def test_fused_rope_ssd_dt_softplus(trap):
    """Raw dt with dt_bias (and raw lam): the angles and the SSD use the mapped
    step."""
    inp = _fused_inputs(2, 150, 4, 1, 128, 1, True, trap, True, 10.0, 210)
    raw, bias = make_raw_step((2, 150, 4), 4, 211, "bf16")
    inp["dt"] = raw
    kw = dict(dt_softplus=True, dt_bias=bias.cuda())
    if trap:
        inp["lam"] = torch.from_numpy(np.random.default_rng(212).standard_normal((2, 150, 4))).to(torch.bfloat16)
        kw["lam_sigmoid"] = True
    y, hl, al, _ = _fused_run(inp, trap, torch.bfloat16, **kw)
    ry, rh, ra, _ = _fused_oracle(inp, trap, dt_bias=bias, lam_sigmoid=trap)
    errs = (rel_err(y, ry), rel_err(hl, rh), angle_err(al, ra))
    assert errs[0] <= TOL_BF16 and errs[1] <= TOL_BF16 and errs[2] <= TOL_F32, errs


def test_fused_rope_trap_chained_in_place():
    """A trapezoidal sequence in two fused calls: the second starts from the
    first's h_last, angle_last (updated in place: angle_last is angle0) and
    B_last with x of the first call's last step, and continues the oracle's
    single pass exactly."""
    batch, L, H, N, T1 = 2, 200, 4, 128, 120
    inp = _fused_inputs(batch, L, H, 1, N, 1, True, True, True, 20.0, 213)
    ry, rh, ra, _ = _fused_oracle(inp, True)
    d = {k: (None if v is None else v.cuda()) for k, v in inp.items()}
    cut = lambda t, a, b: t[:, a:b].contiguous()
    ang = d["angle0"].clone()
    y1, h1, _, b1 = ssm.ssd_rope_trap_chunked_fwd(
        cut(d["x"], 0, T1), cut(d["dt"], 0, T1), cut(d["lam"], 0, T1), d["A"], cut(d["B"], 0, T1),
        cut(d["C"], 0, T1), cut(d["theta"], 0, T1), d["D"], cut(d["z"], 0, T1), h0=d["h0"], angle0=ang,
        angle_last=ang, return_B_last=True)
    y2, h2, _, _ = ssm.ssd_rope_trap_chunked_fwd(
        cut(d["x"], T1, L), cut(d["dt"], T1, L), cut(d["lam"], T1, L), d["A"], cut(d["B"], T1, L),
        cut(d["C"], T1, L), cut(d["theta"], T1, L), d["D"], cut(d["z"], T1, L), h0=h1, angle0=ang,
        angle_last=ang, x_prev=d["x"][:, T1 - 1].contiguous(), B_prev=b1)
    torch.cuda.synchronize()
    got = torch.cat([y1, y2], dim=1).float().cpu()
    errs = (rel_err(got, ry), rel_err(h2.cpu(), rh), angle_err(ang.cpu(), ra))
    assert errs[0] <= TOL_BF16 and errs[1] <= TOL_BF16 and errs[2] <= TOL_F32, errs


def test_fused_rope_trap_prefill_then_128_decode_steps():
    """The serving order with the fused prefill: a 64-token fused rotary
    trapezoidal prefill returns h_last, angle_last and B_last (the last
    token's rotated B); 128 decode tokens follow, each a one-token rotary step
    from the cached angle and an ssd_trap_step that passes the previous
    token's x and rotated B.  Every output against the oracle (rotary step,
    then the trapezoidal SSD) over all 192 tokens."""
    batch, L, H, N, T = 2, 192, 8, 128, 64
    inp = _fused_inputs(batch, L, H, 1, N, 1, True, True, True, 5.0, 215)
    ry, rh, ra, _ = _fused_oracle(inp, True)
    d = {k: (None if v is None else v.cuda()) for k, v in inp.items()}
    pre = lambda t: t[:, :T].contiguous()
    ang = d["angle0"].clone()
    y0, state, _, bp = ssm.ssd_rope_trap_chunked_fwd(
        pre(d["x"]), pre(d["dt"]), pre(d["lam"]), d["A"], pre(d["B"]), pre(d["C"]), pre(d["theta"]), d["D"],
        pre(d["z"]), h0=d["h0"], angle0=ang, angle_last=ang, return_B_last=True)
    ys = [y0.float()]
    xp = d["x"][:, T - 1].contiguous()
    for t in range(T, L):
        one = lambda a: a[:, t:t + 1].contiguous()
        b1, c1, _ = ssm.rope_bc(one(d["dt"]), one(d["theta"]), one(d["B"]), one(d["C"]), angle0=ang, angle_last=ang)
        xt = d["x"][:, t].contiguous()
        y = ssm.ssd_trap_step(xt, d["dt"][:, t].contiguous(), d["lam"][:, t].contiguous(), d["A"],
                              b1[:, 0].contiguous(), c1[:, 0].contiguous(), d["D"], d["z"][:, t].contiguous(),
                              state=state, x_prev=xp, B_prev=bp)
        ys.append(y.float()[:, None])
        xp, bp = xt, b1[:, 0].contiguous()
    torch.cuda.synchronize()
    got = torch.cat(ys, dim=1).cpu()
    errs = (rel_err(got, ry), rel_err(state.cpu(), rh), angle_err(ang.cpu(), ra))
    assert errs[0] <= TOL_BF16 and errs[1] <= TOL_BF16 and errs[2] <= TOL_F32, errs


@pytest.mark.parametrize("trap", [False, True])
def test_fused_rope_ssd_named_workload_full_size(trap):
    """The fused rotary SSD at the SSD workload's full size (32 x 256, 32
    heads, headdim 64, dstate 128, bf16, one set of angles for every head),
    every output against the oracle."""
    s = WORKLOADS["ssd_32x256_h32p64n128_bf16"]
    inp = make_ssd_inputs(s)
    inp["theta"] = make_theta((s.batch, s.seqlen, 1, s.dstate // 2), 71, "bf16", 1.0)
    inp["lam"] = make_lam((s.batch, s.seqlen, s.nheads), 72) if trap else None
    inp["h0"] = None
    inp["angle0"] = None
    y, hl, al, bl = _fused_run(inp, trap, torch.bfloat16, h0=None)
    ry, rh, ra, rb16 = _fused_oracle(inp, trap)
    errs = (rel_err(y, ry), rel_err(hl, rh), angle_err(al, ra), rel_err(bl, rb16[:, -1].float()))
    print(f"fused rotary SSD full size (trap={trap}): y {errs[0]:.2e} h_last {errs[1]:.2e} "
          f"angle_last {errs[2]:.2e} B_last {errs[3]:.2e}", flush=True)
    assert errs[0] <= TOL_BF16 and errs[1] <= TOL_BF16 and errs[2] <= TOL_F32 and errs[3] <= 1e-2, errs


@pytest.mark.parametrize("N", [64, 128])
def test_fused_rope_ssd_repeat_runs_identical(N):
    """Repeated calls on the same inputs give bit-identical outputs (every
    sum in the kernel has a fixed order), at both supported dstates."""
    inp = _fused_inputs(3, 100, 6, 3, N, 1, True, False, True, 5.0, 214)
    first = _fused_run(inp, False, torch.bfloat16)
    for _ in range(4):
        again = _fused_run(inp, False, torch.bfloat16)
        for a, b_ in zip(first, again):
            assert torch.equal(a, b_)


def _sweep_fused_cases(n=10, seed=20263):
    """A seeded random draw of fused-call shapes (the same every run)."""
    rng = np.random.default_rng(seed)
    cases = []
    for i in range(n):
        G = int(rng.choice([1, 1, 2]))
        H = G * int(rng.choice([1, 2, 3, 4]))
        cases.append((int(rng.integers(1, 4)), int(rng.integers(1, 300)), H, G, int(rng.choice([64, 128])),
                      int(rng.choice([1, H])), bool(rng.integers(0, 2)), str(rng.choice(["f32", "bf16"])),
                      bool(rng.integers(0, 2)), bool(rng.integers(0, 2)), float(rng.choice([1.0, 5.0, 20.0])),
                      9000 + i))
    return cases


@pytest.mark.parametrize("case", _sweep_fused_cases(),
                         ids=lambda c: "b{}l{}h{}g{}n{}th{}_z{}_{}_trap{}_a0{}".format(*c[:10]))
def test_fused_rope_ssd_random_sweep(case):
    """Seeded random shapes of the fused calls (groups, per-head or shared
    theta, gate, output dtype, trapezoid, starting angle) against the
    oracle's rotary step followed by its SSD."""
    batch, L, H, G, N, TH, has_z, out, trap, a0, scale, seed = case
    print(f"fused sweep case {case}", flush=True)
    inp = _fused_inputs(batch, L, H, G, N, TH, has_z, trap, a0, scale, seed)
    y, hl, al, bl = _fused_run(inp, trap, DT[out])
    ry, rh, ra, rb16 = _fused_oracle(inp, trap)
    errs = (rel_err(y, ry), rel_err(hl, rh), angle_err(al, ra))
    assert errs[0] <= TOL_BF16 and errs[1] <= TOL_BF16 and errs[2] <= TOL_F32, errs
    assert rel_err(bl, rb16[:, L - 1].float()) <= 1e-2
