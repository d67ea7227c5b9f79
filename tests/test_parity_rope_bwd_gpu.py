"""Parity of the rotary step's backward (``ssm_rope_bc_bwd``) with the
float64 CPU oracle, alone and at the end of the Mamba-3 gradient chain
(rotary step -> SSD -> SSD backward -> rotary backward).

The backward receives the same stored inputs as the oracle (bf16 inputs are
widened exactly) and writes float32, so alone it is held to
max|out - ref| / max|ref| <= 1e-5 for ddt, dtheta, dB, dC and dangle0; the
chain through the bf16 SSD is held to 2e-2 as the SSD backward is.  Outputs
are NaN-poisoned before each call.
"""
import zlib
from concurrent.futures import ThreadPoolExecutor

import numpy as np
import pytest
import torch

import oracle
import state_space_model_ssm_amd as ssm
from state_space_model_ssm_amd.synth import (WORKLOADS, SsdShape, make_raw_step, make_ssd_inputs, make_state,
                                             make_theta)

pytestmark = pytest.mark.gpu

TOL_F32, TOL_BF16 = 1e-5, 2e-2
DT = {"f32": torch.float32, "bf16": torch.bfloat16}
KEYS = ("ddt", "dtheta", "dB", "dC", "dangle0")


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


def _inputs(batch, L, H, G, N, TH, dtype, gdtype, with_a0, with_dal, seed, theta_scale=1.0):
    rng = np.random.default_rng(seed)
    cast = lambda a, d: torch.from_numpy(np.ascontiguousarray(a)).to(DT[d])
    inp = {
        "dt": cast(np.logaddexp(0.0, rng.standard_normal((batch, L, H)) - 4.6), dtype),  # steps around 0.01
        "B": cast(rng.standard_normal((batch, L, G, N)) / np.sqrt(N), dtype),
        "C": cast(rng.standard_normal((batch, L, G, N)) / np.sqrt(N), dtype),
        "theta": make_theta((batch, L, TH, N // 2), seed + 1, dtype, theta_scale),
        "dB_rot": cast(rng.standard_normal((batch, L, H, N)), gdtype),
        "dC_rot": cast(rng.standard_normal((batch, L, H, N)), gdtype),
        "angle0": torch.from_numpy(rng.uniform(-4.0, 4.0, (batch, H, N // 2)).astype(np.float32)) if with_a0 else None,
        "dangle_last": (torch.from_numpy(rng.standard_normal((batch, H, N // 2)).astype(np.float32))
                        if with_dal else None),
    }
    return inp


def _gpu_bwd(inp, **kw):
    cu = {k: (None if v is None else v.cuda()) for k, v in inp.items()}
    batch, L, H = inp["dt"].shape
    nan = lambda shape: torch.full(tuple(shape), float("nan"), dtype=torch.float32, device="cuda")
    out = {"ddt": nan((batch, L, H)), "dtheta": nan(inp["theta"].shape), "dB": nan(inp["B"].shape),
           "dC": nan(inp["C"].shape), "dangle0": nan((batch, H, inp["B"].shape[3] // 2))}
    g = ssm.rope_bc_bwd(cu["dt"], cu["theta"], cu["B"], cu["C"], dB_rot=cu["dB_rot"], dC_rot=cu["dC_rot"],
                        angle0=cu["angle0"], dangle_last=cu["dangle_last"], out=out, **kw)
    torch.cuda.synchronize()
    return {k: (None if v is None else v.cpu()) for k, v in g.items()}


def _oracle_bwd(inp, **kw):
    return oracle.rope_bc_bwd(inp["dt"], inp["theta"], inp["B"], inp["C"], inp["angle0"], inp["dB_rot"],
                              inp["dC_rot"], inp["dangle_last"], **kw)


def _check(g, ref, tol, label):
    errs = {k: rel_err(g[k], ref[k]) for k in KEYS}
    print(f"{label}: " + ", ".join(f"{k} {v:.2e}" for k, v in errs.items()), flush=True)
    for k, e in errs.items():
        assert e <= tol, (k, e)


# (batch, L, H, G, N, theta_heads, in dtype, grad dtype, angle0, dangle_last)
CASES = [
    (2, 200, 4, 1, 16, 1, "f32", "f32", True, True),      # heads share B, C and theta: both head sums
    (1, 1, 2, 2, 2, 2, "f32", "f32", False, False),       # one step, one pair
    (2, 130, 3, 3, 8, 3, "f32", "f32", True, True),       # everything per head: no workspace
    (2, 100, 4, 2, 32, 4, "bf16", "f32", True, True),     # two heads per group, theta per head
    (1, 257, 8, 1, 64, 1, "bf16", "bf16", True, True),    # ragged segments
    (2, 64, 6, 3, 128, 6, "bf16", "f32", False, True),
    (2, 300, 4, 1, 128, 1, "bf16", "f32", True, True),
    (1, 700, 2, 1, 256, 1, "f32", "f32", True, True),     # 32 threads per row, 16 segments
    (1, 33, 5, 5, 4, 1, "f32", "bf16", True, False),      # two pairs per thread, theta shared
    (3, 5, 2, 1, 64, 2, "bf16", "bf16", True, True),      # fewer steps than segments
]


@pytest.mark.parametrize("case", CASES, ids=lambda c: "b{}l{}h{}g{}n{}th{}_{}_{}_a0{}_dal{}".format(*c))
def test_rope_bwd_matches_oracle(case):
    seed = 9100 + zlib.crc32(repr(case).encode()) % 1000
    inp = _inputs(*case, seed=seed)
    _check(_gpu_bwd(inp), _oracle_bwd(inp), TOL_F32, str(case))


def test_rope_bwd_large_angles():
    """Angles that run to ~1e4 rad over 4096 steps (theta scaled up): the
    angle is rebuilt in float64 as in the forward, so the rotations stay
    exact to float32 rounding."""
    inp = _inputs(1, 4096, 2, 1, 32, 1, "f32", "f32", True, True, seed=9201, theta_scale=200.0)
    _check(_gpu_bwd(inp), _oracle_bwd(inp), TOL_F32, "large angles")


@pytest.mark.parametrize("with_bias", [True, False])
def test_rope_bwd_dt_softplus(with_bias):
    """Raw dt with softplus(dt + dt_bias) as the step: ddt is the raw value's
    gradient."""
    batch, L, H = 2, 150, 4
    inp = _inputs(batch, L, H, 1, 64, 1, "bf16", "f32", True, True, seed=9300)
    raw, bias = make_raw_step((batch, L, H), H, 9301, "bf16")
    inp["dt"] = raw
    bias = bias if with_bias else None
    g = _gpu_bwd(inp, dt_softplus=True, dt_bias=None if bias is None else bias.cuda())
    _check(g, _oracle_bwd(inp, dt_softplus=True, dt_bias=bias), TOL_F32, f"softplus bias={with_bias}")


def test_rope_bwd_empty_sequence():
    """L = 0: dangle0 = dangle_last (and zero without it); nothing else."""
    inp = _inputs(2, 0, 4, 1, 16, 1, "bf16", "f32", True, True, seed=9400)
    g = _gpu_bwd(inp)
    assert torch.equal(g["dangle0"], inp["dangle_last"])
    inp["dangle_last"] = None
    g = _gpu_bwd(inp)
    assert torch.equal(g["dangle0"], torch.zeros_like(g["dangle0"]))
    assert g["ddt"].numel() == 0 and g["dB"].numel() == 0


def test_rope_bwd_repeat_runs_identical():
    """Every output element is written by one thread and head sums run in
    head order: two calls give the same bits."""
    inp = _inputs(2, 300, 8, 1, 128, 1, "bf16", "f32", True, True, seed=9500)
    a, b = _gpu_bwd(inp), _gpu_bwd(inp)
    for k in KEYS:
        assert torch.equal(a[k], b[k]), k


def test_rope_bwd_workload_full_size():
    """The SSD workload's rotary shapes (batch 32, 256 steps, 32 heads sharing
    one group of B, C (dstate 128) and one theta, bf16 inputs, float32
    gradients as the SSD backward writes them): every output, whole tensors,
    against one oracle call."""
    batch, L, H, N = 32, 256, 32, 128
    inp = _inputs(batch, L, H, 1, N, 1, "bf16", "f32", True, True, seed=9600)
    _check(_gpu_bwd(inp), _oracle_bwd(inp), TOL_F32, "full size")


def _chain_gpu(inp, theta, dy, dhl):
    """The GPU chain: rotary step (per-head B, C), SSD backward on them, rotary
    backward on its dB, dC; dt's two shares summed."""
    cu = {k: (None if v is None else v.cuda()) for k, v in inp.items()}
    th_c, dy_c, dhl_c = theta.cuda(), dy.cuda(), dhl.cuda()
    br, cr, _ = ssm.rope_bc(cu["dt"], th_c, cu["B"], cu["C"], return_angle_last=False)
    gs = ssm.ssd_bwd(cu["x"], cu["dt"], cu["A"], br, cr, cu["D"], cu["z"], dy=dy_c, dh_last=dhl_c)
    gr = ssm.rope_bc_bwd(cu["dt"], th_c, cu["B"], cu["C"], dB_rot=gs["dB"], dC_rot=gs["dC"])
    torch.cuda.synchronize()
    got = {"dx": gs["dx"], "ddt": gs["ddt"].float() + gr["ddt"], "dtheta": gr["dtheta"], "dB": gr["dB"],
           "dC": gr["dC"], "dA": gs["dA"], "dD": gs["dD"], "dz": gs["dz"]}
    return {k: (None if v is None else v.float().cpu()) for k, v in got.items()}


def _chain_oracle(inp, theta, dy, dhl):
    """The oracle's same chain in float64, one host thread per batch row (dA
    and dD sum over rows; the oracle's rotary step and backwards keep no
    state between calls)."""
    batch = inp["x"].shape[0]

    def one(b):
        r = {k: (None if v is None else (v[b:b + 1] if k in ("x", "dt", "B", "C", "z") else v))
             for k, v in inp.items()}
        rb, rc, _ = oracle.rope_bc(r["dt"], theta[b:b + 1], r["B"], r["C"])
        rs = oracle.ssd_bwd(r["x"], r["dt"], r["A"], rb, rc, r["D"], r["z"], None, dy[b:b + 1], dhl[b:b + 1])
        rr = oracle.rope_bc_bwd(r["dt"], theta[b:b + 1], r["B"], r["C"], None, rs["dB"], rs["dC"], None)
        return {"dx": rs["dx"], "ddt": rs["ddt"] + rr["ddt"], "dtheta": rr["dtheta"], "dB": rr["dB"],
                "dC": rr["dC"], "dA": rs["dA"], "dD": rs["dD"], "dz": rs["dz"]}

    with ThreadPoolExecutor(max_workers=min(batch, 16)) as ex:
        parts = list(ex.map(one, range(batch)))
    out = {}
    for k in parts[0]:
        if parts[0][k] is None:
            out[k] = None
        elif k in ("dA", "dD"):
            out[k] = np.sum([q[k] for q in parts], axis=0)
        else:
            out[k] = np.concatenate([q[k] for q in parts])
    return out


def _check_chain(got, want, label):
    errs = {}
    for k in got:
        if want[k] is None:
            assert got[k] is None, k
            continue
        errs[k] = rel_err(got[k], want[k])
    print(f"{label}: " + ", ".join(f"{k} {v:.2e}" for k, v in errs.items()), flush=True)
    for k, e in errs.items():
        assert e <= TOL_BF16, (k, e)


@pytest.mark.parametrize("case", [(2, 192, 4, 1, 64, 1), (1, 130, 4, 2, 128, 4)],
                         ids=lambda c: "b{}l{}h{}g{}n{}th{}".format(*c))
def test_mamba3_gradient_chain(case):
    """The Mamba-3 SISO layer's gradient path: B, C rotated per head by the
    rotary step, the SSD on the rotated B, C (ngroups = nheads), the SSD
    backward for dy and dh_last, then the rotary backward on the SSD's dB, dC.
    Gradients of x, dt (the SSD's and the rotary step's shares summed),
    theta, B, C, A, D and z against the oracle's same chain in float64."""
    batch, L, H, G, N, TH = case
    seed = 9700 + zlib.crc32(repr(case).encode()) % 1000
    s = SsdShape(batch, L, H, 64, N, G, 64, "bf16", has_z=True, dskip="normal", seed=seed)
    inp = make_ssd_inputs(s)
    theta = make_theta((batch, L, TH, N // 2), seed + 1, "bf16", 1.0)
    dy = make_state((batch, L, H, 64), seed=seed + 2).to(torch.bfloat16)
    dhl = make_state((batch, H, 64, N), seed=seed + 3, scale=0.5)
    _check_chain(_chain_gpu(inp, theta, dy, dhl), _chain_oracle(inp, theta, dy, dhl), f"chain {case}")


def test_mamba3_gradient_chain_full_size():
    """The same chain at the SSD workload's shapes (batch 32, 256 steps, 32
    heads x 64 sharing one group of B, C with dstate 128, one theta, D skip):
    every gradient, whole tensors, against the oracle's chain."""
    s = WORKLOADS["ssd_32x256_h32p64n128_bf16"]
    inp = make_ssd_inputs(s)
    theta = make_theta((s.batch, s.seqlen, 1, s.dstate // 2), 9750, "bf16", 1.0)
    dy = make_state((s.batch, s.seqlen, s.nheads, s.headdim), seed=9751).to(torch.bfloat16)
    dhl = make_state((s.batch, s.nheads, s.headdim, s.dstate), seed=9752, scale=0.5)
    _check_chain(_chain_gpu(inp, theta, dy, dhl), _chain_oracle(inp, theta, dy, dhl), "chain full size")


def _sweep_cases(n=16, seed=20264):
    """A seeded random draw of shapes (the same every run): head counts that
    exercise every head-slot choice (1, 2, 4 or 8 slots, groups that span
    slots and slots that span groups), every dstate, ragged tiles."""
    rng = np.random.default_rng(seed)
    cases = []
    for i in range(n):
        G = int(rng.choice([1, 1, 2, 3]))
        H = G * int(rng.choice([1, 2, 3, 4, 6, 8, 16]))
        N = int(rng.choice([2, 4, 8, 16, 32, 64, 128, 256]))
        cases.append((int(rng.integers(1, 4)), int(rng.integers(1, 400)), H, G, N, int(rng.choice([1, H])),
                      str(rng.choice(["f32", "bf16"])), str(rng.choice(["f32", "bf16"])), bool(rng.integers(0, 2)),
                      bool(rng.integers(0, 2)), float(rng.choice([1.0, 5.0])), 9800 + i))
    return cases


@pytest.mark.parametrize("case", _sweep_cases(),
                         ids=lambda c: "b{}l{}h{}g{}n{}th{}_{}_{}_a0{}_dal{}".format(*c[:10]))
def test_rope_bwd_random_sweep(case):
    """Whole outputs against the oracle on the drawn shapes, at the float32 bar."""
    *shape, scale, seed = case
    print(f"rope bwd sweep case {case}", flush=True)
    inp = _inputs(*shape, seed=seed, theta_scale=scale)
    _check(_gpu_bwd(inp), _oracle_bwd(inp), TOL_F32, f"sweep {case}")


def test_rope_bwd_side_stream_own_workspace():
    """On a side stream with no workspace given, the binding allocates the
    workspace and outputs on that stream; the result equals the default
    stream's bit for bit."""
    inp = _inputs(2, 300, 8, 1, 128, 1, "bf16", "f32", True, True, seed=9900)
    want = _gpu_bwd(inp)
    cu = {k: (None if v is None else v.cuda()) for k, v in inp.items()}
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    g = ssm.rope_bc_bwd(cu["dt"], cu["theta"], cu["B"], cu["C"], dB_rot=cu["dB_rot"], dC_rot=cu["dC_rot"],
                        angle0=cu["angle0"], dangle_last=cu["dangle_last"], stream=s)
    # Work queued on the default stream meanwhile must not disturb it.
    junk = torch.empty(64 << 20, dtype=torch.uint8, device="cuda").fill_(255)
    s.synchronize()
    torch.cuda.synchronize()
    del junk
    for k in KEYS:
        assert torch.equal(g[k].cpu(), want[k]), k
