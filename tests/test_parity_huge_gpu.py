"""Tensors of more than 2^31 elements: the kernels address every tensor with
64-bit offsets (only the offsets inside one chunk's rows are 32-bit, and the
host keeps those rows below 2^25 elements), so outputs past element 2^31 are
as correct as the first ones.

The inputs are drawn on the device by the seeded generators of the synthetic
input module (the host generator would take minutes at this size); the oracle
then checks, row by row, the channel rows or heads that lie past element 2^31,
the one that straddles it, and one near the start, on copies of exactly those
input slices.  Bars as everywhere else: max|y - y_ref| / max|y_ref| <= 2e-2
with bf16 storage, the same for the final state; the rotary backward's
float32 gradients at 1e-5.
"""
import gc
from concurrent.futures import ThreadPoolExecutor

import numpy as np
import pytest
import torch

import oracle
import state_space_model_ssm_amd as ssm
from state_space_model_ssm_amd.synth import ScanShape, SsdShape, make_scan_inputs_on, make_ssd_inputs_on

pytestmark = pytest.mark.gpu

TOL_BF16 = 2e-2


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    torch.cuda.init()
    yield
    gc.collect()
    torch.cuda.empty_cache()


def rel_err(got, want) -> float:
    got = np.asarray(got, dtype=np.float64)
    want = np.asarray(want, dtype=np.float64)
    scale = float(np.max(np.abs(want)))
    diff = np.abs(got - want)
    if np.isnan(diff).any():
        return float("inf")
    return float(np.max(diff)) / (scale if scale > 0 else 1.0)


def _cpu(t):
    return None if t is None else t.contiguous().cpu()


def test_scan_beyond_2pow31_elements():
    """u, delta, z and y of 2 x 2048 channels x 540672 steps (2.21e9 elements
    each, bf16, gate and D): the channel row that straddles element 2^31, one
    wholly past it, the last one and the first one, against the oracle."""
    s = ScanShape(2, 2048, 16, 540672, 1, "bf16", has_z=True, dskip="normal", a_kind="loguniform", seed=41)
    assert s.elements > 2 ** 31
    print(f"scan {s.batch}x{s.dim}x{s.seqlen} bf16: {s.elements} elements per tensor", flush=True)
    inp = make_scan_inputs_on(s, "cuda")
    y = torch.full(inp["u"].shape, float("nan"), dtype=torch.bfloat16, device="cuda")
    h = torch.full((s.batch, s.dim, s.dstate), float("nan"), dtype=torch.float32, device="cuda")
    ssm.scan_fwd(inp["u"], inp["delta"], inp["A"], inp["B"], inp["C"], inp["D"], inp["z"], y=y, h_last=h,
                 n_chunks=1)
    torch.cuda.synchronize()
    first_past = 2 ** 31 // s.seqlen          # the flat row b * dim + d that holds element 2^31
    rows = [0, first_past, first_past + 1, s.batch * s.dim - 1]
    assert first_past * s.seqlen < 2 ** 31 < (first_past + 1) * s.seqlen

    def take(r):
        b, d = divmod(r, s.dim)
        one = {
            "u": _cpu(inp["u"][b:b + 1, d:d + 1]), "delta": _cpu(inp["delta"][b:b + 1, d:d + 1]),
            "z": _cpu(inp["z"][b:b + 1, d:d + 1]), "A": _cpu(inp["A"][d:d + 1]), "D": _cpu(inp["D"][d:d + 1]),
            "B": _cpu(inp["B"][b:b + 1]), "C": _cpu(inp["C"][b:b + 1]),
        }
        return one, _cpu(y[b, d].float()), _cpu(h[b, d])

    picked = [take(r) for r in rows]

    def check(item):
        one, yg, hg = item
        yr, hr = oracle.scan(one["u"], one["delta"], one["A"], one["B"], one["C"], one["D"], one["z"])
        return rel_err(yg, yr[0, 0]), rel_err(hg, hr[0, 0])

    with ThreadPoolExecutor(max_workers=len(rows)) as ex:
        errs = list(ex.map(check, picked))
    for r, (ey, eh) in zip(rows, errs):
        print(f"  flat row {r} (elements {r * s.seqlen} .. {(r + 1) * s.seqlen - 1}): y {ey:.2e} h_last {eh:.2e}",
              flush=True)
        assert ey <= TOL_BF16 and eh <= TOL_BF16, (r, ey, eh)
    del inp, y, h
    gc.collect()
    torch.cuda.empty_cache()


@pytest.mark.parametrize("kind", ["plain", "rotary"])
def test_ssd_beyond_2pow31_elements(kind):
    """x, z and y of 8 x 65600 steps x 64 heads x 64 (2.15e9 elements each,
    bf16, gate and D; 1025 chunks per head): the last batch row's steps
    65088.. lie past element 2^31.  Heads 0 and 63 of that row and head 5 of
    the first row against the oracle (the plain SSD, or the fused rotary SSD
    against the oracle's rotary step followed by its SSD)."""
    s = SsdShape(8, 65600, 64, 64, 128, 1, 64, "bf16", has_z=True, dskip="normal", seed=42)
    assert s.elements > 2 ** 31
    print(f"ssd ({kind}) {s.batch}x{s.seqlen}x{s.nheads}x{s.headdim} bf16: {s.elements} elements per tensor",
          flush=True)
    inp = make_ssd_inputs_on(s, "cuda")
    theta = None
    if kind == "rotary":
        g = torch.Generator(device="cuda")
        g.manual_seed(43)
        theta = torch.randn((s.batch, s.seqlen, 1, s.dstate // 2), generator=g, device="cuda").to(torch.bfloat16)
    y = torch.full(inp["x"].shape, float("nan"), dtype=torch.bfloat16, device="cuda")
    h = torch.full((s.batch, s.nheads, s.headdim, s.dstate), float("nan"), dtype=torch.float32, device="cuda")
    if kind == "plain":
        ssm.ssd_chunked_fwd(inp["x"], inp["dt"], inp["A"], inp["B"], inp["C"], inp["D"], inp["z"], y=y, h_last=h)
    else:
        ssm.ssd_rope_chunked_fwd(inp["x"], inp["dt"], inp["A"], inp["B"], inp["C"], theta, inp["D"], inp["z"],
                                 y=y, h_last=h)
    torch.cuda.synchronize()
    t_past = 2 ** 31 // (s.nheads * s.headdim) - (s.batch - 1) * s.seqlen
    assert 0 < t_past < s.seqlen
    pairs = [(s.batch - 1, 0), (s.batch - 1, s.nheads - 1), (0, 5)]

    def take(bh):
        b, hh = bh
        one = {
            "x": _cpu(inp["x"][b:b + 1, :, hh:hh + 1]), "dt": _cpu(inp["dt"][b:b + 1, :, hh:hh + 1]),
            "z": _cpu(inp["z"][b:b + 1, :, hh:hh + 1]), "A": _cpu(inp["A"][hh:hh + 1]),
            "D": _cpu(inp["D"][hh:hh + 1]), "B": _cpu(inp["B"][b:b + 1]), "C": _cpu(inp["C"][b:b + 1]),
            "theta": None if theta is None else _cpu(theta[b:b + 1]),
        }
        return one, _cpu(y[b, :, hh].float()), _cpu(h[b, hh])

    picked = [take(bh) for bh in pairs]

    def check(item):
        one, yg, hg = item
        Bm, Cm = one["B"], one["C"]
        if one["theta"] is not None:
            rb, rc, _ = oracle.rope_bc(one["dt"], one["theta"], Bm, Cm)
            Bm = torch.from_numpy(rb).to(torch.bfloat16)
            Cm = torch.from_numpy(rc).to(torch.bfloat16)
        yr, hr = oracle.ssd(one["x"], one["dt"], one["A"], Bm, Cm, one["D"], one["z"])
        return rel_err(yg, yr[0, :, 0]), rel_err(hg, hr[0, 0]), rel_err(yg[t_past:], yr[0, t_past:, 0])

    # One at a time: the oracle's forward SSD keeps its state in a static
    # buffer, so it must not run in two host threads at once.
    errs = [check(item) for item in picked]
    for (b, hh), (ey, eh, ep) in zip(pairs, errs):
        print(f"  batch row {b} head {hh}: y {ey:.2e} (steps {t_past}.. {ep:.2e}) h_last {eh:.2e}", flush=True)
        assert ey <= TOL_BF16 and eh <= TOL_BF16 and ep <= TOL_BF16, (b, hh, ey, eh, ep)
    del inp, y, h, theta
    gc.collect()
    torch.cuda.empty_cache()


def test_rope_bwd_beyond_2pow31_elements():
    """The rotary backward with float32 upstream gradients of 8 x 65600
    steps x 64 heads x 128 states (4.3e9 elements each), one head per group
    and theta per head (so every (batch row, head) is independent): heads 0
    and 63 of the last batch row (steps past element 2^31) and head 5 of the
    first, against the oracle on exactly those slices.  Bar: float32 outputs
    from the same stored inputs, 1e-5 of the largest magnitude."""
    batch, L, H, N = 8, 65600, 64, 128
    assert batch * L * H * N > 2 ** 31
    print(f"rope backward {batch}x{L}x{H}x{N}: {batch * L * H * N} elements per gradient", flush=True)
    g = torch.Generator(device="cuda")
    g.manual_seed(44)

    def normal(shape, scale=1.0, dtype=torch.float32):
        return (scale * torch.randn(shape, generator=g, device="cuda")).to(dtype)

    dt = torch.nn.functional.softplus(normal((batch, L, H)) - 4.6).to(torch.bfloat16)
    theta = normal((batch, L, H, N // 2), dtype=torch.bfloat16)
    B = normal((batch, L, H, N), N ** -0.5, torch.bfloat16)
    C = normal((batch, L, H, N), N ** -0.5, torch.bfloat16)
    dB_rot = normal((batch, L, H, N))
    dC_rot = normal((batch, L, H, N))
    angle0 = normal((batch, H, N // 2))
    dal = normal((batch, H, N // 2))
    out = ssm.rope_bc_bwd(dt, theta, B, C, dB_rot=dB_rot, dC_rot=dC_rot, angle0=angle0, dangle_last=dal)
    torch.cuda.synchronize()
    pairs = [(batch - 1, 0), (batch - 1, H - 1), (0, 5)]
    for b, h in pairs:
        s = slice(h, h + 1)
        ref = oracle.rope_bc_bwd(_cpu(dt[b:b + 1, :, s]), _cpu(theta[b:b + 1, :, s]), _cpu(B[b:b + 1, :, s]),
                                 _cpu(C[b:b + 1, :, s]), _cpu(angle0[b:b + 1, s]), _cpu(dB_rot[b:b + 1, :, s]),
                                 _cpu(dC_rot[b:b + 1, :, s]), _cpu(dal[b:b + 1, s]))
        got = {"ddt": out["ddt"][b:b + 1, :, s], "dtheta": out["dtheta"][b:b + 1, :, s],
               "dB": out["dB"][b:b + 1, :, s], "dC": out["dC"][b:b + 1, :, s], "dangle0": out["dangle0"][b:b + 1, s]}
        errs = {k: rel_err(_cpu(v), ref[k]) for k, v in got.items()}
        print(f"  batch row {b} head {h}: " + ", ".join(f"{k} {e:.2e}" for k, e in errs.items()), flush=True)
        for k, e in errs.items():
            assert e <= 1e-5, (b, h, k, e)
    del dt, theta, B, C, dB_rot, dC_rot, angle0, dal, out
    gc.collect()
    torch.cuda.empty_cache()
