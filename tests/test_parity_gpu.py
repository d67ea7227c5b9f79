"""Parity of the HIP path (through the C ABI) with the float64 CPU oracle.

Bar (max over the whole compared tensor):
    max|y - y_ref| / max|y_ref| <= 1e-5 when every stored tensor is float32,
                                 <= 2e-2 when any is bfloat16,
and the same for h_last.  Outputs are NaN-poisoned before each call, so an
element the kernels fail to write shows up as NaN.

Small cases run the oracle on the whole tensor; they span several channel
tiles and time tiles with ragged tails.  The five named workloads run at full
size in the launch configuration the benchmark uses, and the oracle checks the
whole output tensors (y and h_last; every gradient for the backward).  The
scan oracle is independent per batch row, so the large workloads run it on
the batch rows in parallel host threads (the float64 sums over batch rows of
dA and dD are then added here); the measured errors are printed.
"""
import math
import zlib
from concurrent.futures import ThreadPoolExecutor

import numpy as np
import pytest
import torch

import oracle
import state_space_model_ssm_amd as ssm
from state_space_model_ssm_amd.synth import (WORKLOADS, ScanShape, SsdShape, make_lam, make_raw_step,
                                             make_scan_inputs, make_ssd_inputs, make_state)

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
    scale = float(np.max(np.abs(want)))
    diff = np.abs(got - want)
    if np.isnan(diff).any():
        return float("inf")
    return float(np.max(diff)) / (scale if scale > 0 else 1.0)


def _dev(t):
    return None if t is None else t.cuda()


def run_scan(inp, out_dtype=None, n_chunks=0, with_h=True, h0=None):
    u = _dev(inp["u"])
    out_dt = u.dtype if out_dtype is None else out_dtype
    y = torch.full(u.shape, float("nan"), dtype=out_dt, device="cuda")
    h = None
    if with_h:
        h = torch.full((u.shape[0], u.shape[1], inp["B"].shape[2]), float("nan"),
                       dtype=torch.float32, device="cuda")
    y, h = ssm.scan_fwd(u, _dev(inp["delta"]), _dev(inp["A"]), _dev(inp["B"]), _dev(inp["C"]),
                        _dev(inp["D"]), _dev(inp["z"]), h0=_dev(h0), out_dtype=out_dt,
                        n_chunks=n_chunks, y=y, h_last=h, return_h_last=with_h)
    torch.cuda.synchronize()
    return y.float().cpu(), (None if h is None else h.cpu())


def ref_scan(inp, h0=None):
    return oracle.scan(inp["u"], inp["delta"], inp["A"], inp["B"], inp["C"], inp["D"], inp["z"], h0=h0)


def _scan_steps(inp, t0, t1):
    """The inputs restricted to steps [t0, t1) (contiguous copies)."""
    out = dict(inp)
    for k in ("u", "delta", "z", "B", "C"):
        if inp[k] is not None:
            out[k] = inp[k][..., t0:t1].contiguous()
    return out


def tol_for(*dtypes):
    return TOL_BF16 if any(d in ("bf16", torch.bfloat16) for d in dtypes) else TOL_F32


# ---------------------------------------------------------------------------
# Selective scan: small cases, whole-tensor oracle
# ---------------------------------------------------------------------------

SCAN_CASES = [
    # (batch, dim, N, L, G, dtype, has_z, dskip, n_chunks)
    (1, 64, 16, 128, 1, "f32", False, "ones", 1),
    (3, 50, 16, 257, 1, "f32", True, "normal", 1),      # ragged channel tile and time tile
    (2, 48, 16, 100, 2, "f32", True, "normal", 0),      # groups, ragged per group
    (2, 40, 16, 1, 1, "f32", True, "normal", 1),        # L = 1
    (2, 40, 16, 2, 1, "f32", True, "none", 1),
    (1, 33, 16, 31, 1, "f32", False, "none", 1),
    (1, 33, 16, 33, 1, "f32", True, "normal", 1),
    (2, 20, 16, 300, 1, "f32", True, "normal", 3),      # chunked carry
    (2, 20, 16, 301, 1, "f32", True, "normal", 7),      # chunked, ragged chunks
    (1, 16, 16, 1000, 2, "f32", True, "normal", 16),
    (1, 24, 16, 129, 1, "f32", True, "normal", 129),    # 32-step chunks, ragged last
    (2, 64, 1, 77, 1, "f32", True, "normal", 1),
    (2, 300, 1, 40, 3, "f32", True, "normal", 2),       # 256-channel tiles, ragged
    (2, 70, 2, 65, 1, "f32", True, "normal", 1),
    (2, 70, 4, 65, 2, "f32", False, "normal", 2),
    (2, 70, 8, 65, 1, "f32", True, "ones", 1),
    (2, 9, 32, 97, 1, "f32", True, "normal", 1),
    (2, 6, 64, 97, 2, "f32", True, "normal", 3),
    (2, 50, 16, 257, 1, "bf16", True, "normal", 1),
    (2, 50, 16, 257, 1, "bf16", True, "ones", 4),
    (2, 50, 16, 264, 1, "bf16", True, "normal", 1),     # vector tiles, then an element tail
    (1, 12, 64, 130, 1, "bf16", False, "normal", 1),
]


@pytest.mark.parametrize("case", SCAN_CASES, ids=lambda c: "b{}d{}n{}l{}g{}_{}_z{}_{}_k{}".format(*c))
def test_scan_small(case):
    batch, dim, N, L, G, dtype, has_z, dskip, k = case
    s = ScanShape(batch, dim, N, L, G, dtype, has_z=has_z, dskip=dskip, a_kind="loguniform",
                  seed=1000 + zlib.crc32(repr(case).encode()) % 1000)
    inp = make_scan_inputs(s)
    y, h = run_scan(inp, n_chunks=k)
    yr, hr = ref_scan(inp)
    tol = tol_for(dtype)
    assert rel_err(y, yr) <= tol, rel_err(y, yr)
    assert rel_err(h, hr) <= tol, rel_err(h, hr)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_scan_misaligned_rows(dtype):
    """Inputs one element past a 16-byte boundary (L a multiple of the vector
    width): the library must take the element path for every tile."""
    s = ScanShape(2, 40, 16, 128, 1, dtype, has_z=True, dskip="normal", seed=91)
    inp = make_scan_inputs(s)

    def shifted(t):
        flat = torch.empty(t.numel() + 8, dtype=t.dtype, device="cuda")
        v = flat[1:1 + t.numel()].view(t.shape)
        v.copy_(t.to("cuda"))
        return v

    y, h = ssm.scan_fwd(shifted(inp["u"]), shifted(inp["delta"]), _dev(inp["A"]), shifted(inp["B"]),
                        shifted(inp["C"]), _dev(inp["D"]), shifted(inp["z"]))
    torch.cuda.synchronize()
    yr, hr = ref_scan(inp)
    assert rel_err(y.float().cpu(), yr) <= tol_for(dtype)
    assert rel_err(h.cpu(), hr) <= tol_for(dtype)


@pytest.mark.parametrize("in_dt,out_dt", [("f32", "bf16"), ("bf16", "f32")])
def test_scan_mixed_dtypes(in_dt, out_dt):
    s = ScanShape(2, 40, 16, 150, 1, in_dt, has_z=True, dskip="normal", seed=77)
    inp = make_scan_inputs(s)
    y, h = run_scan(inp, out_dtype=DT[out_dt])
    yr, hr = ref_scan(inp)
    tol = tol_for(in_dt, out_dt)
    assert rel_err(y, yr) <= tol
    assert rel_err(h, hr) <= tol_for(in_dt)


def test_scan_without_h_last_and_empty_seqlen():
    s = ScanShape(2, 40, 16, 70, 1, "f32", seed=5)
    inp = make_scan_inputs(s)
    y, _ = run_scan(inp, with_h=False)
    assert rel_err(y, ref_scan(inp)[0]) <= TOL_F32
    # L = 0: nothing to read or write, h_last is the zero initial state.
    e = make_scan_inputs(ScanShape(2, 40, 16, 0, 1, "f32", seed=6))
    y, h = run_scan(e)
    assert y.numel() == 0 and torch.all(h == 0)


def test_scan_degenerate_values():
    """A = 0 (no decay: prefix sums) and delta = 0 (no input: y = D u gate)."""
    s = ScanShape(2, 40, 16, 200, 1, "f32", a_kind="zero", seed=8)
    inp = make_scan_inputs(s)
    y, h = run_scan(inp)
    yr, hr = ref_scan(inp)
    assert rel_err(y, yr) <= TOL_F32 and rel_err(h, hr) <= TOL_F32
    inp["delta"] = torch.zeros_like(inp["delta"])
    y, h = run_scan(inp)
    yr, hr = ref_scan(inp)
    assert rel_err(y, yr) <= TOL_F32 and torch.all(h == 0)


def test_scan_chunk_count_does_not_change_the_result():
    s = ScanShape(2, 32, 16, 1000, 1, "f32", seed=9)
    inp = make_scan_inputs(s)
    yr, hr = ref_scan(inp)
    for k in (1, 2, 5, 16, 64):
        y, h = run_scan(inp, n_chunks=k)
        assert rel_err(y, yr) <= TOL_F32, k
        assert rel_err(h, hr) <= TOL_F32, k


def test_scan_deterministic():
    s = ScanShape(2, 64, 16, 500, 1, "f32", seed=10)
    inp = make_scan_inputs(s)
    for k in (1, 4):
        a = run_scan(inp, n_chunks=k)
        b = run_scan(inp, n_chunks=k)
        assert torch.equal(a[0], b[0]) and torch.equal(a[1], b[1])


def test_side_stream_without_caller_workspace():
    """Calls on a side stream with the workspace left to the binding: the
    binding's workspace and outputs belong to that stream, so memory the
    current stream allocates and overwrites right after the call (while the
    side stream may still be running) cannot be the workspace.  Chunked scan
    forward and scan backward against the oracle."""
    s = ScanShape(4, 256, 16, 2048, 1, "f32", has_z=True, dskip="normal", a_kind="loguniform", seed=4050)
    inp = make_scan_inputs(s)
    dy = make_state((4, 256, 2048), seed=4051)
    side = torch.cuda.Stream()
    d = {k: _dev(v) for k, v in inp.items()}
    dyd = dy.cuda()
    torch.cuda.synchronize()
    need_f = 8 * 4 * 256 * 15 * 16
    with torch.cuda.stream(side):
        # Queue work ahead so the calls below are still pending when they return.
        for _ in range(3):
            ssm.scan_fwd(d["u"], d["delta"], d["A"], d["B"], d["C"], d["D"], d["z"], n_chunks=1)
    y, h = ssm.scan_fwd(d["u"], d["delta"], d["A"], d["B"], d["C"], d["D"], d["z"], n_chunks=16,
                        stream=side)
    g = ssm.scan_bwd(d["u"], d["delta"], d["A"], d["B"], d["C"], d["D"], d["z"], dy=dyd, stream=side)
    junk = [torch.full((need_f // 4,), float("nan"), device="cuda") for _ in range(4)]
    big = torch.full((ssm.scan_bwd_workspace_size(ssm._scan_dims(d["u"], d["B"], 0, 0, 0)) // 4,),
                     float("nan"), device="cuda")
    torch.cuda.synchronize()
    del junk, big
    yr, hr = ref_scan(inp)
    assert rel_err(y.cpu(), yr) <= TOL_F32 and rel_err(h.cpu(), hr) <= TOL_F32
    ref = oracle.scan_bwd(inp["u"], inp["delta"], inp["A"], inp["B"], inp["C"], inp["D"], inp["z"], None, dy, None)
    for k in ("du", "ddelta", "dA", "dB", "dC", "dD", "dz", "dh0"):
        assert rel_err(g[k].cpu(), ref[k]) <= TOL_BWD_F32, k


# ---------------------------------------------------------------------------
# Selective scan: initial state h0 and continuation of a split sequence
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("dtype,N", [("f32", 16), ("f32", 4), ("bf16", 16), ("bf16", 64)])
def test_scan_h0(dtype, N):
    s = ScanShape(2, 50, N, 257, 1, dtype, has_z=True, dskip="normal", a_kind="loguniform",
                  seed=4100 + N)
    inp = make_scan_inputs(s)
    h0 = make_state((2, 50, N), seed=4200 + N)
    yr, hr = ref_scan(inp, h0=h0)
    tol = tol_for(dtype)
    for k in (1, 3, 9):
        y, h = run_scan(inp, n_chunks=k, h0=h0)
        assert rel_err(y, yr) <= tol, (k, rel_err(y, yr))
        assert rel_err(h, hr) <= tol, (k, rel_err(h, hr))


@pytest.mark.parametrize("L1", [1, 100, 128, 257])
def test_scan_split_continuation_in_place(L1):
    """Steps [0, L1) then [L1, L), the state carried in one tensor updated in
    place (h_last is h0), equal one call over [0, L)."""
    L = 300
    s = ScanShape(2, 40, 16, L, 1, "f32", has_z=True, dskip="normal", a_kind="loguniform", seed=4300)
    inp = make_scan_inputs(s)
    yr, hr = ref_scan(inp)
    a, b = _scan_steps(inp, 0, L1), _scan_steps(inp, L1, L)
    state = torch.full((2, 40, 16), float("nan"), dtype=torch.float32, device="cuda")
    ys = []
    for part, k, h0 in ((a, 4, None), (b, 1, state)):
        y, _ = ssm.scan_fwd(_dev(part["u"]), _dev(part["delta"]), _dev(part["A"]), _dev(part["B"]),
                            _dev(part["C"]), _dev(part["D"]), _dev(part["z"]), h0=h0, n_chunks=k,
                            h_last=state)
        ys.append(y.cpu())
    torch.cuda.synchronize()
    assert rel_err(torch.cat(ys, dim=-1), yr) <= TOL_F32
    assert rel_err(state.cpu(), hr) <= TOL_F32


# ---------------------------------------------------------------------------
# Selective scan: the named workloads at full size
# ---------------------------------------------------------------------------

def _batch_rows(inp, b, keys=("u", "delta", "z", "B", "C")):
    """Batch row b of the scan inputs (a view per row; A and D are shared)."""
    return {k: (v[b:b + 1] if (k in keys and v is not None) else v) for k, v in inp.items()}


def ref_scan_rows(inp, h0=None):
    """The scan oracle over the whole tensor, one host thread per batch row
    (the rows are independent; each thread runs the unchanged oracle)."""
    batch = inp["u"].shape[0]

    def one(b):
        return ref_scan(_batch_rows(inp, b), None if h0 is None else h0[b:b + 1])

    with ThreadPoolExecutor(max_workers=min(batch, 16)) as ex:
        parts = list(ex.map(one, range(batch)))
    return np.concatenate([p[0] for p in parts]), np.concatenate([p[1] for p in parts])


@pytest.mark.parametrize("name", ["tiny_f32", "page1_1536x128_f32", "long_prefill_8x1536x2048_f32",
                                  "large_channel_4x5120x4096_bf16"])
def test_scan_named_workload_full_size(name):
    """Each named scan workload at full size, in the launch configuration the
    benchmark times, against the oracle over the whole y and h_last."""
    s = WORKLOADS[name]
    inp = make_scan_inputs(s)
    y, h = run_scan(inp)
    tol = tol_for(s.dtype)
    yr, hr = ref_scan_rows(inp)
    ey, eh = rel_err(y, yr), rel_err(h, hr)
    print(f"{name}: whole-tensor rel err y {ey:.3e}, h_last {eh:.3e} (bar {tol:g})")
    assert ey <= tol, ey
    assert eh <= tol, eh


# ---------------------------------------------------------------------------
# Scalar-decay chunked SSD
# ---------------------------------------------------------------------------

def run_ssd(inp, out_dtype=None, with_h=True, h0=None):
    x = _dev(inp["x"])
    out_dt = x.dtype if out_dtype is None else out_dtype
    y = torch.full(x.shape, float("nan"), dtype=out_dt, device="cuda")
    h = None
    if with_h:
        b, L, H, P = x.shape
        h = torch.full((b, H, P, inp["B"].shape[3]), float("nan"), dtype=torch.float32, device="cuda")
    y, h = ssm.ssd_chunked_fwd(x, _dev(inp["dt"]), _dev(inp["A"]), _dev(inp["B"]), _dev(inp["C"]),
                               _dev(inp["D"]), _dev(inp["z"]), h0=_dev(h0), out_dtype=out_dt, y=y,
                               h_last=h, return_h_last=with_h)
    torch.cuda.synchronize()
    return y.float().cpu(), (None if h is None else h.cpu())


def ref_ssd(inp, h0=None):
    return oracle.ssd(inp["x"], inp["dt"], inp["A"], inp["B"], inp["C"], inp["D"], inp["z"], h0=h0)


SSD_CASES = [
    # (batch, L, H, N, G, has_z, dskip)
    (1, 64, 1, 128, 1, False, "ones"),
    (2, 256, 4, 128, 1, False, "ones"),
    (2, 200, 4, 128, 2, True, "normal"),     # ragged last chunk, groups, gate
    (1, 1, 2, 128, 1, True, "normal"),       # L = 1
    (3, 130, 3, 64, 1, False, "normal"),
    (2, 64, 4, 64, 4, True, "none"),
]


@pytest.mark.parametrize("case", SSD_CASES, ids=lambda c: "b{}l{}h{}n{}g{}_z{}_{}".format(*c))
def test_ssd_small(case):
    batch, L, H, N, G, has_z, dskip = case
    s = SsdShape(batch, L, H, 64, N, G, 64, "bf16", has_z=has_z, dskip=dskip, seed=2000 + L + H)
    inp = make_ssd_inputs(s)
    y, h = run_ssd(inp)
    yr, hr = ref_ssd(inp)
    assert rel_err(y, yr) <= TOL_BF16, rel_err(y, yr)
    assert rel_err(h, hr) <= TOL_BF16, rel_err(h, hr)


# Workgroups take 4 heads of a group when batch * nheads >= 1024, 2 heads when
# it is >= 512 (or a group's head count is even but not a multiple of 4), so
# that the grid still has a workgroup per CU.  These cases run those paths
# with ragged chunks, groups, h0, gate, float32 y and the trapezoid, whole
# tensors against the oracle.
WIDE_SSD_CASES = [
    # (batch, L, H, N, G, has_z, out, trap, h0)           heads per workgroup
    (16, 100, 64, 128, 2, False, "bf16", False, True),   # 4
    (16, 70, 64, 64, 4, False, "bf16", False, False),    # 4, dstate 64
    (16, 100, 64, 128, 1, True, "bf16", True, True),     # 4, trapezoid and gate
    (16, 65, 64, 128, 2, True, "f32", False, False),     # 4, float32 y and gate
    (8, 130, 64, 128, 1, True, "bf16", False, True),     # 2 (gate)
    (8, 65, 64, 128, 2, False, "f32", False, False),     # 2 (float32 y)
    (8, 100, 64, 128, 1, True, "bf16", True, True),      # 2 (trapezoid)
    (86, 64, 6, 128, 1, False, "bf16", False, False),    # 2 (6 heads per group)
]


@pytest.mark.parametrize("case", WIDE_SSD_CASES, ids=lambda c: "b{}l{}h{}n{}g{}_z{}_{}_trap{}_h0{}".format(*c))
def test_ssd_multi_head_workgroups(case):
    batch, L, H, N, G, has_z, out, trap, with_h0 = case
    s = SsdShape(batch, L, H, 64, N, G, 64, "bf16", has_z=has_z, dskip="normal",
                 seed=7400 + zlib.crc32(repr(case).encode()) % 1000)
    inp = make_ssd_inputs(s)
    h0 = make_state((batch, H, 64, N), seed=7500 + L, scale=0.5) if with_h0 else None
    out_dt = DT[out]
    if trap:
        lam = make_lam((batch, L, H), seed=7600 + L)
        y, h = run_trap(inp, lam, h0, out_dtype=out_dt)
        yr, hr = oracle.ssd_trap(inp["x"], inp["dt"], lam, inp["A"], inp["B"], inp["C"], inp["D"], inp["z"], h0)
    else:
        y, h = run_ssd(inp, out_dtype=out_dt, h0=h0)
        yr, hr = ref_ssd(inp, h0=h0)
    assert rel_err(y, yr) <= TOL_BF16, rel_err(y, yr)
    assert rel_err(h, hr) <= TOL_BF16, rel_err(h, hr)


def test_ssd_f32_output_and_empty():
    s = SsdShape(2, 128, 2, 64, 128, 1, 64, "bf16", seed=31)
    inp = make_ssd_inputs(s)
    y, h = run_ssd(inp, out_dtype=torch.float32)
    yr, hr = ref_ssd(inp)
    assert rel_err(y, yr) <= TOL_BF16 and rel_err(h, hr) <= TOL_BF16
    e = make_ssd_inputs(SsdShape(2, 0, 2, 64, 128, 1, 64, "bf16", seed=32))
    y, h = run_ssd(e)
    assert y.numel() == 0 and torch.all(h == 0)


@pytest.mark.parametrize("N", [64, 128])
def test_ssd_h0(N):
    s = SsdShape(2, 200, 4, 64, N, 2, 64, "bf16", has_z=True, dskip="normal", seed=4400 + N)
    inp = make_ssd_inputs(s)
    h0 = make_state((2, 4, 64, N), seed=4500 + N, scale=0.5)
    y, h = run_ssd(inp, h0=h0)
    yr, hr = ref_ssd(inp, h0=h0)
    assert rel_err(y, yr) <= TOL_BF16, rel_err(y, yr)
    assert rel_err(h, hr) <= TOL_BF16, rel_err(h, hr)


@pytest.mark.parametrize("L1", [1, 64, 100])
def test_ssd_split_continuation_in_place(L1):
    L = 256
    s = SsdShape(2, L, 4, 64, 128, 1, 64, "bf16", dskip="normal", seed=4600)
    inp = make_ssd_inputs(s)
    yr, hr = ref_ssd(inp)
    state = torch.full((2, 4, 64, 128), float("nan"), dtype=torch.float32, device="cuda")
    ys = []
    for t0, t1, h0 in ((0, L1, None), (L1, L, state)):
        part = {k: (None if v is None else (v[:, t0:t1].contiguous() if k in ("x", "dt", "B", "C", "z") else v))
                for k, v in inp.items()}
        y, _ = ssm.ssd_chunked_fwd(_dev(part["x"]), _dev(part["dt"]), _dev(part["A"]), _dev(part["B"]),
                                   _dev(part["C"]), _dev(part["D"]), _dev(part["z"]), h0=h0, h_last=state)
        ys.append(y.float().cpu())
    torch.cuda.synchronize()
    assert rel_err(torch.cat(ys, dim=1), yr) <= TOL_BF16
    assert rel_err(state.cpu(), hr) <= TOL_BF16


def test_ssd_named_workload_full_size():
    """The SSD workload (batch 32, 256 steps, 32 heads x 64, dstate 128) at
    full size against the oracle over the whole y and h_last."""
    s = WORKLOADS["ssd_32x256_h32p64n128_bf16"]
    inp = make_ssd_inputs(s)
    y, h = run_ssd(inp)
    yr, hr = ref_ssd(inp)
    ey, eh = rel_err(y, yr), rel_err(h, hr)
    print(f"ssd_32x256_h32p64n128_bf16: whole-tensor rel err y {ey:.3e}, h_last {eh:.3e} (bar {TOL_BF16:g})")
    assert ey <= TOL_BF16, ey
    assert eh <= TOL_BF16, eh


def test_ssd_deterministic():
    s = SsdShape(2, 192, 4, 64, 128, 1, 64, "bf16", seed=33)
    inp = make_ssd_inputs(s)
    a = run_ssd(inp)
    b = run_ssd(inp)
    assert torch.equal(a[0], b[0]) and torch.equal(a[1], b[1])


# ---------------------------------------------------------------------------
# Single-token decode steps (state cache updated in place)
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("dtype,N,G,has_z", [("f32", 16, 1, True), ("f32", 1, 1, False), ("f32", 4, 2, True),
                                             ("f32", 64, 1, True), ("f32", 256, 1, False),
                                             ("bf16", 16, 1, True), ("bf16", 128, 2, True)])
def test_scan_decode_steps(dtype, N, G, has_z):
    """Consecutive ssm_scan_step calls from h0 equal one scan over the same
    steps from h0 (y at every step, and the final state)."""
    L = 12
    s = ScanShape(2, 40, N, L, G, dtype, has_z=has_z, dskip="normal", a_kind="loguniform",
                  seed=4700 + N + G)
    inp = make_scan_inputs(s)
    h0 = make_state((2, 40, N), seed=4800 + N)
    yr, hr = ref_scan(inp, h0=h0)
    state = h0.cuda().clone()
    ys = []
    for t in range(L):
        tok = {k: (None if inp[k] is None else inp[k][..., t].contiguous().cuda())
               for k in ("u", "delta", "z", "B", "C")}
        y = ssm.scan_step(tok["u"], tok["delta"], _dev(inp["A"]), tok["B"], tok["C"], _dev(inp["D"]),
                          tok["z"], state=state)
        ys.append(y.float().cpu())
    torch.cuda.synchronize()
    tol = tol_for(dtype)
    assert rel_err(torch.stack(ys, dim=-1), yr) <= tol
    assert rel_err(state.cpu(), hr) <= tol


@pytest.mark.parametrize("P,N,G,has_z", [(64, 128, 1, False), (64, 64, 2, True), (5, 16, 1, True)])
def test_ssd_decode_steps(P, N, G, has_z):
    L = 10
    s = SsdShape(2, L, 4, P, N, G, 64, "bf16", has_z=has_z, dskip="normal", seed=4900 + P + N)
    inp = make_ssd_inputs(s)
    S0 = make_state((2, 4, P, N), seed=5000 + N, scale=0.5)
    yr, hr = ref_ssd(inp, h0=S0)
    state = S0.cuda().clone()
    ys = []
    for t in range(L):
        tok = {k: (None if inp[k] is None else inp[k][:, t].contiguous().cuda())
               for k in ("x", "dt", "z", "B", "C")}
        y = ssm.ssd_step(tok["x"], tok["dt"], _dev(inp["A"]), tok["B"], tok["C"], _dev(inp["D"]), tok["z"],
                         state=state)
        ys.append(y.float().cpu())
    torch.cuda.synchronize()
    assert rel_err(torch.stack(ys, dim=1), yr) <= TOL_BF16
    assert rel_err(state.cpu(), hr) <= TOL_BF16


def test_decode_steps_at_bench_state_sizes():
    """One step of each decode call on the state sizes the bench times: the
    scan step on (4, 5120, 16) bf16 with a gate, the SSD step on
    (32, 32 heads, 64, 128) bf16; whole outputs and states against the oracle."""
    g = torch.Generator().manual_seed(5990)
    rnd = lambda *sh: torch.randn(*sh, generator=g).to(torch.bfloat16)
    pos = lambda *sh: (torch.rand(*sh, generator=g) * 0.1 + 1e-3).to(torch.bfloat16)
    b, d, n = 4, 5120, 16
    u, dl, z, Bm, Cm = rnd(b, d), pos(b, d), rnd(b, d), rnd(b, 1, n), rnd(b, 1, n)
    A = -torch.rand(d, n, generator=g) - 0.5
    D = torch.randn(d, generator=g)
    S = make_state((b, d, n), seed=5991)
    state = S.cuda().clone()
    y = ssm.scan_step(_dev(u), _dev(dl), _dev(A), _dev(Bm), _dev(Cm), _dev(D), _dev(z), state=state)
    torch.cuda.synchronize()
    yr, hr = oracle.scan_step(u, dl, A, Bm, Cm, D, z, state=S)
    assert rel_err(y.float().cpu(), yr) <= TOL_BF16
    assert rel_err(state.cpu(), hr) <= TOL_BF16
    b, H, P, n = 32, 32, 64, 128
    x, dt, Bm, Cm = rnd(b, H, P), pos(b, H), rnd(b, 1, n), rnd(b, 1, n)
    Ah = -torch.rand(H, generator=g) - 0.5
    Dh = torch.ones(H)
    S = make_state((b, H, P, n), seed=5992, scale=0.1)
    state = S.cuda().clone()
    y = ssm.ssd_step(_dev(x), _dev(dt), _dev(Ah), _dev(Bm), _dev(Cm), _dev(Dh), None, state=state)
    torch.cuda.synchronize()
    yr, hr = oracle.ssd_step(x, dt, Ah, Bm, Cm, Dh, None, state=S)
    assert rel_err(y.float().cpu(), yr) <= TOL_BF16
    assert rel_err(state.cpu(), hr) <= TOL_BF16


def _offset_copy(t, elems=1):
    """A device copy of t whose data starts `elems` elements into its buffer
    (element-aligned, not 16-byte aligned)."""
    buf = torch.empty(t.numel() + elems, dtype=t.dtype, device="cuda")
    v = buf[elems:].view(t.shape)
    v.copy_(t.cuda())
    return v


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_decode_steps_unaligned_bc(dtype):
    """B, C (and B_prev) that are only element-aligned take the element-load
    path of the decode steps: one scan step, one SSD step and one trapezoidal
    step against the oracle, and equal to the same calls on aligned copies."""
    g = torch.Generator().manual_seed(5995)
    cast = torch.float32 if dtype == "f32" else torch.bfloat16
    rnd = lambda *sh: torch.randn(*sh, generator=g).to(cast)
    pos = lambda *sh: (torch.rand(*sh, generator=g) * 0.1 + 1e-3).to(cast)
    b, d, n = 2, 48, 16
    u, dl, z, Bm, Cm = rnd(b, d), pos(b, d), rnd(b, d), rnd(b, 1, n), rnd(b, 1, n)
    A = -torch.rand(d, n, generator=g) - 0.5
    D = torch.randn(d, generator=g)
    S = make_state((b, d, n), seed=5996)
    outs = []
    for mk in (_dev, _offset_copy):
        state = S.cuda().clone()
        y = ssm.scan_step(_dev(u), _dev(dl), _dev(A), mk(Bm), mk(Cm), _dev(D), _dev(z), state=state)
        outs.append((y.float().cpu(), state.cpu()))
    torch.cuda.synchronize()
    yr, hr = oracle.scan_step(u, dl, A, Bm, Cm, D, z, state=S)
    tol = tol_for(dtype)
    assert rel_err(outs[1][0], yr) <= tol and rel_err(outs[1][1], hr) <= tol
    assert torch.equal(outs[0][0], outs[1][0]) and torch.equal(outs[0][1], outs[1][1])
    b, H, P, n = 2, 4, 16, 64
    x, dt, lam, xp = rnd(b, H, P), pos(b, H), torch.rand(b, H, generator=g).to(cast), rnd(b, H, P)
    Bm, Cm, Bp = rnd(b, 1, n), rnd(b, 1, n), rnd(b, 1, n)
    Ah = -torch.rand(H, generator=g) - 0.5
    Dh = torch.randn(H, generator=g)
    S = make_state((b, H, P, n), seed=5997, scale=0.1)
    outs = []
    for mk in (_dev, _offset_copy):
        st1, st2 = S.cuda().clone(), S.cuda().clone()
        y1 = ssm.ssd_step(_dev(x), _dev(dt), _dev(Ah), mk(Bm), mk(Cm), _dev(Dh), None, state=st1)
        y2 = ssm.ssd_trap_step(_dev(x), _dev(dt), _dev(lam), _dev(Ah), mk(Bm), mk(Cm), _dev(Dh), None, state=st2,
                               x_prev=_dev(xp), B_prev=mk(Bp))
        outs.append([t.float().cpu() for t in (y1, st1, y2, st2)])
    torch.cuda.synchronize()
    yr, hr = oracle.ssd_step(x, dt, Ah, Bm, Cm, Dh, None, state=S)
    ytr, htr = oracle.ssd_trap_step(x, dt, lam, Ah, Bm, Cm, Dh, None, state=S, x_prev=xp, B_prev=Bp)
    for got, ref in zip(outs[1], (yr, hr, ytr, htr)):
        assert rel_err(got, ref) <= tol
    for a, b_ in zip(outs[0], outs[1]):
        assert torch.equal(a, b_)


def test_ssd_prefill_then_128_decode_steps():
    """A 64-token chunked prefill leaves its state in a cache; 128 decode steps
    continue from it in place.  Every step's y and the final state match one
    oracle run over all 192 tokens (head dims 32 x 64, dstate 128)."""
    Lp, Ld = 64, 128
    s = SsdShape(1, Lp + Ld, 32, 64, 128, 1, 64, "bf16", dskip="ones", seed=5100)
    inp = make_ssd_inputs(s)
    yr, hr = ref_ssd(inp)
    cache = torch.full((1, 32, 64, 128), float("nan"), dtype=torch.float32, device="cuda")
    pre = {k: (None if v is None else (v[:, :Lp].contiguous() if k in ("x", "dt", "B", "C") else v))
           for k, v in inp.items()}
    y0, _ = ssm.ssd_chunked_fwd(_dev(pre["x"]), _dev(pre["dt"]), _dev(pre["A"]), _dev(pre["B"]),
                                _dev(pre["C"]), _dev(pre["D"]), None, h_last=cache)
    ys = [y0.float().cpu()]
    for t in range(Lp, Lp + Ld):
        tok = {k: inp[k][:, t].contiguous().cuda() for k in ("x", "dt", "B", "C")}
        y = ssm.ssd_step(tok["x"], tok["dt"], _dev(inp["A"]), tok["B"], tok["C"], _dev(inp["D"]), None,
                         state=cache)
        ys.append(y.float().cpu()[:, None])
    torch.cuda.synchronize()
    assert rel_err(torch.cat(ys, dim=1), yr) <= TOL_BF16
    assert rel_err(cache.cpu(), hr) <= TOL_BF16


# ---------------------------------------------------------------------------
# Selective-scan backward
# ---------------------------------------------------------------------------

# Gradients are compared tensor by tensor with the float64 oracle backward,
# max|g - g_ref| / max|g_ref|, against the forward's bars: 1e-5 for float32
# (measured worst case 1.4e-6, on dA, which sums every step of every batch
# row in float32) and 2e-2 with bf16 storage.
TOL_BWD_F32 = 1e-5

BWD_CASES = [
    # (batch, dim, N, L, G, dtype, has_z, dskip, h0, dh_last)
    (1, 16, 16, 16, 1, "f32", False, "none", False, False),
    (2, 40, 16, 100, 1, "f32", True, "normal", True, True),      # ragged channel tile and time tile
    (2, 48, 16, 257, 2, "f32", True, "normal", False, True),     # groups
    (1, 20, 16, 1, 1, "f32", True, "normal", True, True),        # L = 1
    (2, 300, 1, 40, 3, "f32", True, "normal", True, False),
    (2, 70, 4, 65, 2, "f32", False, "normal", True, True),
    (2, 9, 32, 97, 1, "f32", True, "ones", False, True),
    (2, 6, 64, 97, 2, "f32", True, "normal", True, True),
    (2, 50, 16, 257, 1, "bf16", True, "normal", True, True),
    (1, 12, 64, 130, 1, "bf16", False, "normal", False, False),
]


@pytest.mark.parametrize("case", BWD_CASES, ids=lambda c: "b{}d{}n{}l{}g{}_{}_z{}_{}_h0{}_dh{}".format(*c))
def test_scan_backward(case):
    batch, dim, N, L, G, dtype, has_z, dskip, with_h0, with_dhl = case
    s = ScanShape(batch, dim, N, L, G, dtype, has_z=has_z, dskip=dskip, a_kind="loguniform",
                  seed=5200 + zlib.crc32(repr(case).encode()) % 1000)
    inp = make_scan_inputs(s)
    h0 = make_state((batch, dim, N), seed=5300 + N) if with_h0 else None
    dhl = make_state((batch, dim, N), seed=5400 + N) if with_dhl else None
    dy = make_state((batch, dim, L), seed=5500 + L).to(DT[dtype])
    ref = oracle.scan_bwd(inp["u"], inp["delta"], inp["A"], inp["B"], inp["C"], inp["D"], inp["z"], h0, dy, dhl)
    g = ssm.scan_bwd(_dev(inp["u"]), _dev(inp["delta"]), _dev(inp["A"]), _dev(inp["B"]), _dev(inp["C"]),
                     _dev(inp["D"]), _dev(inp["z"]), dy=_dev(dy), h0=_dev(h0), dh_last=_dev(dhl))
    torch.cuda.synchronize()
    tol = TOL_BF16 if dtype == "bf16" else TOL_BWD_F32
    for k in ("du", "ddelta", "dA", "dB", "dC", "dD", "dz", "dh0"):
        if ref[k] is None:
            assert g[k] is None
            continue
        err = rel_err(g[k].float().cpu(), ref[k])
        assert err <= tol, (k, err)


def test_scan_backward_medium_bf16():
    """A larger bf16 case (2 x 256 channels x 1024 steps, gate and D skip):
    dB and dC sum 16 channel tiles of 16 channels per group."""
    s = ScanShape(2, 256, 16, 1024, 1, "bf16", has_z=True, dskip="normal", a_kind="neg_n1", seed=5600)
    inp = make_scan_inputs(s)
    dy = make_state((2, 256, 1024), seed=5601).to(torch.bfloat16)
    ref = oracle.scan_bwd(inp["u"], inp["delta"], inp["A"], inp["B"], inp["C"], inp["D"], inp["z"], None, dy, None)
    g = ssm.scan_bwd(_dev(inp["u"]), _dev(inp["delta"]), _dev(inp["A"]), _dev(inp["B"]), _dev(inp["C"]),
                     _dev(inp["D"]), _dev(inp["z"]), dy=_dev(dy))
    torch.cuda.synchronize()
    for k in ("du", "ddelta", "dA", "dB", "dC", "dD", "dz", "dh0"):
        err = rel_err(g[k].float().cpu(), ref[k])
        assert err <= TOL_BF16, (k, err)


def test_scan_backward_long_prefill_full_size():
    """The long-prefill workload (8 x 1536 channels x 2048 steps, float32,
    gate and D skip) at full size, every gradient against the oracle's
    (about 15 s of oracle time)."""
    s = WORKLOADS["long_prefill_8x1536x2048_f32"]
    inp = make_scan_inputs(s)
    dy = make_state((s.batch, s.dim, s.seqlen), seed=5800)
    dhl = make_state((s.batch, s.dim, s.dstate), seed=5801)
    g = ssm.scan_bwd(_dev(inp["u"]), _dev(inp["delta"]), _dev(inp["A"]), _dev(inp["B"]), _dev(inp["C"]),
                     _dev(inp["D"]), _dev(inp["z"]), dy=_dev(dy), dh_last=_dev(dhl))
    torch.cuda.synchronize()
    g = {k: (None if v is None else v.cpu()) for k, v in g.items()}
    ref = oracle.scan_bwd(inp["u"], inp["delta"], inp["A"], inp["B"], inp["C"], inp["D"], inp["z"], None, dy, dhl)
    for k in ("du", "ddelta", "dA", "dB", "dC", "dD", "dz", "dh0"):
        err = rel_err(g[k], ref[k])
        assert err <= TOL_BWD_F32, (k, err)


def ref_scan_bwd_rows(inp, dy, dh_last=None):
    """The oracle backward over the whole tensor, one host thread per batch row
    (every gradient but dA and dD is per batch row; those two sum over batch
    rows, and the rows' float64 sums are added here)."""
    batch = inp["u"].shape[0]

    def one(b):
        r = _batch_rows(inp, b)
        return oracle.scan_bwd(r["u"], r["delta"], r["A"], r["B"], r["C"], r["D"], r["z"], None,
                               dy[b:b + 1], None if dh_last is None else dh_last[b:b + 1])

    with ThreadPoolExecutor(max_workers=min(batch, 16)) as ex:
        parts = list(ex.map(one, range(batch)))
    out = {}
    for k in ("du", "ddelta", "dB", "dC", "dz", "dh0"):
        out[k] = None if parts[0][k] is None else np.concatenate([p[k] for p in parts])
    for k in ("dA", "dD"):
        out[k] = None if parts[0][k] is None else np.sum([p[k] for p in parts], axis=0)
    return out


def test_scan_backward_large_channel_full_size():
    """The large-channel workload (4 x 5120 channels x 4096 steps, bf16) at
    full size: every gradient (du, ddelta, dz, dA, dB, dC, dD, dh0) over the
    whole tensor against the oracle backward."""
    s = WORKLOADS["large_channel_4x5120x4096_bf16"]
    inp = make_scan_inputs(s)
    dy = make_state((s.batch, s.dim, s.seqlen), seed=5900).to(torch.bfloat16)
    g = ssm.scan_bwd(_dev(inp["u"]), _dev(inp["delta"]), _dev(inp["A"]), _dev(inp["B"]), _dev(inp["C"]),
                     _dev(inp["D"]), _dev(inp["z"]), dy=_dev(dy))
    torch.cuda.synchronize()
    g = {k: (None if v is None else v.cpu()) for k, v in g.items()}
    ref = ref_scan_bwd_rows(inp, dy)
    errs = {}
    for k in ("du", "ddelta", "dA", "dB", "dC", "dD", "dz", "dh0"):
        errs[k] = rel_err(g[k].float(), ref[k])
    print("large_channel_4x5120x4096_bf16 backward: whole-tensor rel err " +
          ", ".join(f"{k} {v:.3e}" for k, v in errs.items()))
    for k, err in errs.items():
        assert err <= TOL_BF16, (k, err)


def test_scan_backward_deterministic():
    """Two calls give bitwise equal gradients: the sums over channel tiles and
    batch rows run in a fixed order."""
    s = ScanShape(3, 96, 16, 300, 2, "f32", has_z=True, dskip="normal", a_kind="loguniform", seed=5650)
    inp = make_scan_inputs(s)
    dy = make_state((3, 96, 300), seed=5651)
    dhl = make_state((3, 96, 16), seed=5652)
    args = [_dev(inp[k]) for k in ("u", "delta", "A", "B", "C", "D", "z")]
    g1 = ssm.scan_bwd(*args, dy=_dev(dy), dh_last=_dev(dhl))
    g2 = ssm.scan_bwd(*args, dy=_dev(dy), dh_last=_dev(dhl))
    torch.cuda.synchronize()
    for k in ("du", "ddelta", "dA", "dB", "dC", "dD", "dz", "dh0"):
        assert torch.equal(g1[k], g2[k]), k


def test_scan_backward_empty_sequence():
    """L = 0: dh0 = dh_last, and dA, dB, dC, dD are all zero (written)."""
    s = ScanShape(2, 40, 16, 0, 1, "f32", has_z=True, dskip="normal", seed=5700)
    inp = make_scan_inputs(s)
    dhl = make_state((2, 40, 16), seed=5701)
    dy = torch.zeros((2, 40, 0))
    g = ssm.scan_bwd(_dev(inp["u"]), _dev(inp["delta"]), _dev(inp["A"]), _dev(inp["B"]), _dev(inp["C"]),
                     _dev(inp["D"]), _dev(inp["z"]), dy=_dev(dy), dh_last=_dev(dhl))
    torch.cuda.synchronize()
    assert torch.equal(g["dh0"].cpu(), dhl)
    assert torch.all(g["dA"] == 0) and torch.all(g["dD"] == 0)


# ---------------------------------------------------------------------------
# Trapezoidal (Mamba-3 SISO) SSD
# ---------------------------------------------------------------------------

TRAP_CASES = [
    # (batch, L, H, N, G, has_z, dskip, h0)
    (1, 64, 1, 128, 1, False, "ones", False),
    (2, 256, 4, 128, 1, False, "ones", True),
    (2, 200, 4, 128, 2, True, "normal", False),    # ragged last chunk: lookahead across chunk ends
    (1, 1, 2, 128, 1, True, "normal", True),       # L = 1
    (3, 130, 3, 64, 1, False, "normal", True),
    (2, 65, 4, 64, 4, True, "none", False),        # one step past a chunk
]


def run_trap(inp, lam, h0=None, out_dtype=None):
    x = _dev(inp["x"])
    out_dt = x.dtype if out_dtype is None else out_dtype
    b, L, H, P = x.shape
    y = torch.full(x.shape, float("nan"), dtype=out_dt, device="cuda")
    h = torch.full((b, H, P, inp["B"].shape[3]), float("nan"), dtype=torch.float32, device="cuda")
    y, h = ssm.ssd_trap_chunked_fwd(x, _dev(inp["dt"]), _dev(lam), _dev(inp["A"]), _dev(inp["B"]),
                                    _dev(inp["C"]), _dev(inp["D"]), _dev(inp["z"]), h0=_dev(h0),
                                    out_dtype=out_dt, y=y, h_last=h)
    torch.cuda.synchronize()
    return y.float().cpu(), h.cpu()


@pytest.mark.parametrize("case", TRAP_CASES, ids=lambda c: "b{}l{}h{}n{}g{}_z{}_{}_h0{}".format(*c))
def test_ssd_trap_small(case):
    batch, L, H, N, G, has_z, dskip, with_h0 = case
    s = SsdShape(batch, L, H, 64, N, G, 64, "bf16", has_z=has_z, dskip=dskip, seed=6000 + L + H)
    inp = make_ssd_inputs(s)
    lam = make_lam((batch, L, H), seed=6100 + L)
    h0 = make_state((batch, H, 64, N), seed=6200 + N, scale=0.5) if with_h0 else None
    y, h = run_trap(inp, lam, h0)
    yr, hr = oracle.ssd_trap(inp["x"], inp["dt"], lam, inp["A"], inp["B"], inp["C"], inp["D"], inp["z"], h0)
    assert rel_err(y, yr) <= TOL_BF16, rel_err(y, yr)
    assert rel_err(h, hr) <= TOL_BF16, rel_err(h, hr)


def test_ssd_trap_lam_one_equals_ssd_bitwise():
    """lam = 1 makes every weight dt: the trapezoidal kernel then computes the
    same values as the plain SSD kernel, bit for bit."""
    s = SsdShape(2, 200, 4, 64, 128, 1, 64, "bf16", has_z=True, dskip="normal", seed=6300)
    inp = make_ssd_inputs(s)
    one = torch.ones((2, 200, 4), dtype=torch.bfloat16)
    a = run_trap(inp, one)
    b = run_ssd(inp)
    assert torch.equal(a[0], b[0]) and torch.equal(a[1], b[1])


def test_ssd_trap_named_workload_full_size():
    """The SSD workload's shapes (batch 32, 256 steps, 32 heads x 64, dstate
    128) with trapezoid weights, against the oracle over the whole y and
    h_last."""
    s = WORKLOADS["ssd_32x256_h32p64n128_bf16"]
    inp = make_ssd_inputs(s)
    lam = make_lam((s.batch, s.seqlen, s.nheads), seed=6400)
    y, h = run_trap(inp, lam)
    yr, hr = oracle.ssd_trap(inp["x"], inp["dt"], lam, inp["A"], inp["B"], inp["C"], inp["D"], inp["z"])
    ey, eh = rel_err(y, yr), rel_err(h, hr)
    print(f"ssd_trap on the SSD workload's shapes: whole-tensor rel err y {ey:.3e}, h_last {eh:.3e}")
    assert ey <= TOL_BF16, ey
    assert eh <= TOL_BF16, eh


@pytest.mark.parametrize("P,N,G,has_z,flags", [(64, 128, 1, False, False), (64, 64, 2, True, False),
                                               (5, 16, 1, True, False), (64, 128, 2, True, True)])
def test_ssd_trap_decode_steps(P, N, G, has_z, flags):
    """Chained ssd_trap_step calls (Eq. 9: alpha h + beta x_prev B_prev +
    gamma x B), each passing the previous token's x and B, from a cached state
    and a given token before the sequence, against one oracle run over the
    same tokens.  flags: raw dt and lam through the fused softplus (with a
    per-head bias) and sigmoid."""
    L, b, H = 10, 2, 4
    s = SsdShape(b, L, H, P, N, G, 64, "bf16", has_z=has_z, dskip="normal", seed=6500 + P + N + G)
    inp = make_ssd_inputs(s)
    lam = make_lam((b, L, H), seed=6501 + N)
    kw, okw = {}, {}
    if flags:
        raw, bias = make_raw_step((b, L, H), H, 6502, "bf16")
        inp["dt"] = raw
        lam = make_state((b, L, H), seed=6503).to(torch.bfloat16)
        kw = dict(dt_softplus=True, dt_bias=bias.cuda(), lam_sigmoid=True)
        okw = dict(dt_softplus=True, dt_bias=bias, lam_sigmoid=True)
    S0 = make_state((b, H, P, N), seed=6504, scale=0.5)
    g = torch.Generator().manual_seed(6505)
    xp0 = torch.randn(b, H, P, generator=g).to(torch.bfloat16)
    bp0 = (torch.randn(b, G, N, generator=g) / N ** 0.5).to(torch.bfloat16)
    yr, hr = oracle.ssd_trap(inp["x"], inp["dt"], lam, inp["A"], inp["B"], inp["C"], inp["D"], inp["z"], S0,
                             x_prev=xp0, B_prev=bp0, **okw)
    state = S0.cuda().clone()
    xp, bp = xp0.cuda(), bp0.cuda()
    ys = []
    for t in range(L):
        tok = {k: (None if inp[k] is None else inp[k][:, t].contiguous().cuda()) for k in ("x", "dt", "z", "B", "C")}
        y = ssm.ssd_trap_step(tok["x"], tok["dt"], lam[:, t].contiguous().cuda(), _dev(inp["A"]), tok["B"],
                              tok["C"], _dev(inp["D"]), tok["z"], state=state, x_prev=xp, B_prev=bp, **kw)
        ys.append(y.float().cpu())
        xp, bp = tok["x"], tok["B"]
    torch.cuda.synchronize()
    assert rel_err(torch.stack(ys, dim=1), yr) <= TOL_BF16, rel_err(torch.stack(ys, dim=1), yr)
    assert rel_err(state.cpu(), hr) <= TOL_BF16, rel_err(state.cpu(), hr)


@pytest.mark.parametrize("batch,H,L1", [(2, 4, 1), (2, 4, 64), (2, 4, 100), (16, 64, 37), (8, 64, 65)])
def test_ssd_trap_split_continuation(batch, H, L1):
    """A trapezoidal sequence in two chunked calls: the second starts from the
    first's h_last (updated in place) and its last token's x and B
    (x_prev, B_prev), and equals one oracle run over the whole sequence (one,
    four and two heads per workgroup)."""
    L, N, G = 130, 128, 2
    s = SsdShape(batch, L, H, 64, N, G, 64, "bf16", has_z=True, dskip="normal", seed=6600 + batch + L1)
    inp = make_ssd_inputs(s)
    lam = make_lam((batch, L, H), seed=6601 + L1)
    h0 = make_state((batch, H, 64, N), seed=6602, scale=0.5)
    yr, hr = oracle.ssd_trap(inp["x"], inp["dt"], lam, inp["A"], inp["B"], inp["C"], inp["D"], inp["z"], h0)
    d = {k: _dev(v) for k, v in inp.items()}
    state = h0.cuda().clone()
    part = lambda t, t0, t1: t[:, t0:t1].contiguous()
    ys = []
    for t0, t1 in ((0, L1), (L1, L)):
        prev = {} if t0 == 0 else dict(x_prev=d["x"][:, t0 - 1].contiguous(), B_prev=d["B"][:, t0 - 1].contiguous())
        y, _ = ssm.ssd_trap_chunked_fwd(part(d["x"], t0, t1), part(d["dt"], t0, t1), part(lam.cuda(), t0, t1),
                                        d["A"], part(d["B"], t0, t1), part(d["C"], t0, t1), d["D"],
                                        part(d["z"], t0, t1), h0=state, h_last=state, **prev)
        ys.append(y.float().cpu())
    torch.cuda.synchronize()
    assert rel_err(torch.cat(ys, dim=1), yr) <= TOL_BF16, rel_err(torch.cat(ys, dim=1), yr)
    assert rel_err(state.cpu(), hr) <= TOL_BF16, rel_err(state.cpu(), hr)


def test_ssd_trap_prefill_then_128_decode_steps():
    """A 64-token trapezoidal chunked prefill leaves its state in a cache; 128
    ssd_trap_step calls continue from it in place, each passing the previous
    token's x and B (the first one the prefill's last token).  Every step's y
    and the final state match one oracle run over all 192 tokens (head dims
    32 x 64, dstate 128)."""
    Lp, Ld = 64, 128
    s = SsdShape(1, Lp + Ld, 32, 64, 128, 1, 64, "bf16", has_z=True, dskip="ones", seed=6700)
    inp = make_ssd_inputs(s)
    lam = make_lam((1, Lp + Ld, 32), seed=6701)
    yr, hr = oracle.ssd_trap(inp["x"], inp["dt"], lam, inp["A"], inp["B"], inp["C"], inp["D"], inp["z"])
    d = {k: _dev(v) for k, v in inp.items()}
    lamd = lam.cuda()
    pre = lambda t: t[:, :Lp].contiguous()
    cache = torch.full((1, 32, 64, 128), float("nan"), dtype=torch.float32, device="cuda")
    y0, _ = ssm.ssd_trap_chunked_fwd(pre(d["x"]), pre(d["dt"]), pre(lamd), d["A"], pre(d["B"]), pre(d["C"]),
                                     d["D"], pre(d["z"]), h_last=cache)
    ys = [y0.float().cpu()]
    for t in range(Lp, Lp + Ld):
        tok = lambda a, tt=t: a[:, tt].contiguous()
        y = ssm.ssd_trap_step(tok(d["x"]), tok(d["dt"]), tok(lamd), d["A"], tok(d["B"]), tok(d["C"]), d["D"],
                              tok(d["z"]), state=cache, x_prev=tok(d["x"], t - 1), B_prev=tok(d["B"], t - 1))
        ys.append(y.float().cpu()[:, None])
    torch.cuda.synchronize()
    got = torch.cat(ys, dim=1)
    print(f"trapezoidal prefill 64 + 128 decode steps: rel err y {rel_err(got, yr):.3e}, "
          f"state {rel_err(cache.cpu(), hr):.3e}")
    assert rel_err(got, yr) <= TOL_BF16
    assert rel_err(cache.cpu(), hr) <= TOL_BF16


# ---------------------------------------------------------------------------
# Fused Phase-0 maps: step = softplus(raw + dt_bias), trapezoid lam = sigmoid(raw)
# ---------------------------------------------------------------------------

PHASE0_SCAN_CASES = [
    # (batch, dim, N, L, G, dtype, n_chunks, with_bias)
    (2, 50, 16, 257, 1, "f32", 1, True),       # sweep, ragged channel and time tiles
    (2, 50, 16, 257, 1, "f32", 3, False),      # chunked carry, no bias
    (2, 48, 16, 100, 2, "bf16", 1, True),
    (2, 50, 16, 264, 1, "bf16", 4, True),      # vector tiles, element tail, chunks
    (2, 70, 4, 65, 2, "f32", 2, True),
    (2, 6, 64, 97, 1, "bf16", 1, True),
]


@pytest.mark.parametrize("case", PHASE0_SCAN_CASES, ids=lambda c: "b{}d{}n{}l{}g{}_{}_k{}_bias{}".format(*c))
def test_scan_dt_softplus(case):
    batch, dim, N, L, G, dtype, k, with_bias = case
    seed = 7000 + zlib.crc32(repr(case).encode()) % 1000
    s = ScanShape(batch, dim, N, L, G, dtype, has_z=True, dskip="normal", a_kind="loguniform", seed=seed)
    inp = make_scan_inputs(s)
    raw, bias = make_raw_step((batch, dim, L), dim, seed + 1, dtype)
    bias = bias if with_bias else None
    h0 = make_state((batch, dim, N), seed=seed + 2)
    inp["delta"] = raw
    y = torch.full((batch, dim, L), float("nan"), dtype=DT[dtype], device="cuda")
    h = torch.full((batch, dim, N), float("nan"), dtype=torch.float32, device="cuda")
    ssm.scan_fwd(*(_dev(inp[k_]) for k_ in ("u", "delta", "A", "B", "C", "D", "z")), h0=_dev(h0), n_chunks=k,
                 y=y, h_last=h, dt_softplus=True, dt_bias=_dev(bias))
    torch.cuda.synchronize()
    yr, hr = oracle.scan(inp["u"], raw, inp["A"], inp["B"], inp["C"], inp["D"], inp["z"], h0,
                         dt_softplus=True, dt_bias=bias)
    tol = tol_for(dtype)
    assert rel_err(y.float().cpu(), yr) <= tol, rel_err(y.float().cpu(), yr)
    assert rel_err(h.cpu(), hr) <= tol, rel_err(h.cpu(), hr)


@pytest.mark.parametrize("trap", [False, True])
def test_ssd_dt_softplus(trap):
    """The SSD (and the trapezoidal SSD with lam = sigmoid(raw lam)) on raw dt
    with a per-head bias, ragged last chunk, groups, gate and h0."""
    batch, L, H, N, G = 2, 200, 4, 128, 2
    s = SsdShape(batch, L, H, 64, N, G, 64, "bf16", has_z=True, dskip="normal", seed=7100 + trap)
    inp = make_ssd_inputs(s)
    raw, bias = make_raw_step((batch, L, H), H, 7110 + trap, "bf16")
    h0 = make_state((batch, H, 64, N), seed=7120, scale=0.5)
    args = [_dev(inp[k]) for k in ("A", "B", "C", "D", "z")]
    if trap:
        lraw = make_state((batch, L, H), seed=7130).to(torch.bfloat16)
        y, h = ssm.ssd_trap_chunked_fwd(_dev(inp["x"]), _dev(raw), _dev(lraw), *args, h0=_dev(h0),
                                        dt_softplus=True, dt_bias=_dev(bias), lam_sigmoid=True)
        yr, hr = oracle.ssd_trap(inp["x"], raw, lraw, inp["A"], inp["B"], inp["C"], inp["D"], inp["z"], h0,
                                 dt_softplus=True, dt_bias=bias, lam_sigmoid=True)
    else:
        y, h = ssm.ssd_chunked_fwd(_dev(inp["x"]), _dev(raw), *args, h0=_dev(h0), dt_softplus=True,
                                   dt_bias=_dev(bias))
        yr, hr = oracle.ssd(inp["x"], raw, inp["A"], inp["B"], inp["C"], inp["D"], inp["z"], h0,
                            dt_softplus=True, dt_bias=bias)
    torch.cuda.synchronize()
    assert rel_err(y.float().cpu(), yr) <= TOL_BF16, rel_err(y.float().cpu(), yr)
    assert rel_err(h.cpu(), hr) <= TOL_BF16, rel_err(h.cpu(), hr)


@pytest.mark.parametrize("trap", [False, True])
def test_ssd_dt_softplus_four_heads_per_workgroup(trap):
    """The Phase-0 maps on the four-heads-per-workgroup path (batch 16 x 64
    heads): each head's bias and, for the trapezoid, sigmoid(raw lam)."""
    batch, L, H, N, G = 16, 100, 64, 128, 2
    s = SsdShape(batch, L, H, 64, N, G, 64, "bf16", has_z=False, dskip="normal", seed=7150 + trap)
    inp = make_ssd_inputs(s)
    raw, bias = make_raw_step((batch, L, H), H, 7160 + trap, "bf16")
    args = [_dev(inp[k]) for k in ("A", "B", "C", "D", "z")]
    if trap:
        lraw = make_state((batch, L, H), seed=7170).to(torch.bfloat16)
        y, h = ssm.ssd_trap_chunked_fwd(_dev(inp["x"]), _dev(raw), _dev(lraw), *args, dt_softplus=True,
                                        dt_bias=_dev(bias), lam_sigmoid=True)
        yr, hr = oracle.ssd_trap(inp["x"], raw, lraw, inp["A"], inp["B"], inp["C"], inp["D"], None, None,
                                 dt_softplus=True, dt_bias=bias, lam_sigmoid=True)
    else:
        y, h = ssm.ssd_chunked_fwd(_dev(inp["x"]), _dev(raw), *args, dt_softplus=True, dt_bias=_dev(bias))
        yr, hr = oracle.ssd(inp["x"], raw, inp["A"], inp["B"], inp["C"], inp["D"], None, None,
                            dt_softplus=True, dt_bias=bias)
    torch.cuda.synchronize()
    assert rel_err(y.float().cpu(), yr) <= TOL_BF16, rel_err(y.float().cpu(), yr)
    assert rel_err(h.cpu(), hr) <= TOL_BF16, rel_err(h.cpu(), hr)


def test_decode_steps_dt_softplus():
    """Scan and SSD decode steps on raw dt with a bias per channel / per head,
    chained over 8 tokens, against the oracle over the same tokens."""
    L = 8
    s = ScanShape(2, 40, 16, L, 1, "f32", has_z=True, dskip="normal", a_kind="loguniform", seed=7200)
    inp = make_scan_inputs(s)
    raw, bias = make_raw_step((2, 40, L), 40, 7201, "f32")
    S0 = make_state((2, 40, 16), seed=7202)
    yr, hr = oracle.scan(inp["u"], raw, inp["A"], inp["B"], inp["C"], inp["D"], inp["z"], S0,
                         dt_softplus=True, dt_bias=bias)
    state, ys = S0.cuda().clone(), []
    for t in range(L):
        tok = {k: inp[k][..., t].contiguous().cuda() for k in ("u", "z", "B", "C")}
        ys.append(ssm.scan_step(tok["u"], raw[..., t].contiguous().cuda(), _dev(inp["A"]), tok["B"], tok["C"],
                                _dev(inp["D"]), tok["z"], state=state, dt_softplus=True,
                                dt_bias=_dev(bias)).cpu())
    torch.cuda.synchronize()
    assert rel_err(torch.stack(ys, dim=-1), yr) <= TOL_F32
    assert rel_err(state.cpu(), hr) <= TOL_F32
    s = SsdShape(2, L, 4, 64, 128, 1, 64, "bf16", has_z=False, dskip="ones", seed=7210)
    inp = make_ssd_inputs(s)
    raw, bias = make_raw_step((2, L, 4), 4, 7211, "bf16")
    S0 = make_state((2, 4, 64, 128), seed=7212, scale=0.5)
    yr, hr = oracle.ssd(inp["x"], raw, inp["A"], inp["B"], inp["C"], inp["D"], None, S0,
                        dt_softplus=True, dt_bias=bias)
    state, ys = S0.cuda().clone(), []
    for t in range(L):
        tok = {k: inp[k][:, t].contiguous().cuda() for k in ("x", "B", "C")}
        ys.append(ssm.ssd_step(tok["x"], raw[:, t].contiguous().cuda(), _dev(inp["A"]), tok["B"], tok["C"],
                               _dev(inp["D"]), None, state=state, dt_softplus=True,
                               dt_bias=_dev(bias)).float().cpu())
    torch.cuda.synchronize()
    assert rel_err(torch.stack(ys, dim=1), yr) <= TOL_BF16
    assert rel_err(state.cpu(), hr) <= TOL_BF16


@pytest.mark.parametrize("dtype,N,with_bias", [("f32", 16, True), ("f32", 4, False), ("bf16", 16, True),
                                               ("f32", 64, True)])
def test_scan_backward_dt_softplus(dtype, N, with_bias):
    """Backward on raw delta: ddelta is the gradient of the raw value (and its
    sum over batch and steps that of dt_bias), every gradient against the
    oracle's chain rule through softplus."""
    batch, dim, L = 2, 40, 100
    seed = 7300 + N + 7 * with_bias + (dtype == "bf16")
    s = ScanShape(batch, dim, N, L, 1, dtype, has_z=True, dskip="normal", a_kind="loguniform", seed=seed)
    inp = make_scan_inputs(s)
    raw, bias = make_raw_step((batch, dim, L), dim, seed + 1, dtype)
    bias = bias if with_bias else None
    h0, dhl = make_state((batch, dim, N), seed=seed + 2), make_state((batch, dim, N), seed=seed + 3)
    dy = make_state((batch, dim, L), seed=seed + 4).to(DT[dtype])
    ref = oracle.scan_bwd(inp["u"], raw, inp["A"], inp["B"], inp["C"], inp["D"], inp["z"], h0, dy, dhl,
                          dt_softplus=True, dt_bias=bias)
    g = ssm.scan_bwd(_dev(inp["u"]), _dev(raw), _dev(inp["A"]), _dev(inp["B"]), _dev(inp["C"]),
                     _dev(inp["D"]), _dev(inp["z"]), dy=_dev(dy), h0=_dev(h0), dh_last=_dev(dhl),
                     dt_softplus=True, dt_bias=_dev(bias))
    torch.cuda.synchronize()
    tol = TOL_BF16 if dtype == "bf16" else TOL_BWD_F32
    for k in ("du", "ddelta", "dA", "dB", "dC", "dD", "dz", "dh0"):
        err = rel_err(g[k].float().cpu(), ref[k])
        assert err <= tol, (k, err)


# ---------------------------------------------------------------------------
# Scalar-decay SSD backward
# ---------------------------------------------------------------------------

SSD_BWD_KEYS = ("dx", "ddt", "dA", "dB", "dC", "dD", "dz", "dh0")

SSD_BWD_CASES = [
    # (batch, L, H, N, G, has_z, dskip, h0, dh_last, dy dtype)
    (1, 64, 1, 128, 1, False, "ones", False, False, "bf16"),
    (2, 203, 4, 128, 2, True, "normal", True, True, "bf16"),   # ragged step tile, groups, gate
    (1, 1, 2, 128, 1, True, "normal", True, True, "bf16"),     # L = 1
    (3, 130, 3, 64, 1, False, "normal", False, True, "f32"),   # dstate 64, float32 dy
    (2, 67, 4, 64, 4, True, "none", True, False, "f32"),       # a group per head
    (2, 97, 8, 128, 2, True, "normal", True, True, "f32"),
    (4, 33, 6, 128, 3, True, "normal", False, True, "bf16"),
]


def _ssd_bwd_pair(inp, dy, h0=None, dhl=None, **kw):
    g = ssm.ssd_bwd(_dev(inp["x"]), _dev(inp["dt"]), _dev(inp["A"]), _dev(inp["B"]), _dev(inp["C"]),
                    _dev(inp["D"]), _dev(inp["z"]), dy=_dev(dy), h0=_dev(h0), dh_last=_dev(dhl),
                    **{k: (_dev(v) if torch.is_tensor(v) else v) for k, v in kw.items()})
    torch.cuda.synchronize()
    return {k: (None if v is None else v.float().cpu()) for k, v in g.items()}


def _check_ssd_bwd(g, ref, label=""):
    errs = {}
    for k in SSD_BWD_KEYS:
        if ref[k] is None:
            assert g[k] is None, k
            continue
        errs[k] = rel_err(g[k], ref[k])
    if label:
        print(f"{label}: whole-tensor rel err " + ", ".join(f"{k} {v:.3e}" for k, v in errs.items()))
    for k, err in errs.items():
        assert err <= TOL_BF16, (k, err)


@pytest.mark.parametrize("case", SSD_BWD_CASES, ids=lambda c: "b{}l{}h{}n{}g{}_z{}_{}_h0{}_dh{}_{}".format(*c))
def test_ssd_backward(case):
    batch, L, H, N, G, has_z, dskip, with_h0, with_dhl, dyt = case
    seed = 8000 + zlib.crc32(repr(case).encode()) % 1000
    s = SsdShape(batch, L, H, 64, N, G, 64, "bf16", has_z=has_z, dskip=dskip, seed=seed)
    inp = make_ssd_inputs(s)
    h0 = make_state((batch, H, 64, N), seed=seed + 1, scale=0.5) if with_h0 else None
    dhl = make_state((batch, H, 64, N), seed=seed + 2, scale=0.5) if with_dhl else None
    dy = make_state((batch, L, H, 64), seed=seed + 3).to(DT[dyt])
    ref = oracle.ssd_bwd(inp["x"], inp["dt"], inp["A"], inp["B"], inp["C"], inp["D"], inp["z"], h0, dy, dhl)
    _check_ssd_bwd(_ssd_bwd_pair(inp, dy, h0, dhl), ref)


def test_ssd_backward_dt_softplus():
    """Raw dt with a per-head bias: ddt is the gradient of the raw value."""
    batch, L, H, N, G = 2, 150, 4, 128, 2
    s = SsdShape(batch, L, H, 64, N, G, 64, "bf16", has_z=True, dskip="normal", seed=8100)
    inp = make_ssd_inputs(s)
    raw, bias = make_raw_step((batch, L, H), H, 8101, "bf16")
    h0 = make_state((batch, H, 64, N), seed=8102, scale=0.5)
    dhl = make_state((batch, H, 64, N), seed=8103, scale=0.5)
    dy = make_state((batch, L, H, 64), seed=8104).to(torch.bfloat16)
    ref = oracle.ssd_bwd(inp["x"], raw, inp["A"], inp["B"], inp["C"], inp["D"], inp["z"], h0, dy, dhl,
                         dt_softplus=True, dt_bias=bias)
    inp = dict(inp, dt=raw)
    _check_ssd_bwd(_ssd_bwd_pair(inp, dy, h0, dhl, dt_softplus=True, dt_bias=bias), ref)


def test_ssd_backward_empty_sequence():
    """L = 0: dh0 = dh_last and dA, dD are zero (written)."""
    s = SsdShape(2, 0, 4, 64, 128, 1, 64, "bf16", has_z=True, dskip="normal", seed=8200)
    inp = make_ssd_inputs(s)
    dhl = make_state((2, 4, 64, 128), seed=8201)
    dy = torch.zeros((2, 0, 4, 64), dtype=torch.bfloat16)
    g = _ssd_bwd_pair(inp, dy, None, dhl)
    assert torch.equal(g["dh0"], dhl)
    assert torch.all(g["dA"] == 0) and torch.all(g["dD"] == 0)


def test_ssd_backward_deterministic():
    s = SsdShape(3, 100, 4, 64, 128, 2, 64, "bf16", has_z=True, dskip="normal", seed=8300)
    inp = make_ssd_inputs(s)
    dy = make_state((3, 100, 4, 64), seed=8301).to(torch.bfloat16)
    dhl = make_state((3, 4, 64, 128), seed=8302)
    a = _ssd_bwd_pair(inp, dy, None, dhl)
    b = _ssd_bwd_pair(inp, dy, None, dhl)
    for k in SSD_BWD_KEYS:
        assert (a[k] is None and b[k] is None) or torch.equal(a[k], b[k]), k


def ref_ssd_bwd_rows(inp, dy, dh_last=None):
    """The oracle SSD backward over the whole tensor, one host thread per batch
    row (dA and dD sum over rows; every other gradient is per row)."""
    batch = inp["x"].shape[0]

    def one(b):
        r = {k: (None if v is None else (v[b:b + 1] if k in ("x", "dt", "B", "C", "z") else v))
             for k, v in inp.items()}
        return oracle.ssd_bwd(r["x"], r["dt"], r["A"], r["B"], r["C"], r["D"], r["z"], None, dy[b:b + 1],
                              None if dh_last is None else dh_last[b:b + 1])

    with ThreadPoolExecutor(max_workers=min(batch, 16)) as ex:
        parts = list(ex.map(one, range(batch)))
    out = {}
    for k in ("dx", "ddt", "dB", "dC", "dz", "dh0"):
        out[k] = None if parts[0][k] is None else np.concatenate([p[k] for p in parts])
    for k in ("dA", "dD"):
        out[k] = None if parts[0][k] is None else np.sum([p[k] for p in parts], axis=0)
    return out


def test_ssd_backward_named_workload_full_size():
    """The SSD workload (batch 32, 256 steps, 32 heads x 64, dstate 128) at
    full size: every gradient over the whole tensor against the oracle."""
    s = WORKLOADS["ssd_32x256_h32p64n128_bf16"]
    inp = make_ssd_inputs(s)
    dy = make_state((s.batch, s.seqlen, s.nheads, s.headdim), seed=8400).to(torch.bfloat16)
    dhl = make_state((s.batch, s.nheads, s.headdim, s.dstate), seed=8401, scale=0.5)
    g = _ssd_bwd_pair(inp, dy, None, dhl)
    _check_ssd_bwd(g, ref_ssd_bwd_rows(inp, dy, dhl), "ssd_32x256_h32p64n128_bf16 backward")


# The chunk kernel sums dB and dC over blocks of 2, 4 or 8 heads of a group
# when the grid has enough workgroups (batch * chunks * nheads / hpw >= 1024).
SSD_BWD_HEAD_BLOCK_CASES = [
    # (batch, L, H, N, G, has_z, h0 and dh_last, dy dtype, dt_softplus)    heads per block
    (16, 130, 64, 128, 2, True, True, "bf16", False),    # 2, groups, ragged last chunk
    (16, 100, 64, 64, 4, False, True, "f32", True),      # 2, dstate 64, raw dt with bias
    (128, 64, 64, 128, 1, True, True, "bf16", False),    # 8, one chunk
    (128, 64, 32, 64, 1, False, False, "f32", False),    # 4, dstate 64
]


@pytest.mark.parametrize("case", SSD_BWD_HEAD_BLOCK_CASES, ids=lambda c: "b{}l{}h{}n{}g{}_z{}_h0{}_{}_sp{}".format(*c))
def test_ssd_backward_head_blocks(case):
    batch, L, H, N, G, has_z, with_h, dyt, softplus = case
    seed = 8500 + zlib.crc32(repr(case).encode()) % 1000
    s = SsdShape(batch, L, H, 64, N, G, 64, "bf16", has_z=has_z, dskip="normal", seed=seed)
    inp = make_ssd_inputs(s)
    h0 = make_state((batch, H, 64, N), seed=seed + 1, scale=0.5) if with_h else None
    dhl = make_state((batch, H, 64, N), seed=seed + 2, scale=0.5) if with_h else None
    dy = make_state((batch, L, H, 64), seed=seed + 3).to(DT[dyt])
    kw = {}
    if softplus:
        raw, bias = make_raw_step((batch, L, H), H, seed + 4, "bf16")
        inp = dict(inp, dt=raw)
        kw = dict(dt_softplus=True, dt_bias=bias)
    g = _ssd_bwd_pair(inp, dy, h0, dhl, **kw)

    def one(b):
        r = {k: (None if v is None else (v[b:b + 1] if k in ("x", "dt", "B", "C", "z") else v)) for k, v in inp.items()}
        return oracle.ssd_bwd(r["x"], r["dt"], r["A"], r["B"], r["C"], r["D"], r["z"],
                              None if h0 is None else h0[b:b + 1], dy[b:b + 1],
                              None if dhl is None else dhl[b:b + 1], **kw)

    with ThreadPoolExecutor(max_workers=16) as ex:
        parts = list(ex.map(one, range(batch)))
    ref = {k: (None if parts[0][k] is None else np.concatenate([q[k] for q in parts]))
           for k in ("dx", "ddt", "dB", "dC", "dz", "dh0")}
    for k in ("dA", "dD"):
        ref[k] = None if parts[0][k] is None else np.sum([q[k] for q in parts], axis=0)
    _check_ssd_bwd(g, ref, "head blocks " + repr(case[:5]))


# ---------------------------------------------------------------------------
# Trapezoidal SSD backward
# ---------------------------------------------------------------------------

TRAP_BWD_KEYS = SSD_BWD_KEYS + ("dlam", "dx_prev", "dB_prev")

TRAP_BWD_CASES = [
    # (batch, L, H, N, G, has_z, h0 and dh_last, previous token, dy dtype, raw dt and lam)
    (1, 64, 1, 128, 1, False, False, False, "bf16", False),
    (2, 203, 4, 128, 2, True, True, True, "bf16", False),     # ragged chunk, groups, gate, previous token
    (1, 1, 2, 128, 1, True, True, True, "f32", False),        # L = 1 with a previous token
    (3, 130, 3, 64, 1, False, False, True, "f32", True),      # dstate 64, softplus and sigmoid
    (2, 67, 4, 64, 4, True, True, False, "bf16", True),
    (16, 130, 64, 128, 2, True, True, True, "bf16", False),   # two heads per block
]


def _trap_bwd_case(case, seed):
    batch, L, H, N, G, has_z, with_h, prev, dyt, raw = case
    s = SsdShape(batch, L, H, 64, N, G, 64, "bf16", has_z=has_z, dskip="normal", seed=seed)
    inp = make_ssd_inputs(s)
    lam = make_lam((batch, L, H), seed=seed + 1)
    kw, okw = {}, {}
    if raw:
        dtr, bias = make_raw_step((batch, L, H), H, seed + 2, "bf16")
        inp = dict(inp, dt=dtr)
        lam = make_state((batch, L, H), seed=seed + 3).to(torch.bfloat16)
        kw = dict(dt_softplus=True, dt_bias=bias, lam_sigmoid=True)
    h0 = make_state((batch, H, 64, N), seed=seed + 4, scale=0.5) if with_h else None
    dhl = make_state((batch, H, 64, N), seed=seed + 5, scale=0.5) if with_h else None
    xp = make_state((batch, H, 64), seed=seed + 6).to(torch.bfloat16) if prev else None
    bp = (make_state((batch, G, N), seed=seed + 7) / math.sqrt(N)).to(torch.bfloat16) if prev else None
    dy = make_state((batch, L, H, 64), seed=seed + 8).to(DT[dyt])
    return inp, lam, h0, dhl, xp, bp, dy, kw


def _trap_bwd_gpu(inp, lam, h0, dhl, xp, bp, dy, kw):
    g = ssm.ssd_trap_bwd(_dev(inp["x"]), _dev(inp["dt"]), _dev(lam), _dev(inp["A"]), _dev(inp["B"]), _dev(inp["C"]),
                         _dev(inp["D"]), _dev(inp["z"]), dy=_dev(dy), h0=_dev(h0), dh_last=_dev(dhl), x_prev=_dev(xp),
                         B_prev=_dev(bp), **{k: (_dev(v) if torch.is_tensor(v) else v) for k, v in kw.items()})
    torch.cuda.synchronize()
    return {k: (None if v is None else v.float().cpu()) for k, v in g.items()}


def _trap_bwd_ref(inp, lam, h0, dhl, xp, bp, dy, kw):
    batch = inp["x"].shape[0]
    sl = lambda t, b: None if t is None else t[b:b + 1]

    def one(b):
        r = {k: (None if v is None else (v[b:b + 1] if k in ("x", "dt", "B", "C", "z") else v)) for k, v in inp.items()}
        return oracle.ssd_trap_bwd(r["x"], r["dt"], sl(lam, b), r["A"], r["B"], r["C"], r["D"], r["z"], sl(h0, b),
                                   sl(xp, b), sl(bp, b), sl(dy, b), sl(dhl, b), **kw)

    with ThreadPoolExecutor(max_workers=min(batch, 16)) as ex:
        parts = list(ex.map(one, range(batch)))
    ref = {k: (None if parts[0][k] is None else np.concatenate([q[k] for q in parts]))
           for k in ("dx", "ddt", "dlam", "dB", "dC", "dz", "dh0", "dx_prev", "dB_prev")}
    for k in ("dA", "dD"):
        ref[k] = None if parts[0][k] is None else np.sum([q[k] for q in parts], axis=0)
    return ref


def _check_trap_bwd(g, ref, label=""):
    errs = {}
    for k in TRAP_BWD_KEYS:
        if ref[k] is None:
            assert g.get(k) is None, k
            continue
        errs[k] = rel_err(g[k], ref[k])
    if label:
        print(f"{label}: whole-tensor rel err " + ", ".join(f"{k} {v:.3e}" for k, v in errs.items()))
    for k, err in errs.items():
        assert err <= TOL_BF16, (k, err)


@pytest.mark.parametrize("case", TRAP_BWD_CASES, ids=lambda c: "b{}l{}h{}n{}g{}_z{}_h{}_prev{}_{}_raw{}".format(*c))
def test_ssd_trap_backward(case):
    args = _trap_bwd_case(case, 8700 + zlib.crc32(repr(case).encode()) % 1000)
    _check_trap_bwd(_trap_bwd_gpu(*args), _trap_bwd_ref(*args), "trapezoidal backward " + repr(case[:5]))


def test_ssd_trap_backward_lam_one_matches_ssd_backward():
    """lam = 1, no previous token: the trapezoidal backward's gradients equal
    the scalar-decay backward's (the kernels take the same products)."""
    s = SsdShape(2, 150, 4, 64, 128, 2, 64, "bf16", has_z=True, dskip="normal", seed=8800)
    inp = make_ssd_inputs(s)
    dy = make_state((2, 150, 4, 64), seed=8801).to(torch.bfloat16)
    dhl = make_state((2, 4, 64, 128), seed=8802, scale=0.5)
    one = torch.ones((2, 150, 4), dtype=torch.bfloat16)
    gt = _trap_bwd_gpu(inp, one, None, dhl, None, None, dy, {})
    gs = _ssd_bwd_pair(inp, dy, None, dhl)
    for k in SSD_BWD_KEYS:
        assert rel_err(gt[k], gs[k].numpy()) <= 1e-5, k


def test_ssd_trap_backward_named_workload_full_size():
    """The trapezoidal SSD on the SSD workload's shapes (batch 32, 256 steps,
    32 heads x 64, dstate 128) with a previous token, every gradient over the
    whole tensor against the oracle."""
    w = WORKLOADS["ssd_32x256_h32p64n128_bf16"]
    inp = make_ssd_inputs(w)
    lam = make_lam((w.batch, w.seqlen, w.nheads), seed=8900)
    xp = make_state((w.batch, w.nheads, w.headdim), seed=8901).to(torch.bfloat16)
    bp = (make_state((w.batch, w.ngroups, w.dstate), seed=8902) / math.sqrt(w.dstate)).to(torch.bfloat16)
    dy = make_state((w.batch, w.seqlen, w.nheads, w.headdim), seed=8903).to(torch.bfloat16)
    dhl = make_state((w.batch, w.nheads, w.headdim, w.dstate), seed=8904, scale=0.5)
    args = (inp, lam, None, dhl, xp, bp, dy, {})
    _check_trap_bwd(_trap_bwd_gpu(*args), _trap_bwd_ref(*args), "ssd_trap_32x256_h32p64n128_bf16 backward")


# ---------------------------------------------------------------------------
# Seeded random sweep over the supported shape space: shapes, group counts,
# dtypes, chunk counts and optional inputs in combinations the hand-picked
# cases above do not list.  The cases are drawn once, from a fixed seed, so
# every run (and every test id) is the same; each is checked against the
# oracle over the whole outputs.
# ---------------------------------------------------------------------------

def _sweep_scan_cases(n=24, seed=20261):
    rng = np.random.default_rng(seed)
    cases = []
    for i in range(n):
        N = int(rng.choice([1, 2, 4, 8, 16, 16, 16, 32, 64]))
        G = int(rng.choice([1, 1, 2, 3]))
        dim = G * int(rng.integers(1, 90))
        L = int(rng.integers(1, 600))
        cases.append((int(rng.integers(1, 4)), dim, N, L, G, str(rng.choice(["f32", "bf16"])),
                      str(rng.choice(["f32", "bf16"])), bool(rng.integers(0, 2)),
                      str(rng.choice(["ones", "normal", "none"])),
                      int(rng.choice([0, 1, 1, 2, 3, max(1, L // 40)])), bool(rng.integers(0, 2)), 7000 + i))
    return cases


@pytest.mark.parametrize("case", _sweep_scan_cases(),
                         ids=lambda c: "b{}d{}n{}l{}g{}_{}to{}_z{}_{}_k{}_h0{}".format(*c[:11]))
def test_scan_random_sweep(case):
    batch, dim, N, L, G, dtype, out, has_z, dskip, k, with_h0, seed = case
    print(f"scan sweep case {case}", flush=True)
    s = ScanShape(batch, dim, N, L, G, dtype, has_z=has_z, dskip=dskip, a_kind="loguniform", seed=seed)
    inp = make_scan_inputs(s)
    h0 = make_state((batch, dim, N), seed + 1, 0.5) if with_h0 else None
    y, h = run_scan(inp, out_dtype=DT[out], n_chunks=k, h0=h0)
    yr, hr = ref_scan(inp, h0=h0)
    tol = tol_for(dtype, out)
    assert rel_err(y, yr) <= tol, (rel_err(y, yr), tol)
    assert rel_err(h, hr) <= tol, (rel_err(h, hr), tol)


def _sweep_ssd_cases(n=16, seed=20262):
    rng = np.random.default_rng(seed)
    cases = []
    for i in range(n):
        G = int(rng.choice([1, 1, 2, 4]))
        H = G * int(rng.choice([1, 1, 2, 3, 4]))
        cases.append((int(rng.integers(1, 4)), int(rng.integers(1, 300)), H, int(rng.choice([64, 128])), G,
                      bool(rng.integers(0, 2)), str(rng.choice(["ones", "normal", "none"])),
                      bool(rng.integers(0, 2)), str(rng.choice(["f32", "bf16"])), bool(rng.integers(0, 2)),
                      8000 + i))
    return cases


@pytest.mark.parametrize("case", _sweep_ssd_cases(),
                         ids=lambda c: "b{}l{}h{}n{}g{}_z{}_{}_h0{}_{}_trap{}".format(*c[:10]))
def test_ssd_random_sweep(case):
    batch, L, H, N, G, has_z, dskip, with_h0, out, trap, seed = case
    print(f"ssd sweep case {case}", flush=True)
    s = SsdShape(batch, L, H, 64, N, G, 64, "bf16", has_z=has_z, dskip=dskip, seed=seed)
    inp = make_ssd_inputs(s)
    h0 = make_state((batch, H, 64, N), seed + 1, 0.5) if with_h0 else None
    if trap:
        lam = make_lam((batch, L, H), seed + 2)
        y, h = run_trap(inp, lam, h0, out_dtype=DT[out])
        yr, hr = oracle.ssd_trap(inp["x"], inp["dt"], lam, inp["A"], inp["B"], inp["C"], inp["D"], inp["z"], h0)
    else:
        y, h = run_ssd(inp, out_dtype=DT[out], h0=h0)
        yr, hr = ref_ssd(inp, h0=h0)
    assert rel_err(y, yr) <= TOL_BF16, rel_err(y, yr)
    assert rel_err(h, hr) <= TOL_BF16, rel_err(h, hr)


def _sweep_scan_bwd_cases(n=12, seed=20264):
    rng = np.random.default_rng(seed)
    cases = []
    for i in range(n):
        N = int(rng.choice([1, 2, 4, 8, 16, 16, 32, 64]))
        G = int(rng.choice([1, 1, 2, 3]))
        cases.append((int(rng.integers(1, 3)), G * int(rng.integers(1, 60)), N, int(rng.integers(1, 300)), G,
                      str(rng.choice(["f32", "bf16"])), bool(rng.integers(0, 2)),
                      str(rng.choice(["ones", "normal", "none"])), bool(rng.integers(0, 2)),
                      bool(rng.integers(0, 2)), 9500 + i))
    return cases


@pytest.mark.parametrize("case", _sweep_scan_bwd_cases(),
                         ids=lambda c: "b{}d{}n{}l{}g{}_{}_z{}_{}_h0{}_dh{}".format(*c[:10]))
def test_scan_backward_random_sweep(case):
    batch, dim, N, L, G, dtype, has_z, dskip, with_h0, with_dhl, seed = case
    print(f"scan backward sweep case {case}", flush=True)
    s = ScanShape(batch, dim, N, L, G, dtype, has_z=has_z, dskip=dskip, a_kind="loguniform", seed=seed)
    inp = make_scan_inputs(s)
    h0 = make_state((batch, dim, N), seed + 1) if with_h0 else None
    dhl = make_state((batch, dim, N), seed + 2) if with_dhl else None
    dy = make_state((batch, dim, L), seed + 3).to(DT[dtype])
    ref = oracle.scan_bwd(inp["u"], inp["delta"], inp["A"], inp["B"], inp["C"], inp["D"], inp["z"], h0, dy, dhl)
    g = ssm.scan_bwd(_dev(inp["u"]), _dev(inp["delta"]), _dev(inp["A"]), _dev(inp["B"]), _dev(inp["C"]),
                     _dev(inp["D"]), _dev(inp["z"]), dy=_dev(dy), h0=_dev(h0), dh_last=_dev(dhl))
    torch.cuda.synchronize()
    tol = TOL_BF16 if dtype == "bf16" else TOL_BWD_F32
    for k in ("du", "ddelta", "dA", "dB", "dC", "dD", "dz", "dh0"):
        if ref[k] is None:
            assert g[k] is None
            continue
        err = rel_err(g[k].float().cpu(), ref[k])
        assert err <= tol, (k, err)


def _sweep_ssd_bwd_cases(n=10, seed=20265):
    rng = np.random.default_rng(seed)
    cases = []
    for i in range(n):
        G = int(rng.choice([1, 1, 2, 4]))
        cases.append((int(rng.integers(1, 4)), int(rng.integers(1, 260)), G * int(rng.choice([1, 2, 3, 4])),
                      int(rng.choice([64, 128])), G, bool(rng.integers(0, 2)), bool(rng.integers(0, 2)),
                      bool(rng.integers(0, 2)), str(rng.choice(["f32", "bf16"])), bool(rng.integers(0, 2)),
                      bool(rng.integers(0, 2)), 9600 + i))
    return cases


def _dA_spread(args, trap, draws=3, seed=0):
    """How far the float64 oracle's dA moves when x, B, C and dy are perturbed
    by up to half a bf16 step (three seeded draws).  dA sums every step's
    log-decay gradient over the batch; where those terms cancel, this spread
    is a sizeable part of dA itself, and no bf16 computation can resolve dA
    more finely."""
    inp, lam, h0, dhl, xp, bp, dy, kw = args
    rng = np.random.default_rng(seed)
    pert = lambda t: torch.from_numpy(t.double().numpy() * (1.0 + rng.uniform(-2.0 ** -9, 2.0 ** -9, tuple(t.shape))))
    ref = None
    out = 0.0
    for k in range(draws + 1):
        q = dict(inp)
        dyq = dy
        if k > 0:
            q["x"], q["B"], q["C"], dyq = pert(inp["x"]), pert(inp["B"]), pert(inp["C"]), pert(dy)
        if trap:
            dA = oracle.ssd_trap_bwd(q["x"], q["dt"], lam, q["A"], q["B"], q["C"], q["D"], q["z"], h0, xp, bp, dyq,
                                     dhl, **kw)["dA"]
        else:
            kw2 = {a: v for a, v in kw.items() if a != "lam_sigmoid"}
            dA = oracle.ssd_bwd(q["x"], q["dt"], q["A"], q["B"], q["C"], q["D"], q["z"], h0, dyq, dhl, **kw2)["dA"]
        dA = np.asarray(dA, dtype=np.float64)
        if ref is None:
            ref = dA
        else:
            out = max(out, float(np.abs(dA - ref).max()))
    return out


@pytest.mark.parametrize("case", _sweep_ssd_bwd_cases(),
                         ids=lambda c: "b{}l{}h{}n{}g{}_z{}_h{}_prev{}_{}_raw{}_trap{}".format(*c[:11]))
def test_ssd_backward_random_sweep(case):
    """Seeded random shapes of the scalar-decay and trapezoidal backwards
    (groups, gate, h0 and dh_last, the previous token, dy dtype, raw dt and
    lam through their maps) against the oracle backward.  Every gradient at
    the usual bar, except dA: one number per head summed over every step,
    whose bar is the larger of 2e-2 of its largest value and twice the spread
    that bf16-resolution perturbations of the inputs cause in the oracle's
    own dA (the kernel also rounds the chunk states to bf16)."""
    batch, L, H, N, G, has_z, with_h, prev, dyt, raw, trap, seed = case
    print(f"ssd backward sweep case {case}", flush=True)
    args = _trap_bwd_case((batch, L, H, N, G, has_z, with_h, prev and trap, dyt, raw), seed)
    inp, lam, h0, dhl, xp, bp, dy, kw = args
    if trap:
        g, ref, keys = _trap_bwd_gpu(*args), _trap_bwd_ref(*args), TRAP_BWD_KEYS
    else:
        kw2 = {k: v for k, v in kw.items() if k != "lam_sigmoid"}
        g = _ssd_bwd_pair(inp, dy, h0, dhl, **kw2)
        ref = oracle.ssd_bwd(inp["x"], inp["dt"], inp["A"], inp["B"], inp["C"], inp["D"], inp["z"], h0, dy, dhl,
                             **kw2)
        keys = SSD_BWD_KEYS
    for k in keys:
        if ref[k] is None:
            assert g.get(k) is None, k
            continue
        err = float(np.abs(np.asarray(g[k], dtype=np.float64) - np.asarray(ref[k], dtype=np.float64)).max())
        scale = float(np.abs(np.asarray(ref[k], dtype=np.float64)).max())
        bar = TOL_BF16 * scale
        if k == "dA":
            bar = max(bar, 2.0 * _dA_spread(args, trap, seed=seed))
        assert err <= bar, (k, err, bar, scale)
