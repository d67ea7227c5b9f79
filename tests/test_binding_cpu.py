"""The Python binding checks caller-given output tensors before any call into
the library (which trusts the sizes it is given): a wrong shape, dtype or
device raises ValueError.  Host tensors suffice; nothing reaches a GPU."""
import pytest
import torch

import state_space_model_ssm_amd as ssm


def test_scan_fwd_rejects_bad_outputs():
    u = torch.zeros(2, 4, 8)
    B = torch.zeros(2, 1, 16, 8)
    A = torch.zeros(4, 16)
    with pytest.raises(ValueError, match="y must be"):
        ssm.scan_fwd(u, u, A, B, B, y=torch.empty(2, 4, 7))
    with pytest.raises(ValueError, match="y must be"):
        ssm.scan_fwd(u, u, A, B, B, y=torch.empty(2, 4, 8, dtype=torch.bfloat16))
    with pytest.raises(ValueError, match="h_last must be"):
        ssm.scan_fwd(u, u, A, B, B, y=torch.empty(2, 4, 8), h_last=torch.empty(2, 4, 8))


def test_ssd_rejects_bad_outputs():
    x = torch.zeros(1, 64, 2, 64, dtype=torch.bfloat16)
    dt = torch.zeros(1, 64, 2, dtype=torch.bfloat16)
    B = torch.zeros(1, 64, 1, 128, dtype=torch.bfloat16)
    A = torch.zeros(2)
    with pytest.raises(ValueError, match="y must be"):
        ssm.ssd_chunked_fwd(x, dt, A, B, B, y=torch.empty(1, 64, 2, 32, dtype=torch.bfloat16))
    with pytest.raises(ValueError, match="h_last must be"):
        ssm.ssd_chunked_fwd(x, dt, A, B, B, h_last=torch.empty(1, 2, 64, 128, dtype=torch.bfloat16))


def test_steps_reject_bad_outputs():
    u = torch.zeros(2, 4)
    B = torch.zeros(2, 1, 16)
    with pytest.raises(ValueError, match="y must be"):
        ssm.scan_step(u, u, torch.zeros(4, 16), B, B, state=torch.zeros(2, 4, 16), y=torch.empty(2, 5))
    x = torch.zeros(2, 3, 8)
    with pytest.raises(ValueError, match="y must be"):
        ssm.ssd_step(x, torch.zeros(2, 3), torch.zeros(3), B, B, state=torch.zeros(2, 3, 8, 16),
                     y=torch.empty(2, 3, 8, dtype=torch.float64))


def test_rope_rejects_bad_outputs():
    dt = torch.zeros(1, 5, 2)
    theta = torch.zeros(1, 5, 1, 8)
    B = torch.zeros(1, 5, 1, 16)
    with pytest.raises(ValueError, match="B_rot must be"):
        ssm.rope_bc(dt, theta, B, B, B_rot=torch.empty(1, 5, 1, 16))
    with pytest.raises(ValueError, match="C_rot must be"):
        ssm.rope_bc(dt, theta, B, B, C_rot=torch.empty(1, 5, 2, 16, dtype=torch.bfloat16))
    with pytest.raises(ValueError, match="angle_last must be"):
        ssm.rope_bc(dt, theta, B, B, angle_last=torch.empty(1, 2, 16))
    with pytest.raises(ValueError, match="angle0 must be"):
        ssm.rope_bc(dt, theta, B, B, angle0=torch.empty(1, 2, 16))


def test_rope_bwd_rejects_bad_arguments():
    dt = torch.zeros(1, 5, 2)
    theta = torch.zeros(1, 5, 1, 8)
    B = torch.zeros(1, 5, 1, 16)
    g = torch.zeros(1, 5, 2, 16)
    with pytest.raises(ValueError, match="dB_rot and dC_rot must be"):
        ssm.rope_bc_bwd(dt, theta, B, B, dB_rot=torch.zeros(1, 5, 1, 16), dC_rot=torch.zeros(1, 5, 1, 16))
    with pytest.raises(TypeError, match="dC_rot must have"):
        ssm.rope_bc_bwd(dt, theta, B, B, dB_rot=g, dC_rot=g.to(torch.bfloat16))
    with pytest.raises(ValueError, match="dangle_last must be"):
        ssm.rope_bc_bwd(dt, theta, B, B, dB_rot=g, dC_rot=g, dangle_last=torch.zeros(1, 2, 16))
    with pytest.raises(ValueError, match="ddt must be"):
        ssm.rope_bc_bwd(dt, theta, B, B, dB_rot=g, dC_rot=g, out={"ddt": torch.empty(1, 5, 3)})
    with pytest.raises(ValueError, match="dB must be"):
        ssm.rope_bc_bwd(dt, theta, B, B, dB_rot=g, dC_rot=g, out={"dB": torch.empty(1, 5, 1, 16, dtype=torch.bfloat16)})
    with pytest.raises(ValueError, match="dtheta must be"):
        ssm.rope_bc_bwd(dt, theta, B, B, dB_rot=g, dC_rot=g, out={"dtheta": torch.empty(1, 5, 2, 8)})
