"""Helpers shared by the GPU tests: moving seeded inputs to the device and the
parity criteria (max abs 2e-2 and relative L2 5e-3 on outputs, 1e-4 on
log-normalisers, exact on integers)."""

import numpy as np
import torch

DEV = "cuda"
A_MAX_ABS = 2e-2
A_REL_L2 = 5e-3
L_ABS = 1e-4


def dev_bits(x):
    """bf16 bit patterns (uint16) -> device bfloat16 tensor, same bits."""
    return torch.from_numpy(np.ascontiguousarray(x).view(np.int16)).to(DEV).view(torch.bfloat16)


def dev_f32(x):
    return torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(DEV)


def dev_in(x, dtype):
    return dev_bits(x) if dtype == "bf16" else dev_f32(x)


def host(t):
    return t.detach().cpu().double().numpy()


def check_a(got, want, what=""):
    got = np.asarray(got, dtype=np.float64)
    want = np.asarray(want, dtype=np.float64)
    assert got.shape == want.shape, (what, got.shape, want.shape)
    assert np.all(np.isfinite(got)), f"{what}: non-finite output"
    err = np.abs(got - want).max(initial=0.0)
    nrm = np.linalg.norm(want)
    rel = np.linalg.norm(got - want) / nrm if nrm > 0 else np.linalg.norm(got)
    assert err <= A_MAX_ABS and rel <= A_REL_L2, f"{what}: max abs {err:.3e}, rel L2 {rel:.3e}"
    return err, rel


def check_l(got, want, what=""):
    got = np.asarray(got, dtype=np.float64)
    want = np.asarray(want, dtype=np.float64)
    assert got.shape == want.shape, (what, got.shape, want.shape)
    ninf_w = np.isneginf(want)
    assert np.array_equal(np.isneginf(got), ninf_w), f"{what}: -inf pattern differs"
    if (~ninf_w).any():
        err = np.abs(got[~ninf_w] - want[~ninf_w]).max()
        assert err <= L_ABS, f"{what}: L max abs {err:.3e}"
        return err
    return 0.0
