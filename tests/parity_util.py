"""Shared helpers for GPU parity tests: moving synth inputs to the device and
the parity metrics.  Tolerances (normalised output y: max-abs 2e-2 and
mean-abs 2e-3; pre-norm output: 5e-3 relative Frobenius) are the acceptance
bounds stated for this path."""
import numpy as np

Y_MAX_ABS = 2e-2
Y_MEAN_ABS = 2e-3
O_REL_F = 5e-3


def to_dev(bits, device="cuda"):
    import torch

    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).to(device)


def f32_dev(a, device="cuda"):
    import torch

    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(device)


def metrics(y_gpu, y_ref, o_gpu, o_ref):
    y_gpu = np.asarray(y_gpu, dtype=np.float64)
    o_gpu = np.asarray(o_gpu, dtype=np.float64)
    dy = np.abs(y_gpu - y_ref)
    nref = np.linalg.norm(o_ref)
    rel = np.linalg.norm(o_gpu - o_ref) / nref if nref > 0 else np.linalg.norm(o_gpu)
    return {"y_max_abs": float(dy.max()), "y_mean_abs": float(dy.mean()), "o_rel_f": float(rel)}


def assert_parity(m, what=""):
    assert np.isfinite(list(m.values())).all(), (what, m)
    assert m["y_max_abs"] <= Y_MAX_ABS, (what, m)
    assert m["y_mean_abs"] <= Y_MEAN_ABS, (what, m)
    assert m["o_rel_f"] <= O_REL_F, (what, m)
