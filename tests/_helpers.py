"""Shared helpers of the GPU parity tests: host <-> device transfer of the
storage arrays produced by rank_decomposed_linear_amd.workloads, and the
error metric max|got - ref| / max|ref|."""
import numpy as np

from rank_decomposed_linear_amd import workloads as W

TOL = {"f32": 1e-4, "bf16": 2e-2}


def torch_mod():
    import torch
    return torch


def to_dev(a: np.ndarray):
    torch = torch_mod()
    a = np.ascontiguousarray(a)
    if a.dtype == np.uint16:
        return torch.from_numpy(a.view(np.int16)).to("cuda:0").view(torch.bfloat16)
    if a.dtype == np.int32:
        return torch.from_numpy(a).to("cuda:0")
    return torch.from_numpy(a.astype(np.float32)).to("cuda:0")


def to_host(t) -> np.ndarray:
    return t.detach().float().cpu().numpy().astype(np.float64)


def f64(a: np.ndarray) -> np.ndarray:
    return W.decode_array(a).astype(np.float64)


def relerr(got, ref) -> float:
    got, ref = np.asarray(got, np.float64), np.asarray(ref, np.float64)
    assert got.shape == ref.shape, (got.shape, ref.shape)
    assert np.all(np.isfinite(got)), "non-finite output"
    den = float(np.max(np.abs(ref)))
    return float(np.max(np.abs(got - ref))) / (den if den > 0 else 1.0)


def rand(rng, shape, std, dtype):
    return W.random_array(rng, shape, std, dtype)
