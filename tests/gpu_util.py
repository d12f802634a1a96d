"""Helpers shared by the GPU tests: bf16 bit patterns <-> device tensors and
the tolerance checks.  Holds no arithmetic of the MLP itself."""
import numpy as np
import torch

from workload import bf16_bits_to_f64

# spec tolerance per tensor: max|gpu - oracle| <= 1e-2 * max|oracle|
REL_TOL = 1e-2
# absolute floor of the 2-ulp elementwise contract (values below it are
# allowed to flush to zero)
ULP_FLOOR = 2.0 ** -100


def to_dev(bits: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).cuda()


def to_f64(t: torch.Tensor) -> np.ndarray:
    return bf16_bits_to_f64(t.detach().contiguous().view(torch.int16).cpu().numpy().view(np.uint16))


def bits(t: torch.Tensor) -> np.ndarray:
    return t.detach().contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


def rel_err(got: np.ndarray, ref: np.ndarray) -> float:
    scale = float(np.max(np.abs(ref)))
    err = float(np.max(np.abs(got - ref))) if got.size else 0.0
    return err / scale if scale > 0 else err


def assert_close(name, got, ref, tol=REL_TOL):
    assert got.shape == ref.shape, (name, got.shape, ref.shape)
    assert np.all(np.isfinite(got)), f"{name}: non-finite output"
    e = rel_err(got, ref)
    assert e <= tol, f"{name}: max|gpu-oracle|/max|oracle| = {e:.3e} > {tol:g}"
    return e


def ulp_bf16(v: np.ndarray) -> np.ndarray:
    """ulp of bf16 at |v|: 2^(max(floor(log2|v|), -126) - 7)."""
    a = np.abs(np.asarray(v, dtype=np.float64))
    with np.errstate(divide="ignore"):
        e = np.floor(np.log2(np.where(a > 0, a, 1.0)))
    e = np.maximum(e, -126.0)
    return np.exp2(e - 7.0)


def assert_ulp(name, got, ref, n_ulp=2.0):
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    err = np.abs(got - ref)
    small = np.abs(ref) < ULP_FLOOR
    bound = np.where(small, ULP_FLOOR, n_ulp * ulp_bf16(ref))
    bad = ~(err <= bound)
    if np.any(bad):
        i = int(np.flatnonzero(bad.ravel())[0])
        raise AssertionError(f"{name}: {int(bad.sum())} values beyond {n_ulp} bf16 ulp; first at flat index {i}: "
                             f"gpu={got.ravel()[i]!r} oracle={ref.ravel()[i]!r}")
    return float(np.max(np.where(small, 0.0, err / ulp_bf16(ref)))) if ref.size else 0.0
