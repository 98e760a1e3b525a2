"""Shared helpers of the GPU parity tests: tolerances and comparisons against the oracle."""
import numpy as np

# Output tolerance: max |gpu - oracle| <= TOL * RMS(oracle output).
# bf16 inputs with fp32 accumulation: 2e-3; fp32 inputs: 1e-5.
TOL = {"bf16": 2e-3, "f32": 1e-5}
# Natural-log sum-exp tolerance (absolute).
LSE_TOL = {"bf16": 1e-4, "f32": 1e-5}


def say(*a):
    print(*a, flush=True)


def check_out(gpu_out, ref_out, dtype, what=""):
    ref = np.asarray(ref_out, dtype=np.float64)
    got = np.asarray(gpu_out, dtype=np.float64)
    assert got.shape == ref.shape, (got.shape, ref.shape)
    assert np.all(np.isfinite(got)), f"{what}: non-finite output"
    rms = float(np.sqrt(np.mean(ref ** 2)))
    err = float(np.max(np.abs(got - ref)))
    assert err <= TOL[dtype] * rms, f"{what}: max err {err:.3e} > {TOL[dtype]} * rms {rms:.3e}"
    return err / rms


def check_lse(gpu_lse, ref_lse, dtype, what=""):
    err = float(np.max(np.abs(np.asarray(gpu_lse, np.float64) - np.asarray(ref_lse, np.float64))))
    assert err <= LSE_TOL[dtype], f"{what}: lse err {err:.3e}"
    return err
