"""Shared helpers of the GPU parity tests (no method arithmetic here)."""
import numpy as np
import torch

# Parity bar: max |gpu - oracle| <= TOL * RMS(oracle), per output tensor.
TOL = {"bf16": 2e-3, "f32": 1e-5}


def dev():
    assert torch.cuda.is_available(), "GPU tests need a ROCm device"
    return torch.device("cuda:0")


def f64(t):
    return t.detach().to("cpu", torch.float64).numpy()


def rel_err(gpu, ref):
    gpu = f64(gpu) if isinstance(gpu, torch.Tensor) else np.asarray(gpu, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    rms = float(np.sqrt(np.mean(ref ** 2)))
    err = float(np.max(np.abs(gpu - ref))) if ref.size else 0.0
    return err / rms if rms > 0 else err, err, rms


def assert_close(gpu, ref, tol, what=""):
    r, err, rms = rel_err(gpu, ref)
    print(f"[parity] {what}: max_abs={err:.3e} rms={rms:.3e} ratio={r:.3e} (tol {tol:g})", flush=True)
    assert np.all(np.isfinite(f64(gpu) if isinstance(gpu, torch.Tensor) else gpu)), f"{what}: non-finite output"
    assert r <= tol, f"{what}: max-abs/RMS = {r:.3e} > {tol:g}"


def bf16_ulp_diff(gpu_bf16, ref_f64):
    """Distance in bf16 ulps between a bf16 GPU result and the fp64 reference rounded to bf16."""
    ref_b = torch.from_numpy(np.asarray(ref_f64)).to(torch.float32).to(torch.bfloat16)
    a = gpu_bf16.detach().cpu().contiguous().view(torch.int16).to(torch.int32)
    b = ref_b.contiguous().view(torch.int16).to(torch.int32)
    # map sign-magnitude bf16 bits to a monotone integer line
    a = torch.where(a < 0, -(a & 0x7FFF), a)
    b = torch.where(b < 0, -(b & 0x7FFF), b)
    return (a - b).abs()
