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


def conv_abs_sum(xe, w):
    """sum_j |w[c,j]| |xe[t+j, c]| for every output of a K-tap causal conv over xe = [history(K-1) + tokens, C]."""
    xe = np.abs(np.asarray(xe, dtype=np.float64))
    w = np.abs(np.asarray(w, dtype=np.float64))
    K = w.shape[1]
    T = xe.shape[0] - (K - 1)
    return sum(w[None, :, j] * xe[j:j + T] for j in range(K))


def assert_conv_close(y_gpu, y_ref, s_abs, what=""):
    """bf16 conv output vs the fp64 reference.

    The kernel accumulates K products in fp32 (each fused multiply-add rounds
    once: error <= K * 2^-24 * sum|w x|), applies SiLU in fp32 and rounds once
    to bf16 (<= half a bf16 ulp). Allowed: one bf16 ulp of |ref| plus twice
    the accumulation bound. Near-zero outputs of cancelling sums may differ by
    several bf16 ulps of their own tiny magnitude; that is still inside it.
    """
    y = f64(y_gpu)
    ref = np.asarray(y_ref, dtype=np.float64)
    K = 4
    ulp = np.exp2(np.floor(np.log2(np.maximum(np.abs(ref), 1e-30))) - 7)
    bound = ulp + 2 * K * 2.0 ** -24 * np.asarray(s_abs)
    err = np.abs(y - ref)
    ulps = bf16_ulp_diff(y_gpu, ref)
    print(f"[parity] {what}: max ulps {int(ulps.max())}, flips {float((ulps > 0).float().mean()):.2e}, "
          f"max err/bound {float(np.max(err / bound)):.3f}", flush=True)
    assert np.all(err <= bound), f"{what}: conv output outside the fp32-accumulation + bf16-rounding bound"
