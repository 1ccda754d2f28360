"""Helpers for the GPU parity tests: host <-> device transfer of bit patterns and
the output tolerance.  No arithmetic of the method lives here."""
import numpy as np
import torch

# GEMM outputs: max |y_gpu - y_ref| <= REL_TOL * RMS(y_ref) over the call's whole output.
REL_TOL = 2e-2


def dev_bf16(bits):
    """uint16 bf16 patterns (numpy) -> torch.bfloat16 tensor on cuda:0."""
    t = torch.from_numpy(np.ascontiguousarray(bits).view(np.int16))
    return t.view(torch.bfloat16).to("cuda:0")


def host_bits16(t):
    return t.detach().contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


def host_u8(t):
    return t.detach().contiguous().cpu().numpy().view(np.uint8)


def host_u32(t):
    return t.detach().contiguous().view(torch.int32).cpu().numpy().view(np.uint32)


def bf16_to_f64(bits):
    return (bits.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def assert_close_rms(y_bits, y_ref, tol=REL_TOL, what=""):
    y = bf16_to_f64(y_bits)
    assert y.shape == y_ref.shape, (y.shape, y_ref.shape)
    rms = float(np.sqrt(np.mean(y_ref ** 2)))
    err = float(np.max(np.abs(y - y_ref))) if y.size else 0.0
    assert np.all(np.isfinite(y)), f"{what}: non-finite output"
    assert err <= tol * rms, f"{what}: max|err| {err:.3e} > {tol} * rms {rms:.3e}"
    return err / rms if rms else 0.0


def announce(msg):
    print(f"[gpu-case] {msg}", flush=True)
