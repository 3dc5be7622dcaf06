"""Helpers shared by the GPU parity tests (no method arithmetic here)."""

import sys

import numpy as np

# Tolerances for floating-point outputs (Y, dX, dA, dB: bf16 with float32
# accumulation) against the float64 oracle on the same dequantised weights.
REL_L2 = 4e-3
MAX_ABS_OVER_RMS = 2e-2


def report(msg):
    """Name the case on stdout before a GPU step (flushed)."""
    print(msg, flush=True)
    sys.stdout.flush()


def assert_close(got, ref, name):
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    assert got.shape == ref.shape, (name, got.shape, ref.shape)
    assert np.all(np.isfinite(got)), f"{name}: non-finite output"
    err = got - ref
    nref = np.linalg.norm(ref)
    rms = np.sqrt(np.mean(ref * ref))
    if nref == 0:
        assert np.max(np.abs(got)) == 0, name
        return 0.0, 0.0
    rel = np.linalg.norm(err) / nref
    mx = np.max(np.abs(err)) / rms
    assert rel <= REL_L2, f"{name}: rel L2 {rel:.3e} > {REL_L2}"
    assert mx <= MAX_ABS_OVER_RMS, f"{name}: max abs / rms {mx:.3e} > {MAX_ABS_OVER_RMS}"
    return rel, mx


def bf16_bits_to_f32(t):
    """torch bf16 tensor (any device) -> numpy float32 of the same values."""
    import torch
    return t.detach().to("cpu").to(torch.float32).numpy()
