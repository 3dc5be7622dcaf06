"""Helpers shared by the GPU parity tests (no method arithmetic here)."""

import os
import sys

import numpy as np

# Tolerances for floating-point outputs (Y, dX, dA, dB: bf16 with float32
# accumulation) against the float64 oracle on the same dequantised weights:
# relative L2 <= 4e-3, and every element within 2e-2 x RMS of the reference
# plus the output's own bf16 rounding, 2^-8 |ref|. The rounding term is there
# because a bf16 output cannot be closer than half an ulp to the float64
# value: where an output's peak is more than ~5 x its RMS (rank-one outer
# products such as dA at one token; gradients summed over few tokens), the
# correctly rounded result alone exceeds 2e-2 x RMS (a CPU test shows this on
# the oracle's own numbers).
REL_L2 = 4e-3
MAX_ABS_OVER_RMS = 2e-2
BF16_ROUNDING = 2.0 ** -8

# Every floating-point comparison made in this session: (test id, output
# name, rel-L2, max-abs / RMS). conftest.py prints them at the end of the run
# and writes them as JSON, so the margin to the tolerance stays visible.
MARGINS = []


def report(msg):
    """Name the case on stdout before a GPU step (flushed)."""
    print(msg, flush=True)
    sys.stdout.flush()


def assert_close(got, ref, name):
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    assert got.shape == ref.shape, (name, got.shape, ref.shape)
    assert np.all(np.isfinite(got)), f"{name}: non-finite output"
    err = np.abs(got - ref)
    nref = np.linalg.norm(ref)
    rms = np.sqrt(np.mean(ref * ref))
    if nref == 0:
        assert np.max(np.abs(got)) == 0, name
        return 0.0, 0.0
    rel = np.linalg.norm(got - ref) / nref
    mx = np.max(err) / rms
    test = os.environ.get("PYTEST_CURRENT_TEST", "?").split(" ")[0]
    MARGINS.append((test, name, float(rel), float(mx)))
    assert rel <= REL_L2, f"{name}: rel L2 {rel:.3e} > {REL_L2}"
    bound = MAX_ABS_OVER_RMS * rms + BF16_ROUNDING * np.abs(ref)
    worst = np.max(err / bound)
    assert worst <= 1.0, (f"{name}: an element's error is {worst:.3f} x (2e-2 RMS + its bf16 rounding); "
                          f"max abs / rms {mx:.3e}")
    return rel, mx


def bf16_bits_to_f32(t):
    """torch bf16 tensor (any device) -> numpy float32 of the same values."""
    import torch
    return t.detach().to("cpu").to(torch.float32).numpy()
