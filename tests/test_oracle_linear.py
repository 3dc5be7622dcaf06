"""Pins for the oracle's LoRA linear forward and backward.

The layer is x_out = (W_q + B A) x_in ("QLoRA: Efficient Fine-Tuning of
Quantized Language Models", mbrenndoerfer.com, section "Low-Rank Adaptation
(LoRA)"), with tokens as rows and a scale s. Pinned by the merged-weight
identity, exact directional derivatives (the loss <dY, Y> is linear in each
of X, A and B separately) and special cases.
"""

import numpy as np
import pytest

import oracle


def _case(M, N, K, r, seed):
    rng = np.random.default_rng(seed)
    X = rng.standard_normal((M, K))
    W = rng.standard_normal((N, K)) * 0.02
    A = rng.standard_normal((r, K)) * 0.02
    B = rng.standard_normal((N, r)) * 0.02
    dY = rng.standard_normal((M, N))
    return X, W, A, B, dY


def test_merged_weight_identity():
    X, W, A, B, _ = _case(7, 40, 64, 4, 0)
    s = 2.0
    Y, T = oracle.linear_fwd(X, W, A, B, s)
    merged = np.einsum("mk,nk->mn", X, W + s * np.einsum("nj,jk->nk", B, A))
    np.testing.assert_allclose(Y, merged, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(T, np.einsum("mk,jk->mj", X, A), rtol=1e-12, atol=1e-13)


@pytest.mark.parametrize("shape", [(16, 256, 256, 8), (1, 96, 128, 3), (5, 33, 64, 1)])
def test_gradients_are_directional_derivatives(shape):
    M, N, K, r = shape
    X, W, A, B, dY = _case(M, N, K, r, 1)
    s = 0.75
    dX, dA, dB = oracle.linear_bwd(X, W, A, B, dY, s)
    loss = lambda X_, A_, B_: float(np.sum(dY * oracle.linear_fwd(X_, W, A_, B_, s)[0]))  # noqa: E731
    base = loss(X, A, B)
    rng = np.random.default_rng(2)
    for _ in range(3):
        VX, VA, VB = rng.standard_normal(X.shape), rng.standard_normal(A.shape), rng.standard_normal(B.shape)
        # L is linear in each argument on its own, so a unit step is exact
        assert abs((loss(X + VX, A, B) - base) - np.sum(dX * VX)) <= 1e-9 * (1 + abs(base))
        assert abs((loss(X, A + VA, B) - base) - np.sum(dA * VA)) <= 1e-9 * (1 + abs(base))
        assert abs((loss(X, A, B + VB) - base) - np.sum(dB * VB)) <= 1e-9 * (1 + abs(base))
    assert dX.shape == X.shape and dA.shape == A.shape and dB.shape == B.shape


def test_special_cases():
    X, W, A, B, dY = _case(6, 20, 64, 4, 3)
    Y, _ = oracle.linear_fwd(X, W, A, np.zeros_like(B), 1.0)
    np.testing.assert_allclose(Y, X @ W.T, rtol=1e-13, atol=1e-13)
    dX, dA, dB = oracle.linear_bwd(X, W, A, np.zeros_like(B), dY, 1.0)
    assert np.all(dA == 0)
    dX, dA, dB = oracle.linear_bwd(X, W, np.zeros_like(A), B, dY, 1.0)
    assert np.all(dB == 0)
    dX, dA, dB = oracle.linear_bwd(X, W, A, B, dY, 0.0)
    assert np.all(dA == 0) and np.all(dB == 0)
    np.testing.assert_allclose(dX, dY @ W, rtol=1e-13, atol=1e-13)


def test_single_token_is_dot_products():
    X, W, A, B, dY = _case(1, 9, 64, 2, 4)
    s = 0.25
    Y, T = oracle.linear_fwd(X, W, A, B, s)
    for n in range(9):
        t = [sum(X[0, k] * A[j, k] for k in range(64)) for j in range(2)]
        ref = sum(X[0, k] * W[n, k] for k in range(64)) + s * sum(t[j] * B[n, j] for j in range(2))
        assert abs(Y[0, n] - ref) <= 1e-13


def test_merged_weight_reproduces_the_adapted_layer():
    # the layer rule x_out = (W + s B A) x_in: the merged weight without adapters
    # gives the same output as the frozen weight with them
    rng = np.random.default_rng(42)
    M, N, K, r, s = 9, 33, 70, 6, 0.375
    X, W = rng.standard_normal((M, K)), rng.standard_normal((N, K))
    A, B = rng.standard_normal((r, K)), rng.standard_normal((N, r))
    Wm = oracle.merge_lora(W, A, B, s)
    Y_adapted, _ = oracle.linear_fwd(X, W, A, B, s)
    Y_merged, _ = oracle.linear_fwd(X, Wm, np.zeros((r, K)), np.zeros((N, r)), s)
    np.testing.assert_allclose(Y_merged, Y_adapted, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(oracle.merge_lora(W, A, B, 0.0), W, rtol=0, atol=0)


@pytest.mark.parametrize("M", [1, 16])
def test_plain_max_abs_bound_is_unattainable_for_peaked_bf16_outputs(M):
    """Why the GPU parity tests add each element's own bf16 rounding to the
    2e-2 x RMS budget: dA = s U^T X over few tokens has a peak of more than
    2e-2 / 2^-8 = 5.12 times its RMS, so rounding its largest elements to bf16
    (up to 2^-8 relative, a full ulp ~2^-7 when a float32 value next to a tie
    rounds the other way) can exceed 2e-2 x RMS. At one token (a rank-one
    product) even the correctly rounded oracle value does. Shapes: the q/k/v
    unit of a LLaMA-7B layer (K = 4096, rank 3 x 64), inputs like the tests'."""
    rng = np.random.default_rng(7)
    K, N, r = 4096, 3 * 4096, 192
    X = rng.standard_normal((M, K))
    A = rng.standard_normal((r, K)) * 0.02
    B = rng.standard_normal((N, r)) * 0.02
    dY = rng.standard_normal((M, N))
    _, dA, _ = oracle.linear_bwd(X, None, A, B, dY, 0.25, need_dX=False)
    rms = np.sqrt(np.mean(dA * dA))
    assert np.max(np.abs(dA)) / rms > 2e-2 / 2.0 ** -8
    # (the float32 step is exact to 2^-24, far below the bf16 step)
    rounded = oracle.bf16_round(dA.astype(np.float32)).astype(np.float64)
    assert np.all(np.abs(rounded - dA) <= 2.0 ** -8 * np.abs(dA) * (1 + 1e-6))
    if M == 1:
        assert np.max(np.abs(rounded - dA)) / rms > 2e-2
