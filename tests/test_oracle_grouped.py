"""Pins of the grouped-linear oracle (linears sharing one input).

The oracle composes the per-segment linear layer; the pins compute the same
quantities a different way: one product with the stacked weight and a
block-diagonal B (scipy's block_diag), and the dB blocks as the diagonal
blocks of the full product s dY^T T.
"""

import numpy as np
import pytest
from scipy.linalg import block_diag

import oracle


@pytest.mark.parametrize("g,ns,K,r,M", [(1, 48, 40, 4, 7), (3, 32, 24, 5, 9), (2, 16, 64, 8, 3)])
def test_grouped_equals_block_diagonal_form(g, ns, K, r, M):
    rng = np.random.default_rng(g * 100 + ns)
    X = rng.standard_normal((M, K))
    W = rng.standard_normal((g * ns, K))
    A = rng.standard_normal((g * r, K))
    B = rng.standard_normal((g * ns, r))
    dY = rng.standard_normal((M, g * ns))
    s = 0.7
    Bd = block_diag(*[B[i * ns:(i + 1) * ns] for i in range(g)])       # [g ns, g r]
    Y, T = oracle.grouped_linear_fwd(X, W, A, B, s, g)
    np.testing.assert_allclose(T, X @ A.T, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(Y, X @ W.T + s * (X @ A.T) @ Bd.T, rtol=1e-12, atol=1e-11)
    dX, dA, dB = oracle.grouped_linear_bwd(X, W, A, B, dY, s, g)
    U = dY @ Bd                                                      # [M, g r]
    np.testing.assert_allclose(dX, dY @ W + s * U @ A, rtol=1e-12, atol=1e-11)
    np.testing.assert_allclose(dA, s * U.T @ X, rtol=1e-12, atol=1e-11)
    full = s * dY.T @ T                                              # [g ns, g r]
    mask = block_diag(*[np.ones((ns, r))] * g)
    np.testing.assert_allclose(dB, (full * mask).reshape(g * ns, g, r).sum(axis=1), rtol=1e-12, atol=1e-11)
    _, dA2, dB2 = oracle.grouped_linear_bwd(X, None, A, B, dY, s, g, need_dX=False)
    np.testing.assert_array_equal(dA2, dA)
    np.testing.assert_array_equal(dB2, dB)
