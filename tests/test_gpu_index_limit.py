"""GPU parity of the LoRA linear layer at the largest shape the 32-bit indexing
admits: 64 ceil(M / 64) * max(N, K, 64 ceil(r / 64)) = 2^31 - 4096 elements
(M = 33,554,368 tokens, N = K = r = 64), so that every M-scaled operand (X,
Y, dY, dX, the LoRA planes and split partials) ends just below 2^31 elements.

Y, T and dX are compared on seeded rows spread over the whole range (first
and last rows, the rows around 2^24 where byte offsets pass 2^31); dA and dB, reductions over all
M rows, in full: the oracle's backward is applied to 2^20-row chunks of X and
dY streamed back from the device and the chunk results are summed (dA and dB
are sums over rows). Tolerance as for every linear layer test.
"""

import numpy as np
import pytest
import torch

import bit_nf4_quantized_12_amd as q
import oracle
from bit_nf4_quantized_12_amd import synth
from tests.parity import assert_close, bf16_bits_to_f32, report  # noqa: F401

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def _rows(t, rows):
    # each row copied to the host as its own view (host-side bounds check)
    return np.stack([t[int(i)].cpu().float().numpy() for i in rows])


def test_linear_at_the_32bit_index_limit():
    N = K = r = 64
    M = (1 << 31) // 64 - 64
    s = 16.0 / r
    report(f"index-limit linear: M={M} N={N} K={K} r={r}")
    assert q.qlora_linear_workspace_bytes(M, N, K, r) > 0
    assert q.qlora_linear_workspace_bytes(M + 1, N, K, r) == 0
    Wt, w32 = synth.normal((N, K), 0.02, 0, (190, 0, synth.W_ID))
    At, a = synth.normal((r, K), 0.02, 0, (190, 0, synth.A_ID))
    Bt, b = synth.normal((N, r), 0.02, 0, (190, 0, synth.B_ID))
    X = synth.device_normal_bf16(M * K, 1.0, 191, DEV).view(M, K)
    dY = synth.device_normal_bf16(M * N, 1.0, 192, DEV).view(M, N)
    W = q.quantize_weight(Wt.to(DEV))
    A, B = At.to(DEV), Bt.to(DEV)
    Y, T = q.qlora_linear_fwd(W, X, A, B, s)
    dX, dA, dB = q.qlora_linear_bwd(W, X, A, B, dY, T, s)
    torch.cuda.synchronize()

    pk, c2, c1 = oracle.quantize_nf4_dq(w32.ravel())
    Wo = oracle.bf16_round(oracle.dequant(pk, c2, c1, w32.size)).reshape(N, K)
    rng = np.random.default_rng(193)
    # row 2^24 starts at byte 2^31 of X, Y, dY and dX
    edges = [0, 1, (1 << 24) - 1, 1 << 24, M - 2, M - 1]
    assert max(edges) < M
    rows = np.unique(np.concatenate([edges, rng.choice(M, 248, replace=False)]))
    x = _rows(X, rows)
    dy = _rows(dY, rows)
    Yr, Tr = oracle.linear_fwd(x, Wo, a, b, s)
    assert_close(_rows(Y, rows), Yr, "Y (sampled rows)")
    assert_close(_rows(T, rows), Tr, "T (sampled rows)")
    dXr, _, _ = oracle.linear_bwd(x, Wo, a, b, dy, s)
    assert_close(_rows(dX, rows), dXr, "dX (sampled rows)")

    dAr = np.zeros((r, K))
    dBr = np.zeros((N, r))
    chunk = 1 << 20
    for c0 in range(0, M, chunk):
        c1r = min(M, c0 + chunk)
        xc = X[c0:c1r].cpu().float().numpy()
        dyc = dY[c0:c1r].cpu().float().numpy()
        _, dAc, dBc = oracle.linear_bwd(xc, None, a, b, dyc, s, need_dX=False)
        dAr += dAc
        dBr += dBc
    assert_close(bf16_bits_to_f32(dA), dAr, "dA (all rows)")
    assert_close(bf16_bits_to_f32(dB), dBr, "dB (all rows)")
    del X, dY, Y, T, dX
    torch.cuda.empty_cache()
