"""GPU parity of the LoRA linear forward and backward against the float64 oracle.

The oracle quantises the same bf16 weight itself (its own codes), dequantises
to W~ = bf16(W^) and evaluates the layer in float64. Outputs must be within
rel-L2 4e-3 and max-abs 2e-2 x RMS (tests/parity.py). Large shapes compare
sampled rows of Y and dX (each an independent set of dot products) and the
full dA, dB.
"""

import numpy as np
import pytest
import torch

import bit_nf4_quantized_12_amd as q
import oracle
from bit_nf4_quantized_12_amd import synth
from tests import oracle_pool
from tests.parity import assert_close, bf16_bits_to_f32, report

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def _oracle_weight(w32, pool=None):
    if pool is not None:
        pk, c2, c1 = oracle_pool.quantize_parallel(w32, pool)
    else:
        pk, c2, c1 = oracle.quantize_nf4_dq(w32)
    return oracle.bf16_round(oracle.dequant(pk, c2, c1, w32.size)).reshape(w32.shape)


@pytest.fixture(scope="module")
def pool():
    with oracle_pool.make_pool() as p:
        yield p


def run_case(M, N, K, r, alpha, seed=0, cfg=100, rows=None, w_dist="normal", backward=True,
             save_T=True, pool=None):
    report(f"linear parity: M={M} N={N} K={K} r={r} alpha={alpha} save_T={save_T}")
    case = synth.linear_case(M, N, K, r, seed=seed, cfg=cfg, w_dist=w_dist)
    s = alpha / r
    Wt, Xt, At, Bt, dYt = (case[k][0].to(DEV) for k in ("W", "X", "A", "B", "dY"))
    w32, x, a, b, dy = (case[k][1] for k in ("W", "X", "A", "B", "dY"))
    W = q.quantize_weight(Wt)
    Y, T = q.qlora_linear_fwd(W, Xt, At, Bt, s, save_T=save_T)
    out = {"Y": Y}
    if backward:
        dX, dA, dB = q.qlora_linear_bwd(W, Xt, At, Bt, dYt, T, s)
        out.update(dX=dX, dA=dA, dB=dB)
    torch.cuda.synchronize()
    got = {k: bf16_bits_to_f32(v) for k, v in out.items()}
    if T is not None:
        got["T"] = T.cpu().numpy()

    Wo = _oracle_weight(w32, pool)
    sel = np.arange(M) if rows is None else np.asarray(rows)
    Yr, Tr = oracle.linear_fwd(x[sel], Wo, a, b, s)
    assert_close(got["Y"][sel], Yr, "Y")
    if T is not None:
        assert_close(got["T"][sel], Tr, "T")
    if backward:
        dXr, _, _ = oracle.linear_bwd(x[sel], Wo, a, b, dy[sel], s)
        assert_close(got["dX"][sel], dXr, "dX")
        _, dAr, dBr = oracle.linear_bwd(x, None, a, b, dy, s, need_dX=False)
        assert_close(got["dA"], dAr, "dA")
        assert_close(got["dB"], dBr, "dB")
    return got


def test_single_linear_256_r8():
    # 256 x 256 weight, 16 tokens, r = 8, alpha = 16 -> s = 2
    run_case(16, 256, 256, 8, 16.0, cfg=1)


@pytest.mark.parametrize("M,N,K,r", [
    (1, 100, 64, 1), (3, 257, 192, 5), (16, 300, 320, 8), (17, 129, 128, 16),
    (130, 200, 384, 33), (256, 512, 512, 64), (70, 1000, 640, 64), (129, 131, 64, 256),
    (200, 96, 1024, 2), (8, 136, 256, 100), (16, 72, 128, 256),
    # few-token T projection with a partial pass of 9..15 tokens
    (11, 260, 448, 24), (13, 520, 1024, 64),
    # more than 8 tokens with a weight whose block constants fill less than 16 bytes (the read-ahead
    # workgroups of the T launch skip that part)
    (9, 3, 64, 2), (16, 1, 64, 1),
    # from 1024 tokens the GEMM runs 512 x 128 tiles: ragged M, N and reductions there too
    (1030, 200, 384, 33), (1500, 1000, 640, 64), (2048, 131, 64, 256), (1100, 96, 1024, 2),
    # input gradient whose last 128-column tile is half past K (quads of lanes whose block lies
    # past the end share a clamped block), with 512 x 128 and 128 x 128 tiles
    (1040, 300, 192, 16), (200, 448, 192, 8),
    # 256 x 256 tiles (under 1024 tokens, at least 192 tiles): forward, then input gradient
    (600, 16640, 256, 16), (600, 256, 16640, 16),
])
def test_ragged_shapes(M, N, K, r):
    run_case(M, N, K, r, 16.0, cfg=101)


@pytest.mark.parametrize("M", [1, 13, 16, 40])
def test_recompute_T_matches_saved_T(M):
    # M <= 16: the few-token projection runs in the forward and in the recompute
    got_saved = run_case(M, 200, 256, 16, 16.0, cfg=102, save_T=True)
    got_none = run_case(M, 200, 256, 16, 16.0, cfg=102, save_T=False)
    for k in ("Y", "dX", "dA", "dB"):
        np.testing.assert_array_equal(got_saved[k], got_none[k])


def test_gemv_agrees_with_gemm_path():
    # M = 16 runs the few-token kernel, M = 17 the tiled GEMM; row 0..15 agree
    case = synth.linear_case(17, 700, 512, 64, cfg=103)
    Wt, Xt, At, Bt = (case[k][0].to(DEV) for k in ("W", "X", "A", "B"))
    W = q.quantize_weight(Wt)
    Y16, _ = q.qlora_linear_fwd(W, Xt[:16].contiguous(), At, Bt, 0.25)
    Y17, _ = q.qlora_linear_fwd(W, Xt, At, Bt, 0.25)
    torch.cuda.synchronize()
    a = bf16_bits_to_f32(Y16)
    b = bf16_bits_to_f32(Y17)[:16]
    assert np.max(np.abs(a - b)) <= 2e-2 * np.sqrt(np.mean(b * b))


def test_backward_is_deterministic():
    case = synth.linear_case(300, 520, 256, 64, cfg=104)
    Wt, Xt, At, Bt, dYt = (case[k][0].to(DEV) for k in ("W", "X", "A", "B", "dY"))
    W = q.quantize_weight(Wt)
    _, T = q.qlora_linear_fwd(W, Xt, At, Bt, 0.25)
    r1 = q.qlora_linear_bwd(W, Xt, At, Bt, dYt, T, 0.25)
    r2 = q.qlora_linear_bwd(W, Xt, At, Bt, dYt, T, 0.25)
    torch.cuda.synchronize()
    for x, y in zip(r1, r2):
        assert torch.equal(x, y)


@pytest.mark.parametrize("M,N,K,r", [
    # few output tiles: the GEMM reduction is split (8 splits of 8 steps, the
    # last of 7; the dX product 4 splits over a ragged 1000-long reduction)
    (300, 1000, 4032, 64),
    # 512 x 128 tiles, 15 of them: 8 splits of 4 steps
    (1100, 520, 2048, 32),
    (512, 4096, 4096, 64),
])
def test_split_reduction_shapes(M, N, K, r):
    rows = None if M <= 300 else np.random.default_rng(M + N).choice(M, 128, replace=False)
    run_case(M, N, K, r, 16.0, cfg=105, rows=rows)


def test_split_reduction_is_deterministic():
    case = synth.linear_case(512, 1000, 4096, 64, cfg=106)
    Wt, Xt, At, Bt, dYt = (case[k][0].to(DEV) for k in ("W", "X", "A", "B", "dY"))
    W = q.quantize_weight(Wt)
    outs = []
    for _ in range(2):
        Y, T = q.qlora_linear_fwd(W, Xt, At, Bt, 0.25)
        outs.append((Y,) + tuple(q.qlora_linear_bwd(W, Xt, At, Bt, dYt, T, 0.25)))
    torch.cuda.synchronize()
    for x, y in zip(*outs):
        assert torch.equal(x, y)


@pytest.mark.parametrize("M", [1, 16, 512])
@pytest.mark.parametrize("N", [4096, 11008])
def test_llama7b_projections_forward(M, N):
    # few-token and small-GEMM regime: forward only
    rows = None if M <= 16 else np.random.default_rng(M).choice(M, 128, replace=False)
    run_case(M, N, 4096, 64, 16.0, cfg=2, rows=rows, backward=False)


@pytest.mark.parametrize("N,K", [(4096, 4096), (11008, 4096), (4096, 11008)])
def test_llama7b_layer_linears_8192_tokens(N, K, pool):
    rows = np.random.default_rng(N + K).choice(8192, 96, replace=False)
    run_case(8192, N, K, 64, 16.0, cfg=3, rows=rows, pool=pool)


@pytest.mark.parametrize("N,K", [(8192, 8192), (22016, 8192), (8192, 22016)])
def test_65b_layer_linears_8192_tokens(N, K, pool):
    # 65B-class layer shapes, weights 0.02 * Student-t(5) (heavy tails stress
    # the block absmax); Y and dX on 256 seeded rows, dA and dB in full
    rows = np.random.default_rng(N + 3 * K).choice(8192, 256, replace=False)
    run_case(8192, N, K, 64, 16.0, cfg=4, rows=rows, w_dist="student_t", pool=pool)


def test_binding_rejects_malformed_buffers():
    # caught in the binding, before anything is launched
    case = synth.linear_case(16, 256, 256, 8, cfg=107)
    Wt, Xt, At, Bt, dYt = (case[k][0].to(DEV) for k in ("W", "X", "A", "B", "dY"))
    W = q.quantize_weight(Wt)
    with pytest.raises(ValueError):
        q.qlora_linear_fwd(W, Xt, At, Bt, 1.0, Y=torch.empty(16, 255, dtype=torch.bfloat16, device=DEV))
    with pytest.raises(ValueError):
        q.qlora_linear_fwd(W._replace(codes=W.codes[:1000]), Xt, At, Bt, 1.0)
    with pytest.raises(ValueError):
        q.qlora_linear_fwd(W._replace(c1=W.c1[:0]), Xt, At, Bt, 1.0)
    with pytest.raises(ValueError):
        q.qlora_linear_bwd(W, Xt, At, Bt, dYt, torch.empty(16, 7, device=DEV), 1.0)
    with pytest.raises(TypeError):
        q.qlora_linear_bwd(W, Xt, At, Bt, dYt, None, 1.0, dA=torch.empty(8, 256, dtype=torch.float32, device=DEV))
    with pytest.raises(ValueError):
        q.qlora_dequant(W.codes, W.c2, W.c1, 256 * 256 + 64)
    with pytest.raises(ValueError):
        q.qlora_merge_lora(W, At, Bt, 1.0, out=torch.empty(256 * 256, dtype=torch.bfloat16, device=DEV))
    Y, _ = q.qlora_linear_fwd(W, Xt, At, Bt, 1.0)  # the well-formed call still runs
    torch.cuda.synchronize()
    assert Y.shape == (16, 256)


@pytest.mark.parametrize("M", [16, 300])
def test_autograd_wrapper_non_contiguous_input(M):
    """LoRALinear4bitFunction on a transposed (non-contiguous) X: the forward
    equals qlora_linear_fwd on the contiguous copy, and the backward (which
    gets the contiguous copy the forward used) equals qlora_linear_bwd."""
    report(f"autograd wrapper: M={M}, X a transposed view")
    case = synth.linear_case(M, 320, 256, 16, cfg=108)
    Wt, Xt, At, Bt, dYt = (case[k][0].to(DEV) for k in ("W", "X", "A", "B", "dY"))
    W = q.quantize_weight(Wt)
    Xv = Xt.t().contiguous().t()              # same values, column-major strides
    assert not Xv.is_contiguous()
    Xv.requires_grad_(True)
    Ag = At.clone().requires_grad_(True)
    Bg = Bt.clone().requires_grad_(True)
    Y = q.LoRALinear4bitFunction.apply(Xv, Ag, Bg, W, 0.5)
    Y.backward(dYt)
    Yr, Tr = q.qlora_linear_fwd(W, Xt, At, Bt, 0.5)
    dXr, dAr, dBr = q.qlora_linear_bwd(W, Xt, At, Bt, dYt, Tr, 0.5)
    torch.cuda.synchronize()
    assert torch.equal(Y, Yr)
    assert torch.equal(Xv.grad, dXr)
    assert torch.equal(Ag.grad, dAr)
    assert torch.equal(Bg.grad, dBr)


@pytest.mark.parametrize("M,N,K,rp,transposed", [
    (1100, 520, 2048, 64, False), (1100, 520, 2048, 192, True), (300, 1000, 640, 128, False),
    (2048, 384, 1024, 64, True)])
def test_matmul_lora_entry_point(M, N, K, rp, transposed):
    """qlora_4bit_matmul_lora: act op(W~) + L R^T against the oracle's base
    product (linear layer with zero adapters) plus the float64 rank term."""
    report(f"matmul_lora: M={M} N={N} K={K} rp={rp} transposed={transposed}")
    kin, nout = (N, K) if transposed else (K, N)
    case = synth.linear_case(M, N, K, 8, cfg=109)
    Wt = case["W"][0].to(DEV)
    w32 = case["W"][1]
    act_t, act = synth.normal((M, kin), 1.0, 0, (109, 1, 3))
    l_t, l64 = synth.normal((M, rp), 0.5, 0, (109, 2, 3))
    r_t, r64 = synth.normal((nout, rp), 0.02, 0, (109, 3, 3))
    W = q.quantize_weight(Wt)
    out = q.qlora_4bit_matmul_lora(W, act_t.to(DEV), l_t.to(DEV), r_t.to(DEV), transposed=transposed)
    torch.cuda.synchronize()
    Wo = _oracle_weight(w32)
    za, zb = np.zeros((8, K)), np.zeros((N, 8))
    if transposed:
        base, _, _ = oracle.linear_bwd(np.zeros((M, K)), Wo, za, zb, act, 0.0)
    else:
        base, _ = oracle.linear_fwd(act, Wo, za, zb, 0.0)
    ref = base + l64.astype(np.float64) @ r64.astype(np.float64).T
    assert_close(bf16_bits_to_f32(out), ref, "out")
