"""GPU parity of the merged deployment weight bf16(W^ + s B A) against the
float64 oracle. The kernel rounds once to bf16 from a float32 value whose
error is at most (r + 2) u (|W^| + s sum_j |B A|), u = 2^-24; the output must
equal bf16(exact) wherever the exact value is farther than that from a bf16
rounding boundary, and be within one bf16 step everywhere."""

import numpy as np
import pytest
import torch

import bit_nf4_quantized_12_amd as q
import oracle
from bit_nf4_quantized_12_amd import synth
from tests.parity import report

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def _check(N, K, r, cb, dq, seed):
    report(f"merge parity: N={N} K={K} r={r} {cb} dq={dq}")
    tw, w32 = synth.normal((N, K), 0.02, seed, (180, 0, synth.W_ID))
    ta, a = synth.normal((r, K), 0.02, seed, (180, 0, synth.A_ID))
    tb, b = synth.normal((N, r), 0.02, seed, (180, 0, synth.B_ID))
    s = 16.0 / r
    W = q.quantize_weight(tw.to(DEV), codebook=cb, double_quant=dq)
    out = q.qlora_merge_lora(W, ta.to(DEV), tb.to(DEV), s)
    torch.cuda.synchronize()
    got = out.cpu().float().numpy().astype(np.float64)
    lv = oracle.codebook_levels(cb)
    if dq:
        pk, c2, c1 = oracle.quantize_nf4_dq(w32.ravel(), levels=lv)
        What = oracle.dequant(pk, c2, c1, w32.size, levels=lv).reshape(N, K)
    else:
        pk, am = oracle.quantize_blockwise(w32.ravel(), lv)
        What = oracle.dequant_blockwise(pk, am, w32.size, lv).reshape(N, K)
    ref = oracle.merge_lora(What, a, b, s)
    eps = (r + 2) * 2.0 ** -24 * (np.abs(What) + s * (np.abs(b) @ np.abs(a)))
    rounded = oracle.bf16_round(ref.astype(np.float32)).astype(np.float64)
    # bf16 steps around `rounded` (8 significant bits): above it 2^(e-8) for
    # |rounded| = m 2^e, m in [0.5, 1); below it half that at a power of two
    m, e = np.frexp(np.abs(rounded))
    up = np.ldexp(1.0, e - 8)
    down = np.where(m == 0.5, up / 2, up)
    sgn = np.where(rounded < 0, -1.0, 1.0)
    b_out = rounded + sgn * up / 2          # rounding boundary away from zero
    b_in = rounded - sgn * down / 2         # rounding boundary toward zero
    margin = np.minimum(np.abs(ref - b_out), np.abs(ref - b_in))
    clear = margin > eps + np.abs(ref) * 2.0 ** -24
    assert clear.mean() > 0.9  # most elements are checked for exact equality
    np.testing.assert_array_equal(got[clear], rounded[clear])
    assert np.all(np.abs(got - ref) <= up + eps)


@pytest.mark.parametrize("N,K,r", [(256, 256, 8), (300, 520, 33), (4096, 4096, 64), (100, 64, 256)])
def test_merge_nf4_dq(N, K, r):
    _check(N, K, r, "nf4", True, seed=N)


# K % 64 == 0 runs the MFMA form (64 x 256 tiles, 64-deep rank chunks): ragged
# rows and columns, odd ranks, a partial last rank chunk, K = 11008
@pytest.mark.parametrize("N,K,r", [(300, 576, 33), (130, 11008, 100), (64, 320, 200), (17, 64, 1)])
def test_merge_mfma_tiles(N, K, r):
    _check(N, K, r, "nf4", True, seed=N + r)


@pytest.mark.parametrize("cb,dq", [("int4", False), ("fp4", True), ("nf4", False)])
def test_merge_other_formats(cb, dq):
    _check(384, 1024, 64, cb, dq, seed=7)


def test_merged_weight_serves_the_adapted_layer():
    # Y from the merged dense weight matches Y of the LoRA layer (same tolerance as the layer)
    from tests.parity import assert_close, bf16_bits_to_f32
    M, N, K, r = 64, 512, 768, 16
    case = synth.linear_case(M, N, K, r, seed=3, cfg=181)
    Wt, Xt, At, Bt = (case[k][0].to(DEV) for k in ("W", "X", "A", "B"))
    s = 2.0
    W = q.quantize_weight(Wt)
    Y, _ = q.qlora_linear_fwd(W, Xt, At, Bt, s)
    Wm = q.qlora_merge_lora(W, At, Bt, s)
    Ym = (Xt.float() @ Wm.float().t())
    torch.cuda.synchronize()
    assert_close(bf16_bits_to_f32(Y), Ym.cpu().numpy().astype(np.float64), "Y via merged weight")
