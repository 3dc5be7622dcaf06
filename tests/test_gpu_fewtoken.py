"""GPU checks of the few-token forward (M <= 16): a T launch (T = X A^T) and
a weight-streaming launch that adds s T B^T at its epilogue.

Parity against the float64 oracle at the grouped decoder-layer units the
benchmark times (q/k/v and gate/up of a LLaMA-7B layer, one token and 16),
bit-identical repeats on a reused workspace, and a captured HIP graph of a
chain of calls replayed several times with eager work in between, every
replay equal to the eager result."""

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


@pytest.fixture(scope="module")
def pool():
    with oracle_pool.make_pool() as p:
        yield p


@pytest.mark.parametrize("M", [1, 16])
@pytest.mark.parametrize("g,ns", [(3, 4096), (2, 11008)], ids=["qkv", "gate_up"])
def test_grouped_few_token_units(M, g, ns, pool):
    K, r = 4096, 64
    N = g * ns
    report(f"few-token grouped parity: M={M} g={g} Ns={ns} K={K} r={r}")
    case = synth.linear_case(M, N, K, g * r, seed=11, cfg=172)
    Wt, Xt, At, dYt = (case[k][0].to(DEV) for k in ("W", "X", "A", "dY"))
    w32, x, a, dy = (case[k][1] for k in ("W", "X", "A", "dY"))
    bt, b = synth.normal((N, r), 0.02, 11, (172, 0, synth.B_ID))
    s = 16.0 / r
    W = q.quantize_weight(Wt)
    Y, T = q.qlora_linear_fwd_grouped(W, g, Xt, At, bt.to(DEV), s)
    dX, dA, dB = q.qlora_linear_bwd_grouped(W, g, Xt, At, bt.to(DEV), dYt, None, s)   # T recomputed
    torch.cuda.synchronize()
    pk, c2, c1 = oracle_pool.quantize_parallel(w32.ravel(), pool)
    Wo = oracle.bf16_round(oracle.dequant(pk, c2, c1, w32.size)).reshape(N, K)
    Yr, Tr = oracle.grouped_linear_fwd(x, Wo, a, b, s, g)
    assert_close(bf16_bits_to_f32(Y), Yr, "Y")
    assert_close(T.cpu().numpy(), Tr, "T")
    dXr, dAr, dBr = oracle.grouped_linear_bwd(x, Wo, a, b, dy, s, g)
    assert_close(bf16_bits_to_f32(dX), dXr, "dX")
    assert_close(bf16_bits_to_f32(dA), dAr, "dA")
    assert_close(bf16_bits_to_f32(dB), dBr, "dB")


@pytest.mark.parametrize("M,N,K,r", [(1, 4096, 4096, 64), (16, 11008, 4096, 64), (3, 1000, 8192, 16),
                                     (16, 8192, 22016, 64), (1, 300, 64, 256)])
def test_repeats_identical_on_a_reused_workspace(M, N, K, r):
    report(f"few-token repeats: M={M} N={N} K={K} r={r}")
    case = synth.linear_case(M, N, K, r, seed=12, cfg=173)
    Wt, Xt, At, Bt = (case[k][0].to(DEV) for k in ("W", "X", "A", "B"))
    W = q.quantize_weight(Wt)
    ws = q.new_workspace(q.qlora_linear_workspace_bytes(M, N, K, r), DEV)
    outs = []
    for _ in range(3):
        Y, T = q.qlora_linear_fwd(W, Xt, At, Bt, 0.25, workspace=ws)
        outs.append((Y, T))
    torch.cuda.synchronize()
    for Y, T in outs[1:]:
        assert torch.equal(Y, outs[0][0]) and torch.equal(T, outs[0][1])
    assert torch.isfinite(outs[0][0].float()).all()


def test_graph_replays_match_eager():
    """A chain of few-token calls (three weights, one workspace) captured once
    and replayed three times, with eager calls and synchronisations between the
    replays; each replay's outputs equal the eager ones bit for bit."""
    report("few-token HIP graph replays")
    M, K, r = 1, 4096, 64
    sets = []
    for j, N in enumerate((4096, 11008, 2048)):
        case = synth.linear_case(M, N, K, r, seed=20 + j, cfg=174)
        Wt, Xt, At, Bt = (case[k][0].to(DEV) for k in ("W", "X", "A", "B"))
        sets.append((q.quantize_weight(Wt), At, Bt, torch.empty(M, N, dtype=torch.bfloat16, device=DEV)))
    X = synth.linear_case(M, 64, K, r, seed=30, cfg=174)["X"][0].to(DEV)
    ws = q.new_workspace(max(q.qlora_linear_workspace_bytes(M, W.rows, K, r) for W, _, _, _ in sets), DEV)

    def chain():
        for W, A, B, Y in sets:
            q.qlora_linear_fwd(W, X, A, B, 0.25, save_T=False, Y=Y, workspace=ws)

    chain()
    torch.cuda.synchronize()
    eager = [Y.clone() for _, _, _, Y in sets]
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.stream(s):
        with torch.cuda.graph(graph, stream=s):
            chain()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    for rep in range(3):
        for _, _, _, Y in sets:
            Y.zero_()
        graph.replay()
        torch.cuda.synchronize()
        for (_, _, _, Y), e in zip(sets, eager):
            assert torch.equal(Y, e), f"replay {rep} differs from the eager result"
        chain()          # eager work between the replays
        torch.cuda.synchronize()
