"""GPU parity of the adapters' optimizer step (AdamW reading) against the
oracle, with the optimizer state in HBM and paged out to pinned host memory.

Tolerance, derived from the float32 arithmetic (each operation rounded to
nearest, u = 2^-24) and checked per step against the float64 oracle applied
to the GPU's own previous state:
  m, v:  |err| <= 4u (beta |old| + (1 - beta) |g| or g^2)
  p:     |err| <= 2u |p| + 16u lr (weight_decay |p| + (|m_hat| + M) / (sqrt(v_hat) + eps)),
         M = (beta1 |m_old| + (1 - beta1) |g|) / (1 - beta1^step) (the first moment may cancel)
The bf16 copy must be bf16(updated float32 weight) exactly, and the state's
placement must not change any bit.
"""

import numpy as np
import pytest
import torch

import bit_nf4_quantized_12_amd as q
import oracle
from tests.parity import report

pytestmark = pytest.mark.gpu
DEV = "cuda:0"
U = 2.0 ** -24
HP = dict(lr=2e-3, beta1=0.9, beta2=0.999, eps=1e-8, weight_decay=0.01)


def _f32(x):
    return np.float64(np.float32(x))


def _check_step(p0, g, m0, v0, p1, m1, v1, step, hp):
    b1, b2, lr, wd, eps = (_f32(hp[k]) for k in ("beta1", "beta2", "lr", "weight_decay", "eps"))
    pr, mr, vr = oracle.adamw_step(p0, g, m0, v0, step, lr=lr, beta1=b1, beta2=b2, eps=eps, weight_decay=wd)
    assert np.all(np.abs(m1 - mr) <= 4 * U * (b1 * np.abs(m0) + (1 - b1) * np.abs(g)) + 1e-45)
    assert np.all(np.abs(v1 - vr) <= 4 * U * (b2 * np.abs(v0) + (1 - b2) * g * g) + 1e-45)
    mh = mr / (1 - b1 ** step)
    vh = vr / (1 - b2 ** step)
    # the first moment may cancel: its error scales with the magnitudes that enter it
    mmag = (b1 * np.abs(m0) + (1 - b1) * np.abs(g)) / (1 - b1 ** step)
    bound = 2 * U * np.abs(pr) + 16 * U * lr * (wd * np.abs(p0) + (np.abs(mh) + mmag) / (np.sqrt(vh) + eps)) + 1e-45
    assert np.all(np.abs(p1 - pr) <= bound), float(np.max(np.abs(p1 - pr) / bound))


def _bf16_bits(x32):
    return (oracle.bf16_round(x32.astype(np.float32)).view(np.uint32) >> 16).astype(np.uint16)


def _run(n, steps, placement, seed=0, hp=HP):
    report(f"adamw parity: n={n} steps={steps} state={placement}")
    rng = np.random.default_rng(seed)
    p = torch.from_numpy((rng.standard_normal(n) * 0.02).astype(np.float32)).to(DEV)
    p16 = torch.empty(n, dtype=torch.bfloat16, device=DEV)
    if placement == "device":
        m = torch.zeros(n, dtype=torch.float32, device=DEV)
        v = torch.zeros(n, dtype=torch.float32, device=DEV)
    else:
        m = torch.zeros(n, dtype=torch.float32).pin_memory()
        v = torch.zeros(n, dtype=torch.float32).pin_memory()
    history = []
    for step in range(1, steps + 1):
        g32 = (rng.standard_normal(n) * 10.0 ** rng.uniform(-5, -1)).astype(np.float32)
        g = torch.from_numpy(g32).to(torch.bfloat16).to(DEV)
        p0, m0, v0 = p.cpu().numpy().astype(np.float64), m.cpu().numpy().astype(np.float64), v.cpu().numpy().astype(np.float64)
        q.qlora_adamw_step(p, g, m, v, step, p16=p16, **hp)
        torch.cuda.synchronize()
        p1, m1, v1 = p.cpu().numpy(), m.cpu().numpy(), v.cpu().numpy()
        gd = g.float().cpu().numpy().astype(np.float64)
        _check_step(p0, gd, m0, v0, p1.astype(np.float64), m1.astype(np.float64), v1.astype(np.float64), step, hp)
        np.testing.assert_array_equal(p16.cpu().view(torch.int16).numpy().view(np.uint16), _bf16_bits(p1))
        history.append((p1.copy(), m1.copy(), v1.copy()))
    return history


# 1024-parameter boundaries: one workgroup each
@pytest.mark.parametrize("n", [1, 7, 8, 9, 1000, 1023, 1024, 1025, 3 * 1024 + 3, 65536 + 5, 1_000_003])
def test_device_state(n):
    _run(n, 4, "device", seed=n)


@pytest.mark.parametrize("n", [9, 1_000_003])
def test_pinned_host_state_is_bit_identical(n):
    a = _run(n, 3, "device", seed=11)
    b = _run(n, 3, "pinned", seed=11)
    for (pa, ma, va), (pb, mb, vb) in zip(a, b):
        for x, y in ((pa, pb), (ma, mb), (va, vb)):
            np.testing.assert_array_equal(x.view(np.uint32), y.view(np.uint32))


def test_no_weight_decay_and_large_step_count():
    hp = dict(HP, weight_decay=0.0)
    rng = np.random.default_rng(3)
    n = 4099
    p = torch.from_numpy(rng.standard_normal(n).astype(np.float32)).to(DEV)
    m = torch.from_numpy(np.abs(rng.standard_normal(n)).astype(np.float32) * 1e-3).to(DEV)
    v = torch.from_numpy(np.abs(rng.standard_normal(n)).astype(np.float32) * 1e-6).to(DEV)
    g = torch.from_numpy(rng.standard_normal(n).astype(np.float32) * 1e-3).to(torch.bfloat16).to(DEV)
    p0, m0, v0 = (t.cpu().numpy().astype(np.float64) for t in (p, m, v))
    q.qlora_adamw_step(p, g, m, v, 100_000, **hp)
    torch.cuda.synchronize()
    _check_step(p0, g.float().cpu().numpy().astype(np.float64), m0, v0, p.cpu().numpy().astype(np.float64),
                m.cpu().numpy().astype(np.float64), v.cpu().numpy().astype(np.float64), 100_000, hp)


def test_pageable_host_memory_is_refused():
    n = 64
    p = torch.zeros(n, dtype=torch.float32, device=DEV)
    g = torch.zeros(n, dtype=torch.bfloat16, device=DEV)
    m = torch.zeros(n, dtype=torch.float32)              # pageable host memory
    v = torch.zeros(n, dtype=torch.float32, device=DEV)
    lib = q.load_library()
    h = q._AdamWParams(1e-3, 0.9, 0.999, 1e-8, 0.0, 1)
    st = lib.qlora_adamw_step(q._ptr(p), None, q._ptr(g), q._ptr(m), q._ptr(v), n, q.ctypes.byref(h), None)
    assert st == 4  # QLORA_ERR_UNSUPPORTED, nothing launched
    torch.cuda.synchronize()
    assert torch.count_nonzero(p).item() == 0
    # the refused call leaves no error behind for the next call
    mm = torch.zeros(n, dtype=torch.float32, device=DEV)
    q.qlora_adamw_step(p, g, mm, v, 1)
    torch.cuda.synchronize()
