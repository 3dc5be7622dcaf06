"""Oracle for NF4 quantisation, double quantisation and the LoRA linear layer.

TEST INFRASTRUCTURE ONLY -- see the package docstring. Written from these pages:

* "QLoRA: Efficient Finetuning of Quantized LLMs" (inquiringlines.com paper
  text), section "Method": the storage / compute data types, the paragraph
  "4-bit NormalFloat Quantization" and the paragraph "Double Quantization".
* "QLoRA: Efficient Fine-Tuning of Quantized Language Models"
  (mbrenndoerfer.com), sections "Double Quantization" and "Low-Rank
  Adaptation (LoRA)" (the forward rule x_out = (W_q + BA) x_in).
* "Efficient Language Model Fine-Tuning with QLoRA on Resource-Constrained
  Hardware" (marciocunha.net): the LoraConfig fields r and lora_alpha.

Where the pages are silent the reading taken is stated at the point of use.
"""

import math

import numpy as np

# Block of 64 weights per absmax constant: "Double Quantization" paragraph,
# which prices 32-bit constants at a blocksize of 64 for W.
NF4_BLOCK = 64
# Second-level block: 256 first-level constants share one fp32 constant.
# The pages only motivate double quantisation; the block of 256 with an 8-bit
# float second level is the workload's stated configuration.
DQ_BLOCK = 256

# Tail probability used for the outermost quantile. The pages give the
# construction but garble the formula and omit the table (their Appendix E),
# so this is a READING: the mean of the centre probabilities of the outermost
# bin for 16 and for 15 equal-mass bins, 1 - (1/32 + 1/30)/2.
DELTA = 1.0 - 0.5 * (1.0 / 32.0 + 1.0 / 30.0)


# ---------------------------------------------------------------------------
# Levels: "4-bit NormalFloat Quantization" paragraph, steps (1) and (2) and
# the asymmetric construction with one shared zero.
# ---------------------------------------------------------------------------

def _phi(x):
    """Standard normal CDF, written with the complementary error function."""
    return 0.5 * math.erfc(-x / math.sqrt(2.0))


def phi_inv(p):
    """Inverse standard normal CDF for p in [0.5, 1), by bisection on _phi.

    Bisection runs until the bracket is two adjacent doubles; the endpoint
    whose CDF is closer to p is returned.
    """
    if not (0.5 <= p < 1.0):
        raise ValueError("phi_inv is only needed on [0.5, 1)")
    if p == 0.5:
        return 0.0
    lo, hi = 0.0, 40.0
    while True:
        mid = 0.5 * (lo + hi)
        if mid == lo or mid == hi:
            break
        if _phi(mid) < p:
            lo = mid
        else:
            hi = mid
    return lo if abs(_phi(lo) - p) <= abs(_phi(hi) - p) else hi


def nf4_levels_f64(delta=DELTA):
    """The 16 NF4 values in float64, ascending.

    Quantiles of N(0, 1): 2^(k-1) + 1 = 9 for the positive side (probabilities
    1/2 + j (delta - 1/2) / 8, j = 0..8) and 2^(k-1) = 8 for the negative side
    (1/2 + j (delta - 1/2) / 7, j = 0..7, negated). Both sets contain zero;
    one zero is dropped, giving 2^k = 16 values, which are divided by the
    largest magnitude Phi^-1(delta) so that the range is exactly [-1, 1].
    """
    positive = [phi_inv(0.5 + j * (delta - 0.5) / 8.0) for j in range(9)]
    negative = [-phi_inv(0.5 + j * (delta - 0.5) / 7.0) for j in range(8)]
    union = positive + negative[1:]  # negative[0] is the second zero
    assert len(union) == 16
    top = phi_inv(delta)
    return np.array(sorted(v / top for v in union), dtype=np.float64)


def nf4_levels(delta=DELTA):
    """The NF4 values rounded (to nearest even) to float32, code 0 .. 15."""
    return nf4_levels_f64(delta).astype(np.float32)


# ---------------------------------------------------------------------------
# 8-bit float for the second-level constants (OCP FP8 E4M3, "FN" variant:
# bias 7, no infinities, 0x7F / 0xFF are NaN, largest finite 448).
# ---------------------------------------------------------------------------

def e4m3_decode(code):
    """Value of each E4M3 byte, as float64 (exact)."""
    code = np.asarray(code, dtype=np.int64)
    sign = (code >> 7) & 1
    e = (code >> 3) & 0xF
    m = code & 0x7
    mag = np.where(e == 0, m * 2.0 ** -9, (1.0 + m / 8.0) * np.exp2(e - 7.0))
    mag = np.where((e == 15) & (m == 7), np.nan, mag)
    return np.where(sign == 1, -mag, mag)


_E4M3_POS_CODES = np.arange(0, 0x7F, dtype=np.int64)       # 0x00 .. 0x7E
_E4M3_POS_VALUES = e4m3_decode(_E4M3_POS_CODES)


def e4m3_encode_rne(x):
    """Nearest non-negative finite E4M3 byte to each x >= 0, ties to even code.

    Brute force over all 127 non-negative finite codes: the distance to every
    code is computed and the closest wins; of two equally close codes the one
    with an even last mantissa bit (an even byte) wins.
    """
    x = np.asarray(x, dtype=np.float64).ravel()
    if np.any(~np.isfinite(x)) or np.any(x < 0) or np.any(x > 448.0):
        raise ValueError("e4m3_encode_rne takes finite values in [0, 448]")
    out = np.empty(x.shape, dtype=np.uint8)
    chunk = 1 << 16
    for start in range(0, x.size, chunk):
        xs = x[start:start + chunk]
        d = np.abs(xs[:, None] - _E4M3_POS_VALUES[None, :])
        best = d.min(axis=1, keepdims=True)
        tied = d == best
        even = tied & ((_E4M3_POS_CODES[None, :] & 1) == 0)
        pick = np.where(even.any(axis=1), even.argmax(axis=1), tied.argmax(axis=1))
        out[start:start + chunk] = _E4M3_POS_CODES[pick]
    return out


# ---------------------------------------------------------------------------
# bfloat16: "QLORA has one low-precision storage data type ... and one
# computation data type that is usually BFloat16" ("Method" paragraph).
# ---------------------------------------------------------------------------

def bf16_round(x):
    """Round float32 values to the nearest bfloat16 (ties to even), as float32.

    On the sign-magnitude bit pattern: keep the top 16 bits, and step the
    magnitude up by one bfloat16 ulp when the dropped 16 bits exceed half an
    ulp, or equal it and the kept last bit is odd.
    """
    x = np.ascontiguousarray(x, dtype=np.float32)
    if not np.all(np.isfinite(x)):
        raise ValueError("bf16_round takes finite values")
    bits = x.view(np.uint32).astype(np.uint64)
    kept = bits & 0xFFFF0000
    dropped = bits & 0xFFFF
    odd = (kept >> 16) & 1
    up = (dropped > 0x8000) | ((dropped == 0x8000) & (odd == 1))
    out = np.where(up, kept + 0x10000, kept).astype(np.uint32)
    return out.view(np.float32).reshape(x.shape)


# ---------------------------------------------------------------------------
# Quantisation: "4-bit NormalFloat Quantization" step (3) (absmax rescaling
# into [-1, 1], then "quantize as usual" = nearest value of the data type) and
# "Double Quantization" (the absmax constants are themselves quantised).
# ---------------------------------------------------------------------------

def _codes_for_blocks(blocks, levels):
    """Codes of a (nblocks, 64) float32 array of bf16 weights.

    c_b = max |w| over the block (exact in float32). x = w / c_b in IEEE
    float32 (round to nearest even). code = index of the nearest level,
    measured in float64, the lower index on a tie. An all-zero block gets the
    code of the exact zero (7) everywhere.
    """
    absmax = np.max(np.abs(blocks), axis=1)
    safe = np.where(absmax > 0, absmax, np.float32(1.0)).astype(np.float32)
    x = (blocks / safe[:, None]).astype(np.float32)  # float32 / float32: IEEE RNE
    q = levels.astype(np.float64)
    dist = np.abs(x.astype(np.float64)[..., None] - q)
    codes = np.argmin(dist, axis=-1).astype(np.uint8)  # first minimum = lower index
    zero_code = np.uint8(int(np.flatnonzero(levels == 0.0)[0]))
    codes[absmax == 0] = zero_code
    return codes, absmax.astype(np.float32)


def quantize_nf4_dq(w, levels=None):
    """NF4 + double quantisation of a flat array of bf16 values.

    ``w``: float32 array holding bfloat16 values (any shape; flattened in C
    order). Returns ``(packed, c2, c1)``:

    * packed: uint8[ceil(n/2)], element 2i in the low nibble of byte i and
      element 2i+1 in the high nibble (a pad nibble of 0 when n is odd);
    * c2: uint8[ceil(n/64)], E4M3 code of c_b / c1_g;
    * c1: float32[ceil(ceil(n/64)/256)], the largest c_b of each group of 256
      consecutive blocks.

    The codes use the exact per-block absmax; only the stored constants are
    double quantised. A final block or group may be short.
    """
    if levels is None:
        levels = nf4_levels()
    w = np.ascontiguousarray(w, dtype=np.float32).ravel()
    if not np.all(np.isfinite(w)):
        raise ValueError("weights must be finite")
    n = w.size
    if n == 0:
        raise ValueError("empty input")
    nb = -(-n // NF4_BLOCK)
    ng = -(-nb // DQ_BLOCK)
    padded = np.zeros(nb * NF4_BLOCK, dtype=np.float32)
    padded[:n] = w
    blocks = padded.reshape(nb, NF4_BLOCK)

    codes = np.empty((nb, NF4_BLOCK), dtype=np.uint8)
    absmax = np.empty(nb, dtype=np.float32)
    step = 16384  # blocks per chunk, bounds the float64 distance array
    for b0 in range(0, nb, step):
        codes[b0:b0 + step], absmax[b0:b0 + step] = _codes_for_blocks(
            blocks[b0:b0 + step], levels)
    # Short final block: only the elements present exist; the zeros padded in
    # above cannot raise a block's absmax.
    flat = codes.ravel()[:n]
    if n % 2:
        flat = np.concatenate([flat, np.zeros(1, dtype=np.uint8)])
    packed = (flat[0::2] | (flat[1::2] << 4)).astype(np.uint8)

    # Double quantisation of the constants.
    gpad = np.zeros(ng * DQ_BLOCK, dtype=np.float32)
    gpad[:nb] = absmax
    c1 = gpad.reshape(ng, DQ_BLOCK).max(axis=1).astype(np.float32)
    c1_per_block = np.repeat(c1, DQ_BLOCK)[:nb]
    c2 = np.zeros(nb, dtype=np.uint8)
    live = c1_per_block > 0
    rho = (absmax[live] / c1_per_block[live]).astype(np.float32)  # IEEE RNE
    c2[live] = e4m3_encode_rne(rho)
    return packed, c2, c1


# ---------------------------------------------------------------------------
# The 4-bit data types NF4 is compared with ("Introduction", contribution (1):
# NF4 gives better empirical results than 4-bit Integers and 4-bit Floats).
# The pages name these types but do not define them. READINGS: the plainest
# common ones, normalised like NF4 into [-1, 1] by the block absmax, with the
# exact zero at code 7 and the same nearest-value rule (a tie to the lower
# code). Both have 15 distinct values; code 15 repeats +1 and is therefore
# never chosen.
# ---------------------------------------------------------------------------

def int4_levels():
    """Symmetric 4-bit integers k / 7, k = -7 .. 7 (code k + 7), as float32;
    code 15 repeats +1."""
    v = [k / 7.0 for k in range(-7, 8)] + [1.0]
    return np.array(v, dtype=np.float64).astype(np.float32)


def e2m1_decode(code):
    """Value of a 4-bit float bit pattern: 1 sign bit, 2 exponent bits with
    bias 1, 1 mantissa bit; exponent 0 is subnormal (0.5 * mantissa)."""
    code = int(code)
    sign, e, m = (code >> 3) & 1, (code >> 1) & 3, code & 1
    mag = 0.5 * m if e == 0 else (1.0 + 0.5 * m) * 2.0 ** (e - 1)
    return -mag if sign else mag


def fp4_levels():
    """The 15 distinct values of the 16 E2M1 bit patterns (+0 and -0 merge
    into +0), ascending, divided by the largest magnitude 6, as float32;
    code 15 repeats +1."""
    vals = sorted({e2m1_decode(c) + 0.0 for c in range(16)})  # + 0.0 turns -0 into +0
    assert len(vals) == 15
    top = max(abs(v) for v in vals)
    return (np.array(vals + [vals[-1]], dtype=np.float64) / top).astype(np.float32)


def codebook_levels(name):
    """Level table of a 4-bit data type by name: "nf4", "int4" or "fp4"."""
    table = {"nf4": nf4_levels, "int4": int4_levels, "fp4": fp4_levels}
    if name not in table:
        raise ValueError("unknown 4-bit data type %r" % (name,))
    return table[name]()


def quantize_blockwise(w, levels=None):
    """Blockwise 4-bit quantisation WITHOUT double quantisation: the baseline
    the "Double Quantization" paragraph prices at 32/64 = 0.5 bit per weight.

    Same codes as quantize_nf4_dq (exact per-block absmax, IEEE float32
    quotient, nearest level); the constants are stored as they are: float32
    absmax per block of 64. Returns ``(packed, absmax)``.
    """
    if levels is None:
        levels = nf4_levels()
    w = np.ascontiguousarray(w, dtype=np.float32).ravel()
    if not np.all(np.isfinite(w)):
        raise ValueError("weights must be finite")
    n = w.size
    if n == 0:
        raise ValueError("empty input")
    nb = -(-n // NF4_BLOCK)
    padded = np.zeros(nb * NF4_BLOCK, dtype=np.float32)
    padded[:n] = w
    blocks = padded.reshape(nb, NF4_BLOCK)
    codes = np.empty((nb, NF4_BLOCK), dtype=np.uint8)
    absmax = np.empty(nb, dtype=np.float32)
    step = 16384
    for b0 in range(0, nb, step):
        codes[b0:b0 + step], absmax[b0:b0 + step] = _codes_for_blocks(
            blocks[b0:b0 + step], levels)
    flat = codes.ravel()[:n]
    if n % 2:
        flat = np.concatenate([flat, np.zeros(1, dtype=np.uint8)])
    packed = (flat[0::2] | (flat[1::2] << 4)).astype(np.uint8)
    return packed, absmax


def dequant_blockwise(packed, absmax, n, levels=None):
    """W_hat_i = fp32(q[code_i] * absmax_b): one float32 product per weight."""
    if levels is None:
        levels = nf4_levels()
    codes = unpack_codes(packed, n)
    absmax = np.asarray(absmax, dtype=np.float32)
    return (levels[codes] * absmax[np.arange(n) // NF4_BLOCK]).astype(np.float32)


def unpack_codes(packed, n):
    """The n 4-bit codes stored in ``packed`` (inverse of the packing above)."""
    packed = np.asarray(packed, dtype=np.uint8)
    both = np.empty(packed.size * 2, dtype=np.uint8)
    both[0::2] = packed & 0xF
    both[1::2] = packed >> 4
    return both[:n]


def dequant(packed, c2, c1, n, levels=None):
    """Dequantised weights W_hat (float32) of n elements.

    c_hat_b = fp32(dec(c2_b) * c1_g), then W_hat_i = fp32(q[code_i] * c_hat_b):
    two float32 products in this order. The bfloat16 operand of the matmul is
    ``bf16_round(W_hat)``.
    """
    if levels is None:
        levels = nf4_levels()
    codes = unpack_codes(packed, n)
    nb = -(-n // NF4_BLOCK)
    c2 = np.asarray(c2, dtype=np.uint8)[:nb]
    c1 = np.asarray(c1, dtype=np.float32)
    dec = e4m3_decode(c2).astype(np.float32)  # E4M3 values are exact in float32
    c1_per_block = c1[np.arange(nb) // DQ_BLOCK]
    chat = (dec * c1_per_block).astype(np.float32)
    chat_per_elem = chat[np.arange(n) // NF4_BLOCK]
    return (levels[codes] * chat_per_elem).astype(np.float32)


def storage_bits_per_param(n, double_quant=True):
    """Stored bits per weight: 4-bit codes plus, with double quantisation, one
    byte c2 per 64 and an fp32 c1 per 256 blocks; without it, an fp32 absmax
    per block of 64."""
    nb = -(-n // NF4_BLOCK)
    ng = -(-nb // DQ_BLOCK)
    if not double_quant:
        return (8.0 * (-(-n // 2)) + 32.0 * nb) / n
    return (8.0 * (-(-n // 2)) + 8.0 * nb + 32.0 * ng) / n


# ---------------------------------------------------------------------------
# LoRA linear layer on the frozen dequantised weight ("Low-Rank Adaptation"
# section: x_out = (W_q + B A) x_in with A: r x d, B: d x r). Rows of X are
# tokens, so the layer is Y = X W^T + s (X A^T) B^T with s = lora_alpha / r.
# Gradients reach only the adapters and the input ("backpropagates gradients
# through a frozen, 4-bit quantized pretrained language model into Low Rank
# Adapters"), so there is no weight gradient.
# ---------------------------------------------------------------------------

def linear_fwd(X, W, A, B, s):
    """Y = X W^T + s T B^T with T = X A^T, all in float64. Returns (Y, T).

    X: [M, K]; W: [N, K] (the bfloat16-rounded dequantised weight);
    A: [r, K]; B: [N, r]; s: LoRA scale.
    """
    X, W, A, B = (np.asarray(t, dtype=np.float64) for t in (X, W, A, B))
    T = X @ A.T
    Y = X @ W.T + float(s) * (T @ B.T)
    return Y, T


def linear_bwd(X, W, A, B, dY, s, need_dX=True):
    """Input and adapter gradients of linear_fwd for the upstream gradient dY.

    U = dY B; dX = dY W + s U A; dA = s U^T X; dB = s dY^T T with T = X A^T.
    Returns (dX, dA, dB), float64; dX is None when need_dX is false (W is
    then not used and may be None).
    """
    X, A, B, dY = (np.asarray(t, dtype=np.float64) for t in (X, A, B, dY))
    s = float(s)
    T = X @ A.T
    U = dY @ B
    dX = None
    if need_dX:
        dX = dY @ np.asarray(W, dtype=np.float64) + s * (U @ A)
    dA = s * (U.T @ X)
    dB = s * (dY.T @ T)
    return dX, dA, dB


def grouped_linear_fwd(X, W, A, B, s, groups):
    """Linears that share the input X (q / k / v of a decoder layer).

    W [g Ns, K], A [g r, K] and B [g Ns, r] stack the segments; segment i is
    linear_fwd(X, W_i, A_i, B_i, s). Returns (Y [M, g Ns], T [M, g r]).
    """
    W, A, B = (np.asarray(t, dtype=np.float64) for t in (W, A, B))
    g = int(groups)
    ns, r = W.shape[0] // g, A.shape[0] // g
    outs = [linear_fwd(X, W[i * ns:(i + 1) * ns], A[i * r:(i + 1) * r], B[i * ns:(i + 1) * ns], s)
            for i in range(g)]
    return np.concatenate([o[0] for o in outs], axis=1), np.concatenate([o[1] for o in outs], axis=1)


def grouped_linear_bwd(X, W, A, B, dY, s, groups, need_dX=True):
    """Backward of grouped_linear_fwd: dX summed over the segments (they share
    X), dA [g r, K] and dB [g Ns, r] stacked like A and B."""
    A, B, dY = (np.asarray(t, dtype=np.float64) for t in (A, B, dY))
    g = int(groups)
    ns, r = B.shape[0] // g, A.shape[0] // g
    dX, dA, dB = None, [], []
    for i in range(g):
        Wi = None if W is None else np.asarray(W, dtype=np.float64)[i * ns:(i + 1) * ns]
        dXi, dAi, dBi = linear_bwd(X, Wi, A[i * r:(i + 1) * r], B[i * ns:(i + 1) * ns],
                                   dY[:, i * ns:(i + 1) * ns], s, need_dX=need_dX)
        if need_dX:
            dX = dXi if dX is None else dX + dXi
        dA.append(dAi)
        dB.append(dBi)
    return dX, np.concatenate(dA, axis=0), np.concatenate(dB, axis=0)


def merge_lora(W, A, B, s):
    """The merged weight W + s B A in float64 ("Low-Rank Adaptation (LoRA)":
    x_out = (W_q + B A) x_in), before any rounding."""
    W, A, B = (np.asarray(t, dtype=np.float64) for t in (W, A, B))
    return W + float(s) * (B @ A)
