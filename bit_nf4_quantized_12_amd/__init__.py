"""Python binding of the MI355X (gfx950) NF4 + double-quantisation + LoRA library.

Argument marshalling only: every step runs in the HIP kernels of
``libqlora.so`` (built in-tree by ``bit_nf4_quantized_12_amd.build``).
PyTorch provides device memory and the current stream. There is no CPU
fallback: when the library is missing or fails to load, every call raises.

The function names are those of the C ABI (include/qlora.h):

* ``qlora_nf4_levels()``
* ``qlora_quantize_nf4_dq(w)``
* ``qlora_dequant(codes, c2, c1, n, dtype)``
* ``qlora_nf4_matmul(W, act, transposed)``
* ``qlora_4bit_matmul_lora(W, act, L, R, transposed)``: the same product with a
  rank term L R^T fused into its epilogue (the kernel the linear layer runs)
* ``qlora_linear_workspace_bytes(M, N, K, r)``
* ``qlora_linear_fwd(W, X, A, B, scale, ...)``
* ``qlora_linear_bwd(W, X, A, B, dY, T, scale, ...)``
* ``qlora_linear_fwd_grouped`` / ``qlora_linear_bwd_grouped``: linears that share
  one input (q / k / v, gate / up), weights and adapters stacked by segment
* ``qlora_merge_lora(W, A, B, scale)``: the dense bf16 weight W~ + scale B A for serving
* ``qlora_adamw_step(p32, grad, m, v, step, ...)``: the adapters' optimizer
  step; the state may sit in HBM or in pinned host memory (paged out)
* ``qlora_levels(codebook)``, ``qlora_quantize_4bit(w, codebook, double_quant)``,
  ``qlora_dequant_4bit(...)``: the Int4 / FP4 comparison types and the format
  without double quantisation; a weight quantised that way carries its
  ``codebook`` and ``double_quant`` and goes through ``qlora_4bit_matmul`` /
  ``qlora_linear_fwd_4bit`` / ``qlora_linear_bwd_4bit`` (chosen by the wrappers
  below from the weight).
"""

import ctypes
import os
import threading
from collections import namedtuple

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libqlora.so")

QLORA_F32 = 0
QLORA_BF16 = 1
CODEBOOKS = {"nf4": 0, "int4": 1, "fp4": 2}

_lock = threading.Lock()
_lib = None


class QloraError(RuntimeError):
    """A library call returned a non-zero status."""


class _Weight(ctypes.Structure):
    _fields_ = [
        ("codes", ctypes.c_void_p),
        ("c2_fp8", ctypes.c_void_p),
        ("c1", ctypes.c_void_p),
        ("rows", ctypes.c_int64),
        ("cols", ctypes.c_int64),
    ]


class _Weight4bit(ctypes.Structure):
    _fields_ = [
        ("codes", ctypes.c_void_p),
        ("consts", ctypes.c_void_p),
        ("c1", ctypes.c_void_p),
        ("rows", ctypes.c_int64),
        ("cols", ctypes.c_int64),
        ("codebook", ctypes.c_int32),
        ("double_quant", ctypes.c_int32),
    ]


class _AdamWParams(ctypes.Structure):
    _fields_ = [
        ("lr", ctypes.c_float),
        ("beta1", ctypes.c_float),
        ("beta2", ctypes.c_float),
        ("eps", ctypes.c_float),
        ("weight_decay", ctypes.c_float),
        ("step", ctypes.c_int64),
    ]


def load_library(path=LIB_PATH):
    """Load libqlora.so (once). Raises ImportError if it is missing or broken."""
    global _lib
    with _lock:
        if _lib is not None:
            return _lib
        if not os.path.exists(path):
            raise ImportError(
                f"{path} not found: build it with `python -m bit_nf4_quantized_12_amd.build`")
        lib = ctypes.CDLL(path)
        vp, i64, f32, sz, i32 = ctypes.c_void_p, ctypes.c_int64, ctypes.c_float, ctypes.c_size_t, ctypes.c_int
        sig = {
            "qlora_nf4_levels": ([ctypes.POINTER(ctypes.c_float)], i32),
            "qlora_quantize_nf4_dq": ([vp, i64, vp, vp, vp, vp], i32),
            "qlora_dequant": ([vp, vp, vp, i64, i32, vp, vp], i32),
            "qlora_linear_workspace_bytes": ([i64, i64, i64, i64], sz),
            "qlora_nf4_matmul": ([ctypes.POINTER(_Weight), vp, i64, i32, vp, vp], i32),
            "qlora_linear_fwd": ([ctypes.POINTER(_Weight), vp, vp, vp, i64, i64, f32, vp, vp, vp, sz, vp], i32),
            "qlora_linear_fwd_noalloc": ([ctypes.POINTER(_Weight), vp, vp, vp, i64, i64, f32, vp, vp, vp], i32),
            "qlora_linear_bwd": ([ctypes.POINTER(_Weight), vp, vp, vp, vp, vp, i64, i64, f32, vp, vp, vp, vp, sz, vp], i32),
            "qlora_status_string": ([i32], ctypes.c_char_p),
            "qlora_levels": ([i32, ctypes.POINTER(ctypes.c_float)], i32),
            "qlora_adamw_step": ([vp, vp, vp, vp, vp, i64, ctypes.POINTER(_AdamWParams), vp], i32),
            "qlora_linear_grouped_workspace_bytes": ([i64, i64, i64, i64, i64], sz),
            "qlora_merge_lora": ([ctypes.POINTER(_Weight4bit), vp, vp, i64, f32, vp, vp], i32),
            "qlora_quantize_4bit_batch": ([i32, ctypes.POINTER(vp), ctypes.POINTER(i64), i32, i32,
                                           ctypes.POINTER(vp), ctypes.POINTER(vp), ctypes.POINTER(vp), vp], i32),
            "qlora_linear_fwd_grouped": ([ctypes.POINTER(_Weight4bit), i64, vp, vp, vp, i64, i64, f32, vp, vp, vp, sz, vp], i32),
            "qlora_linear_bwd_grouped": ([ctypes.POINTER(_Weight4bit), i64, vp, vp, vp, vp, vp, i64, i64, f32, vp, vp, vp, vp, sz, vp], i32),
            "qlora_quantize_4bit": ([vp, i64, i32, i32, vp, vp, vp, vp], i32),
            "qlora_dequant_4bit": ([vp, vp, vp, i64, i32, i32, i32, vp, vp], i32),
            "qlora_4bit_matmul": ([ctypes.POINTER(_Weight4bit), vp, i64, i32, vp, vp], i32),
            "qlora_4bit_matmul_lora": ([ctypes.POINTER(_Weight4bit), vp, i64, i32, vp, vp, i64, vp, vp], i32),
            "qlora_linear_fwd_4bit": ([ctypes.POINTER(_Weight4bit), vp, vp, vp, i64, i64, f32, vp, vp, vp, sz, vp], i32),
            "qlora_linear_bwd_4bit": ([ctypes.POINTER(_Weight4bit), vp, vp, vp, vp, vp, i64, i64, f32, vp, vp, vp, vp, sz, vp], i32),
        }
        for name, (args, res) in sig.items():
            fn = getattr(lib, name)
            fn.argtypes = args
            fn.restype = res
        _lib = lib
        return lib


def _check(status):
    if status != 0:
        msg = load_library().qlora_status_string(status).decode()
        raise QloraError(f"qlora status {status}: {msg}")


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(device):
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def _need(t, dtype, name):
    if not isinstance(t, torch.Tensor) or not t.is_cuda:
        raise TypeError(f"{name} must be a CUDA (HIP) tensor")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def _same_device(dev, **tensors):
    for name, t in tensors.items():
        if t is not None and t.device != dev:
            raise ValueError(f"{name} is on {t.device}, the other operands on {dev}")


def _buf(t, shape, dtype, dev, name):
    """A new tensor of this shape, or the caller's one after checking it (the
    library writes shape[0] * shape[1] elements through its pointer)."""
    if t is None:
        return torch.empty(shape, dtype=dtype, device=dev)
    _need(t, dtype, name)
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")
    _same_device(dev, **{name: t})
    return t


def _check_stored(n, codes, consts, c1, double_quant, dev):
    """The stored buffers of n weights hold what the library reads."""
    nb = -(-n // 64)
    need = [("codes", codes, -(-n // 2)), ("block constants", consts, nb)]
    if double_quant:
        need.append(("c1", c1, -(-nb // 256)))
    for name, t, cnt in need:
        if t.numel() < cnt:
            raise ValueError(f"{name} holds {t.numel()} elements, {n} weights need {cnt}")
        _same_device(dev, **{name: t})


def _check_weight(W, dev):
    _check_stored(W.rows * W.cols, W.codes, W.c2, W.c1, W.double_quant, dev)


NF4Weight = namedtuple("NF4Weight", ["codes", "c2", "c1", "rows", "cols", "codebook", "double_quant"],
                       defaults=("nf4", True))
NF4Weight.__doc__ = (
    "Stored 4-bit weight [rows, cols]: device tensors codes (uint8) and, with double quantisation, "
    "c2 (uint8) and c1 (float32); without it, c2 holds the float32 block absmax and c1 is None. "
    "codebook: 'nf4' (default), 'int4' or 'fp4'.")


def _codebook_id(codebook):
    if codebook not in CODEBOOKS:
        raise ValueError(f"codebook must be one of {sorted(CODEBOOKS)}")
    return CODEBOOKS[codebook]


def storage_sizes(n):
    """(bytes of codes, bytes of c2, number of c1 floats) for n weights."""
    nb = -(-n // 64)
    return -(-n // 2), nb, -(-nb // 256)


def qlora_nf4_levels():
    """The 16 NF4 levels (float32, ascending) as a CPU tensor."""
    out = (ctypes.c_float * 16)()
    _check(load_library().qlora_nf4_levels(out))
    return torch.tensor(list(out), dtype=torch.float32)


def qlora_quantize_nf4_dq(w, out=None):
    """Quantise bf16 weights (any shape, C order) -> (codes, c2, c1) device tensors.

    ``out`` may supply preallocated (codes, c2, c1) tensors of the right sizes.
    """
    _need(w, torch.bfloat16, "w")
    n = w.numel()
    nc, nb, ng = storage_sizes(n)
    if out is None:
        dev = w.device
        codes = torch.empty(nc, dtype=torch.uint8, device=dev)
        c2 = torch.empty(nb, dtype=torch.uint8, device=dev)
        c1 = torch.empty(ng, dtype=torch.float32, device=dev)
    else:
        codes, c2, c1 = out
    lib = load_library()
    _check(lib.qlora_quantize_nf4_dq(_ptr(w), n, _ptr(codes), _ptr(c2), _ptr(c1), _stream(w.device)))
    return codes, c2, c1


def qlora_levels(codebook="nf4"):
    """The 16 levels (float32, ascending) of a 4-bit data type as a CPU tensor."""
    out = (ctypes.c_float * 16)()
    _check(load_library().qlora_levels(_codebook_id(codebook), out))
    return torch.tensor(list(out), dtype=torch.float32)


def qlora_quantize_4bit(w, codebook="nf4", double_quant=True, out=None):
    """Quantise bf16 weights with a 4-bit data type -> (codes, consts, c1).

    consts is c2 (uint8, E4M3) with double quantisation, else the float32 block
    absmax; c1 is None without double quantisation.
    """
    _need(w, torch.bfloat16, "w")
    cb = _codebook_id(codebook)
    n = w.numel()
    nc, nb, ng = storage_sizes(n)
    if out is None:
        dev = w.device
        codes = torch.empty(nc, dtype=torch.uint8, device=dev)
        consts = torch.empty(nb, dtype=torch.uint8 if double_quant else torch.float32, device=dev)
        c1 = torch.empty(ng, dtype=torch.float32, device=dev) if double_quant else None
    else:
        codes, consts, c1 = out
    _check(load_library().qlora_quantize_4bit(_ptr(w), n, cb, 1 if double_quant else 0, _ptr(codes),
                                              _ptr(consts), _ptr(c1), _stream(w.device)))
    return codes, consts, c1


def qlora_dequant_4bit(codes, consts, c1, n, codebook="nf4", double_quant=True, dtype=torch.float32,
                       out=None):
    """Dequantise n weights of a stored 4-bit format to float32 (W^) or bfloat16 (W~)."""
    _need(codes, torch.uint8, "codes")
    _need(consts, torch.uint8 if double_quant else torch.float32, "consts")
    if double_quant:
        _need(c1, torch.float32, "c1")
    code = {torch.float32: QLORA_F32, torch.bfloat16: QLORA_BF16}.get(dtype)
    if code is None:
        raise TypeError("dtype must be float32 or bfloat16")
    _check_stored(n, codes, consts, c1, double_quant, codes.device)
    out = _buf(out, (n,), dtype, codes.device, "out")
    _check(load_library().qlora_dequant_4bit(_ptr(codes), _ptr(consts), _ptr(c1) if double_quant else None, n,
                                             _codebook_id(codebook), 1 if double_quant else 0, code,
                                             _ptr(out), _stream(codes.device)))
    return out


def quantize_weight(w, codebook="nf4", double_quant=True):
    """Quantise a 2-D bf16 weight [N, K] (NF4 + double quantisation by default)."""
    if w.dim() != 2:
        raise ValueError("weight must be 2-D [out, in]")
    if codebook == "nf4" and double_quant:
        codes, c2, c1 = qlora_quantize_nf4_dq(w)
    else:
        codes, c2, c1 = qlora_quantize_4bit(w, codebook, double_quant)
    return NF4Weight(codes, c2, c1, w.shape[0], w.shape[1], codebook, bool(double_quant))


def dequant_weight(W, dtype=torch.bfloat16):
    """The dequantised weight [rows, cols] of a stored weight."""
    n = W.rows * W.cols
    if W.codebook == "nf4" and W.double_quant:
        return qlora_dequant(W.codes, W.c2, W.c1, n, dtype).view(W.rows, W.cols)
    return qlora_dequant_4bit(W.codes, W.c2, W.c1, n, W.codebook, W.double_quant, dtype).view(W.rows, W.cols)


def qlora_dequant(codes, c2, c1, n, dtype=torch.float32, out=None):
    """Dequantise n stored weights to float32 (W^) or bfloat16 (W~)."""
    _need(codes, torch.uint8, "codes")
    _need(c2, torch.uint8, "c2")
    _need(c1, torch.float32, "c1")
    code = {torch.float32: QLORA_F32, torch.bfloat16: QLORA_BF16}.get(dtype)
    if code is None:
        raise TypeError("dtype must be float32 or bfloat16")
    _check_stored(n, codes, c2, c1, True, codes.device)
    out = _buf(out, (n,), dtype, codes.device, "out")
    _check(load_library().qlora_dequant(_ptr(codes), _ptr(c2), _ptr(c1), n, code, _ptr(out),
                                        _stream(codes.device)))
    return out


def qlora_nf4_matmul(W, act, transposed=False, out=None):
    """Base product on the frozen weight: act W~^T ([M, N]) or, transposed, act W~ ([M, K])."""
    _need(act, torch.bfloat16, "act")
    M = act.shape[0]
    if act.shape[1] != (W.rows if transposed else W.cols):
        raise ValueError("act has the wrong number of columns")
    _check_weight(W, act.device)
    out = _buf(out, (M, W.cols if transposed else W.rows), torch.bfloat16, act.device, "out")
    w, sfx = _weight_struct(W)
    fn = load_library().qlora_nf4_matmul if not sfx else load_library().qlora_4bit_matmul
    _check(fn(ctypes.byref(w), _ptr(act), M, 1 if transposed else 0, _ptr(out), _stream(act.device)))
    return out


qlora_4bit_matmul = qlora_nf4_matmul  # one wrapper serves every stored format


def qlora_4bit_matmul_lora(W, act, L, R, transposed=False, out=None):
    """Base product with a rank term in its epilogue: act W~^T + L R^T ([M, N]) or,
    transposed, act W~ + L R^T ([M, K]); L [M, rp] and R [Nout, rp] bf16, rp % 64 == 0."""
    _need(act, torch.bfloat16, "act")
    _need(L, torch.bfloat16, "L")
    _need(R, torch.bfloat16, "R")
    M = act.shape[0]
    nout = W.cols if transposed else W.rows
    if act.shape[1] != (W.rows if transposed else W.cols):
        raise ValueError("act has the wrong number of columns")
    rp = L.shape[1]
    if L.shape[0] != M or tuple(R.shape) != (nout, rp):
        raise ValueError(f"L must be [M, rp] and R [{nout}, rp]")
    _same_device(act.device, L=L, R=R)
    _check_weight(W, act.device)
    out = _buf(out, (M, nout), torch.bfloat16, act.device, "out")
    w = _weight4_struct(W)
    _check(load_library().qlora_4bit_matmul_lora(ctypes.byref(w), _ptr(act), M, 1 if transposed else 0, _ptr(L),
                                                 _ptr(R), rp, _ptr(out), _stream(act.device)))
    return out


def qlora_linear_workspace_bytes(M, N, K, r):
    return int(load_library().qlora_linear_workspace_bytes(M, N, K, r))


def _is_nf4_dq(W):
    return W.codebook == "nf4" and W.double_quant


def _weight_struct(W):
    """(struct, entry-point suffix): the NF4 + DQ struct, or the general 4-bit one."""
    _need(W.codes, torch.uint8, "W.codes")
    if _is_nf4_dq(W):
        _need(W.c2, torch.uint8, "W.c2")
        _need(W.c1, torch.float32, "W.c1")
        return _Weight(W.codes.data_ptr(), W.c2.data_ptr(), W.c1.data_ptr(), W.rows, W.cols), ""
    if W.double_quant:
        _need(W.c2, torch.uint8, "W.c2")
        _need(W.c1, torch.float32, "W.c1")
    else:
        _need(W.c2, torch.float32, "W.c2 (block absmax)")
    c1 = W.c1.data_ptr() if W.double_quant else None
    return _Weight4bit(W.codes.data_ptr(), W.c2.data_ptr(), c1, W.rows, W.cols,
                       _codebook_id(W.codebook), 1 if W.double_quant else 0), "_4bit"


def new_workspace(nbytes, device):
    """A workspace of nbytes (at least 256) for the linear entry points."""
    return torch.empty(max(int(nbytes), 256), dtype=torch.uint8, device=device)


def _workspace(M, N, K, r, device, workspace):
    need = qlora_linear_workspace_bytes(M, N, K, r)
    if workspace is None or workspace.numel() < need:
        workspace = new_workspace(need, device)
    return workspace


def qlora_linear_fwd(W, X, A, B, scale, save_T=True, Y=None, T=None, workspace=None):
    """Y = X W~^T + scale (X A^T) B^T (bf16). Returns (Y, T) with T float32 [M, r] or None."""
    _need(X, torch.bfloat16, "X")
    _need(A, torch.bfloat16, "A")
    _need(B, torch.bfloat16, "B")
    M, K = X.shape
    r = A.shape[0]
    if K != W.cols or A.shape[1] != K or B.shape != (W.rows, r):
        raise ValueError("shape mismatch: X [M, K], A [r, K], B [N, r], W [N, K]")
    dev = X.device
    _same_device(dev, A=A, B=B)
    _check_weight(W, dev)
    Y = _buf(Y, (M, W.rows), torch.bfloat16, dev, "Y")
    T = _buf(T, (M, r), torch.float32, dev, "T") if save_T else None
    ws = _workspace(M, W.rows, K, r, dev, workspace)
    w, sfx = _weight_struct(W)
    fn = getattr(load_library(), "qlora_linear_fwd" + sfx)
    _check(fn(ctypes.byref(w), _ptr(X), _ptr(A), _ptr(B), M, r, float(scale), _ptr(Y), _ptr(T), _ptr(ws),
              ws.numel(), _stream(dev)))
    return Y, T


def qlora_linear_fwd_noalloc(W, X, A, B, scale, Y, T=None):
    """qlora_linear_fwd with the library's fixed scratch in place of a workspace:
    allocates nothing (Y, and T if given, are the caller's buffers). NF4 + DQ
    weights only; sizes needing more than 64 MiB of scratch raise QloraError."""
    for t, name in ((X, "X"), (A, "A"), (B, "B")):
        _need(t, torch.bfloat16, name)
    if not _is_nf4_dq(W):
        raise ValueError("qlora_linear_fwd_noalloc takes NF4 + double-quantised weights")
    M, K = X.shape
    r = A.shape[0]
    if K != W.cols or A.shape[1] != K or B.shape != (W.rows, r):
        raise ValueError("shape mismatch: X [M, K], A [r, K], B [N, r], W [N, K]")
    dev = X.device
    _same_device(dev, A=A, B=B)
    _check_weight(W, dev)
    _buf(Y, (M, W.rows), torch.bfloat16, dev, "Y")
    if T is not None:
        _buf(T, (M, r), torch.float32, dev, "T")
    w, _ = _weight_struct(W)
    _check(load_library().qlora_linear_fwd_noalloc(ctypes.byref(w), _ptr(X), _ptr(A), _ptr(B), M, r,
                                                   float(scale), _ptr(Y), _ptr(T), _stream(dev)))
    return Y, T


def qlora_linear_bwd(W, X, A, B, dY, T, scale, need_dX=True, dX=None, dA=None, dB=None,
                     workspace=None):
    """Gradients (dX or None, dA, dB), all bf16, of qlora_linear_fwd for dY."""
    for t, name in ((X, "X"), (A, "A"), (B, "B"), (dY, "dY")):
        _need(t, torch.bfloat16, name)
    if T is not None:
        _need(T, torch.float32, "T")
    M, K = X.shape
    r = A.shape[0]
    N = W.rows
    if dY.shape != (M, N) or K != W.cols or A.shape[1] != K or B.shape != (N, r):
        raise ValueError("shape mismatch")
    if T is not None and tuple(T.shape) != (M, r):
        raise ValueError(f"T must have shape {(M, r)}")
    dev = X.device
    _same_device(dev, A=A, B=B, dY=dY, T=T)
    _check_weight(W, dev)
    dX = _buf(dX, (M, K), torch.bfloat16, dev, "dX") if need_dX else None
    dA = _buf(dA, (r, K), torch.bfloat16, dev, "dA")
    dB = _buf(dB, (N, r), torch.bfloat16, dev, "dB")
    ws = _workspace(M, N, K, r, dev, workspace)
    w, sfx = _weight_struct(W)
    fn = getattr(load_library(), "qlora_linear_bwd" + sfx)
    _check(fn(ctypes.byref(w), _ptr(X), _ptr(A), _ptr(B), _ptr(dY), _ptr(T), M, r, float(scale), _ptr(dX),
              _ptr(dA), _ptr(dB), _ptr(ws), ws.numel(), _stream(dev)))
    return dX, dA, dB


class LoRALinear4bitFunction(torch.autograd.Function):
    """Autograd wrapper: frozen NF4 weight, trainable A and B, input X."""

    @staticmethod
    def forward(ctx, X, A, B, W, scale):
        # the kernels need contiguous operands; the backward gets the same copies
        Xc, Ac, Bc = X.contiguous(), A.contiguous(), B.contiguous()
        Y, T = qlora_linear_fwd(W, Xc, Ac, Bc, scale)
        ctx.save_for_backward(Xc, Ac, Bc, T)
        ctx.W = W
        ctx.scale = scale
        return Y

    @staticmethod
    def backward(ctx, dY):
        X, A, B, T = ctx.saved_tensors
        dX, dA, dB = qlora_linear_bwd(ctx.W, X, A, B, dY.contiguous(), T, ctx.scale,
                                      need_dX=ctx.needs_input_grad[0])
        return dX, dA, dB, None, None


# the general-format entry points have the same wrappers (dispatch on the weight)
qlora_linear_fwd_4bit = qlora_linear_fwd
qlora_linear_bwd_4bit = qlora_linear_bwd


def qlora_adamw_step(p32, grad, m, v, step, lr=1e-3, beta1=0.9, beta2=0.999, eps=1e-8,
                     weight_decay=0.0, p16=None):
    """One AdamW step in place on float32 master weights ``p32`` with moments ``m``, ``v``
    (float32) and a bf16 gradient; ``p16`` (bf16) receives the updated weights if given.

    Every tensor may live on the GPU or in pinned host memory (``pin_memory=True``);
    the work runs on the current stream of the GPU that holds ``grad`` (or GPU 0).
    """
    for t, dt, name in ((p32, torch.float32, "p32"), (grad, torch.bfloat16, "grad"),
                        (m, torch.float32, "m"), (v, torch.float32, "v")):
        if not isinstance(t, torch.Tensor) or t.dtype != dt or not t.is_contiguous():
            raise TypeError(f"{name} must be a contiguous {dt} tensor")
        if not (t.is_cuda or t.is_pinned()):
            raise TypeError(f"{name} must be a GPU tensor or pinned host memory")
    n = p32.numel()
    if grad.numel() != n or m.numel() != n or v.numel() != n or (p16 is not None and p16.numel() != n):
        raise ValueError("size mismatch")
    if p16 is not None and (p16.dtype != torch.bfloat16 or not p16.is_contiguous()):
        raise TypeError("p16 must be a contiguous bfloat16 tensor")
    dev = next((t.device for t in (grad, p32, m, v) if t.is_cuda), torch.device("cuda", 0))
    h = _AdamWParams(lr, beta1, beta2, eps, weight_decay, int(step))
    _check(load_library().qlora_adamw_step(_ptr(p32), _ptr(p16), _ptr(grad), _ptr(m), _ptr(v), n,
                                           ctypes.byref(h), _stream(dev)))


def _weight4_struct(W):
    """The general 4-bit weight struct for any stored format (grouped entry points)."""
    _need(W.codes, torch.uint8, "W.codes")
    _need(W.c2, torch.uint8 if W.double_quant else torch.float32, "W.c2")
    if W.double_quant:
        _need(W.c1, torch.float32, "W.c1")
    c1 = W.c1.data_ptr() if W.double_quant else None
    return _Weight4bit(W.codes.data_ptr(), W.c2.data_ptr(), c1, W.rows, W.cols, _codebook_id(W.codebook),
                       1 if W.double_quant else 0)


def qlora_linear_grouped_workspace_bytes(M, N, K, r, groups):
    return int(load_library().qlora_linear_grouped_workspace_bytes(M, N, K, r, groups))


def qlora_linear_fwd_grouped(W, groups, X, A, B, scale, save_T=True, Y=None, T=None, workspace=None):
    """Grouped forward: W [g Ns, K] stacked weights, A [g r, K], B [g Ns, r].

    Returns (Y [M, g Ns] bf16, T [M, g r] float32 or None).
    """
    _need(X, torch.bfloat16, "X")
    _need(A, torch.bfloat16, "A")
    _need(B, torch.bfloat16, "B")
    M, K = X.shape
    g = int(groups)
    r = A.shape[0] // g
    if A.shape != (g * r, K) or B.shape != (W.rows, r) or W.cols != K:
        raise ValueError("shape mismatch: X [M, K], A [g r, K], B [g Ns, r], W [g Ns, K]")
    dev = X.device
    _same_device(dev, A=A, B=B)
    _check_weight(W, dev)
    Y = _buf(Y, (M, W.rows), torch.bfloat16, dev, "Y")
    T = _buf(T, (M, g * r), torch.float32, dev, "T") if save_T else None
    need = qlora_linear_grouped_workspace_bytes(M, W.rows, K, r, g)
    ws = workspace if workspace is not None and workspace.numel() >= need else new_workspace(need, dev)
    w = _weight4_struct(W)
    _check(load_library().qlora_linear_fwd_grouped(ctypes.byref(w), g, _ptr(X), _ptr(A), _ptr(B), M, r,
                                                   float(scale), _ptr(Y), _ptr(T), _ptr(ws), ws.numel(),
                                                   _stream(dev)))
    return Y, T


def qlora_linear_bwd_grouped(W, groups, X, A, B, dY, T, scale, need_dX=True, dX=None, dA=None, dB=None,
                             workspace=None):
    """Grouped backward: (dX [M, K] summed over the segments or None, dA [g r, K], dB [g Ns, r])."""
    for t, name in ((X, "X"), (A, "A"), (B, "B"), (dY, "dY")):
        _need(t, torch.bfloat16, name)
    if T is not None:
        _need(T, torch.float32, "T")
    M, K = X.shape
    g = int(groups)
    r = A.shape[0] // g
    N = W.rows
    if dY.shape != (M, N) or A.shape != (g * r, K) or B.shape != (N, r) or W.cols != K:
        raise ValueError("shape mismatch")
    if T is not None and tuple(T.shape) != (M, g * r):
        raise ValueError(f"T must have shape {(M, g * r)}")
    dev = X.device
    _same_device(dev, A=A, B=B, dY=dY, T=T)
    _check_weight(W, dev)
    dX = _buf(dX, (M, K), torch.bfloat16, dev, "dX") if need_dX else None
    dA = _buf(dA, (g * r, K), torch.bfloat16, dev, "dA")
    dB = _buf(dB, (N, r), torch.bfloat16, dev, "dB")
    need = qlora_linear_grouped_workspace_bytes(M, N, K, r, g)
    ws = workspace if workspace is not None and workspace.numel() >= need else new_workspace(need, dev)
    w = _weight4_struct(W)
    _check(load_library().qlora_linear_bwd_grouped(ctypes.byref(w), g, _ptr(X), _ptr(A), _ptr(B), _ptr(dY),
                                                   _ptr(T), M, r, float(scale), _ptr(dX), _ptr(dA), _ptr(dB),
                                                   _ptr(ws), ws.numel(), _stream(dev)))
    return dX, dA, dB


def qlora_merge_lora(W, A, B, scale, out=None):
    """Dense bf16 weight [N, K] = bf16(W^ + scale B A): the adapters folded into the frozen weight."""
    _need(A, torch.bfloat16, "A")
    _need(B, torch.bfloat16, "B")
    r = A.shape[0]
    if A.shape != (r, W.cols) or B.shape != (W.rows, r):
        raise ValueError("shape mismatch: A [r, K], B [N, r], W [N, K]")
    _same_device(A.device, B=B)
    _check_weight(W, A.device)
    out = _buf(out, (W.rows, W.cols), torch.bfloat16, A.device, "out")
    w = _weight4_struct(W)
    _check(load_library().qlora_merge_lora(ctypes.byref(w), _ptr(A), _ptr(B), r, float(scale), _ptr(out),
                                           _stream(A.device)))
    return out


def qlora_quantize_4bit_batch(ws, codebook="nf4", double_quant=True, outs=None):
    """Quantise up to 16 bf16 tensors with one launch -> list of (codes, consts, c1)."""
    k = len(ws)
    if not 1 <= k <= 16:
        raise ValueError("1 to 16 tensors per batch")
    for i, w in enumerate(ws):
        _need(w, torch.bfloat16, f"ws[{i}]")
    if outs is None:
        outs = []
        for w in ws:
            nc, nb, ng = storage_sizes(w.numel())
            outs.append((torch.empty(nc, dtype=torch.uint8, device=w.device),
                         torch.empty(nb, dtype=torch.uint8 if double_quant else torch.float32, device=w.device),
                         torch.empty(ng, dtype=torch.float32, device=w.device) if double_quant else None))
    arr = ctypes.c_void_p * k
    wp = arr(*[w.data_ptr() for w in ws])
    cp = arr(*[o[0].data_ptr() for o in outs])
    kp = arr(*[o[1].data_ptr() for o in outs])
    c1p = arr(*[(o[2].data_ptr() if double_quant else 0) for o in outs])
    n = (ctypes.c_int64 * k)(*[w.numel() for w in ws])
    _check(load_library().qlora_quantize_4bit_batch(k, wp, n, _codebook_id(codebook), 1 if double_quant else 0,
                                                    cp, kp, c1p, _stream(ws[0].device)))
    return outs
