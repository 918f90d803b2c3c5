"""Python binding of libconvrot.so, the ConvRot W8A8 rotated-INT8 linear layer for
AMD Instinct MI355X (gfx950).

Argument marshalling only: every step of the layer runs in the library's HIP
kernels.  PyTorch supplies device memory and the current HIP stream.  The C ABI
and its contract are in ``include/convrot.h``.

bf16 tensors are ``torch.bfloat16``; codes ``torch.int8``; scales ``torch.float32``.
All tensors must be contiguous CUDA (HIP) tensors on the current device.
"""
from __future__ import annotations

import ctypes as C
import os

import torch

__all__ = [
    "BLOCK", "BWD_BF16", "BWD_INT8", "ConvRotError", "lib", "library_path",
    "quantize_weight", "quantize_act", "linear_fwd", "gemm_i8_bf16", "gemm_i8_i32",
    "bwd_quant_dy", "linear_bwd_dx", "dequant_weight_t", "embedding_lookup",
    "workspace_bytes", "linear_fwd_lora", "lora_down", "linear_fwd_noalloc",
    "NOALLOC_SCRATCH_BYTES", "EXPORTS",
]

BLOCK = 128
BWD_BF16 = 0
BWD_INT8 = 1
OP_LINEAR_FWD = 0
OP_LINEAR_BWD_DX = 1
OP_LINEAR_FWD_LORA = 2  # mode = LoRA rank
NOALLOC_SCRATCH_BYTES = 96 << 20  # static scratch of the allocation-free forward, per GPU

_HERE = os.path.dirname(os.path.abspath(__file__))
library_path = os.path.join(_HERE, "libconvrot.so")

# Every symbol declared in include/convrot.h.
EXPORTS = (
    "convrot_quantize_weight", "convrot_linear_fwd", "convrot_linear_bwd_dx",
    "convrot_embedding_lookup", "convrot_workspace_bytes", "convrot_status_string",
    "convrot_quantize_act", "convrot_gemm_i8_bf16", "convrot_gemm_i8_i32",
    "convrot_bwd_quant_dy", "convrot_dequant_weight_t", "convrot_linear_fwd_lora",
    "convrot_lora_down", "convrot_linear_fwd_noalloc",
)


class ConvRotError(RuntimeError):
    def __init__(self, fn: str, status: int):
        super().__init__(f"{fn}: status {status} ({status_string(status)})")
        self.status = status


_lib = None


def lib():
    """Load libconvrot.so (built by ``w8a8_rotated_int8_amd/build.py``).  Raises if
    it is missing: there is no fallback path."""
    global _lib
    if _lib is None:
        if not os.path.exists(library_path):
            raise ImportError(f"{library_path} is not built; run `python __graft_entry__.py` "
                              "or `python w8a8_rotated_int8_amd/build.py`")
        L = C.CDLL(library_path)
        p, i64, i32, sz = C.c_void_p, C.c_int64, C.c_int32, C.c_size_t
        sig = {
            "convrot_quantize_weight": [p, i64, i64, i32, i64, p, p, p],
            "convrot_linear_fwd": [p, i64, i64, p, p, i64, p, p, p, sz, p],
            "convrot_linear_bwd_dx": [p, i64, i64, p, p, i64, i32, p, p, sz, p],
            "convrot_embedding_lookup": [p, i64, p, p, i64, i64, p, p, p],
            "convrot_workspace_bytes": [i32, i64, i64, i64, i32],
            "convrot_status_string": [C.c_int],
            "convrot_quantize_act": [p, i64, i64, p, p, p],
            "convrot_gemm_i8_bf16": [p, p, p, p, i64, i64, i64, p, p, p],
            "convrot_gemm_i8_i32": [p, p, i64, i64, i64, i32, p, p],
            "convrot_bwd_quant_dy": [p, i64, i64, p, p, p, p],
            "convrot_dequant_weight_t": [p, p, i64, i64, p, p],
            "convrot_linear_fwd_lora": [p, i64, i64, p, p, i64, p, p, p, i32, C.c_float, p, p,
                                        sz, p],
            "convrot_lora_down": [p, i64, i64, p, i32, p, p],
            "convrot_linear_fwd_noalloc": [p, i64, i64, p, p, i64, p, p, p],
        }
        for name, argt in sig.items():
            f = getattr(L, name)
            f.argtypes = argt
            f.restype = C.c_int
        L.convrot_workspace_bytes.restype = C.c_size_t
        L.convrot_status_string.restype = C.c_char_p
        _lib = L
    return _lib


def status_string(status: int) -> str:
    return lib().convrot_status_string(int(status)).decode()


def _stream():
    return C.c_void_p(torch.cuda.current_stream().cuda_stream)


def _ptr(t):
    return None if t is None else C.c_void_p(t.data_ptr())


def _req(t: torch.Tensor, name: str, dtype, ndim: int):
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if t.device.type != "cuda":
        raise ValueError(f"{name} must be on the GPU")
    if t.dim() != ndim:
        raise ValueError(f"{name} must have {ndim} dims, got {tuple(t.shape)}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    return t


def _like(t, name: str, dtype, shape):
    """Check a tensor handed to the kernels: dtype, GPU, contiguous, exact shape."""
    _req(t, name, dtype, len(shape))
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")
    return t


def _out(t, name: str, dtype, shape, device):
    if t is None:
        return torch.empty(shape, dtype=dtype, device=device)
    return _like(t, name, dtype, shape)


def _ws(t, need: int, device):
    if t is None:
        return _workspace(need, device)
    _req(t, "workspace", torch.uint8, 1)
    if t.numel() < need:
        raise ValueError(f"workspace holds {t.numel()} bytes, {need} needed")
    return t


def _call(name: str, *args):
    st = getattr(lib(), name)(*args)
    if st != 0:
        raise ConvRotError(name, st)


def workspace_bytes(op: int, M: int, N: int, K: int, mode: int = 0) -> int:
    return int(lib().convrot_workspace_bytes(op, M, N, K, mode))


def _workspace(nbytes: int, device) -> torch.Tensor:
    return torch.empty(max(nbytes, 256), dtype=torch.uint8, device=device)


# --------------------------------------------------------------------------

def quantize_weight(w: torch.Tensor, block: int = BLOCK, chunk_rows: int = 0, out=None):
    """Load-time quantization of a bf16 weight [rows, cols] -> (int8 codes, fp32 scales)."""
    _req(w, "w", torch.bfloat16, 2)
    rows, cols = w.shape
    q0, s0 = out if out is not None else (None, None)
    q = _out(q0, "q", torch.int8, (rows, cols), w.device)
    s = _out(s0, "scale", torch.float32, (rows,), w.device)
    _call("convrot_quantize_weight", _ptr(w), rows, cols, block, chunk_rows, _ptr(q), _ptr(s),
          _stream())
    return q, s


def quantize_act(x: torch.Tensor, out=None):
    """Online activation rotation + per-row quantization -> (q_x, s_x)."""
    _req(x, "x", torch.bfloat16, 2)
    M, K = x.shape
    q0, s0 = out if out is not None else (None, None)
    q = _out(q0, "q", torch.int8, (M, K), x.device)
    s = _out(s0, "scale", torch.float32, (M,), x.device)
    _call("convrot_quantize_act", _ptr(x), M, K, _ptr(q), _ptr(s), _stream())
    return q, s


def linear_fwd(x, qw, sw, bias=None, out=None, workspace=None):
    """y = ConvRot-int8 linear of x [M, K] with (qw [N, K], sw [N]) -> bf16 [M, N]."""
    _req(x, "x", torch.bfloat16, 2)
    _req(qw, "qw", torch.int8, 2)
    _req(sw, "sw", torch.float32, 1)
    M, K = x.shape
    N = qw.shape[0]
    _like(qw, "qw", torch.int8, (N, K))
    _like(sw, "sw", torch.float32, (N,))
    if bias is not None:
        _like(bias, "bias", torch.bfloat16, (N,))
    y = _out(out, "out", torch.bfloat16, (M, N), x.device)
    ws = _ws(workspace, workspace_bytes(OP_LINEAR_FWD, M, N, K), x.device)
    _call("convrot_linear_fwd", _ptr(x), M, K, _ptr(qw), _ptr(sw), N, _ptr(bias), _ptr(y),
          _ptr(ws), ws.numel(), _stream())
    return y


def linear_fwd_noalloc(x, qw, sw, bias=None, out=None):
    """The forward without a workspace: q_x, s_x and any partial sums live in the
    library's static per-GPU scratch (NOALLOC_SCRATCH_BYTES).  Same result as
    linear_fwd bit for bit.  Calls that overlap in time on one GPU race.  With
    ``out`` given, the call allocates nothing."""
    _req(x, "x", torch.bfloat16, 2)
    _req(qw, "qw", torch.int8, 2)
    _req(sw, "sw", torch.float32, 1)
    M, K = x.shape
    N = qw.shape[0]
    _like(qw, "qw", torch.int8, (N, K))
    _like(sw, "sw", torch.float32, (N,))
    if bias is not None:
        _like(bias, "bias", torch.bfloat16, (N,))
    y = _out(out, "out", torch.bfloat16, (M, N), x.device)
    _call("convrot_linear_fwd_noalloc", _ptr(x), M, K, _ptr(qw), _ptr(sw), N, _ptr(bias), _ptr(y),
          _stream())
    return y


def linear_fwd_lora(x, qw, sw, lora_a, lora_b, lora_scale: float, bias=None, out=None,
                    workspace=None):
    """ConvRot-int8 linear plus a LoRA branch on the unrotated input:
    y = linear_fwd(x) + lora_scale * bf16(x . lora_a^T) . lora_b^T, one bf16 rounding.
    lora_a bf16 [R, K], lora_b bf16 [N, R], R in {16, 32}."""
    _req(x, "x", torch.bfloat16, 2)
    _req(qw, "qw", torch.int8, 2)
    _req(lora_a, "lora_a", torch.bfloat16, 2)
    M, K = x.shape
    N = qw.shape[0]
    R = lora_a.shape[0]
    _like(qw, "qw", torch.int8, (N, K))
    _like(sw, "sw", torch.float32, (N,))
    _like(lora_a, "lora_a", torch.bfloat16, (R, K))
    _like(lora_b, "lora_b", torch.bfloat16, (N, R))
    if bias is not None:
        _like(bias, "bias", torch.bfloat16, (N,))
    y = _out(out, "out", torch.bfloat16, (M, N), x.device)
    ws = _ws(workspace, workspace_bytes(OP_LINEAR_FWD_LORA, M, N, K, R), x.device)
    _call("convrot_linear_fwd_lora", _ptr(x), M, K, _ptr(qw), _ptr(sw), N, _ptr(bias),
          _ptr(lora_a), _ptr(lora_b), R, float(lora_scale), _ptr(y), _ptr(ws), ws.numel(),
          _stream())
    return y


def lora_down(x, lora_a):
    """First stage of the LoRA forward: xa = bf16(x . lora_a^T) [M, R]."""
    _req(x, "x", torch.bfloat16, 2)
    _req(lora_a, "lora_a", torch.bfloat16, 2)
    M, K = x.shape
    R = lora_a.shape[0]
    _like(lora_a, "lora_a", torch.bfloat16, (R, K))
    xa = torch.empty((M, R), dtype=torch.bfloat16, device=x.device)
    _call("convrot_lora_down", _ptr(x), M, K, _ptr(lora_a), R, _ptr(xa), _stream())
    return xa


def gemm_i8_bf16(qx, sx, qw, sw, bias=None, out=None):
    """Second stage of the forward: int8 GEMM + dequantizing epilogue."""
    _req(qx, "qx", torch.int8, 2)
    _req(qw, "qw", torch.int8, 2)
    M, K = qx.shape
    N = qw.shape[0]
    _like(qw, "qw", torch.int8, (N, K))
    _like(sx, "sx", torch.float32, (M,))
    _like(sw, "sw", torch.float32, (N,))
    if bias is not None:
        _like(bias, "bias", torch.bfloat16, (N,))
    y = _out(out, "out", torch.bfloat16, (M, N), qx.device)
    _call("convrot_gemm_i8_bf16", _ptr(qx), _ptr(sx), _ptr(qw), _ptr(sw), M, N, K, _ptr(bias),
          _ptr(y), _stream())
    return y


def gemm_i8_i32(a, b, b_layout: int = 0, out=None):
    """Raw int32 contraction (b_layout 0: b [N, K]; 1: b [K, N])."""
    _req(a, "a", torch.int8, 2)
    _req(b, "b", torch.int8, 2)
    M, K = a.shape
    if b_layout == 0:
        N = b.shape[0]
        _like(b, "b", torch.int8, (N, K))
    else:
        N = b.shape[1]
        _like(b, "b", torch.int8, (K, N))
    acc = _out(out, "out", torch.int32, (M, N), a.device)
    _call("convrot_gemm_i8_i32", _ptr(a), _ptr(b), M, N, K, b_layout, _ptr(acc), _stream())
    return acc


def bwd_quant_dy(dy, sw, out=None):
    """First stage of the int8 input gradient -> (q_g, s_g)."""
    _req(dy, "dy", torch.bfloat16, 2)
    _req(sw, "sw", torch.float32, 1)
    M, N = dy.shape
    _like(sw, "sw", torch.float32, (N,))
    q0, s0 = out if out is not None else (None, None)
    q = _out(q0, "q", torch.int8, (M, N), dy.device)
    s = _out(s0, "scale", torch.float32, (M,), dy.device)
    _call("convrot_bwd_quant_dy", _ptr(dy), M, N, _ptr(sw), _ptr(q), _ptr(s), _stream())
    return q, s


def linear_bwd_dx(dy, qw, sw, mode: int = BWD_BF16, out=None, workspace=None):
    """grad_x of the frozen ConvRot linear -> bf16 [M, K]."""
    _req(dy, "dy", torch.bfloat16, 2)
    _req(qw, "qw", torch.int8, 2)
    _req(sw, "sw", torch.float32, 1)
    M, N = dy.shape
    K = qw.shape[1]
    _like(qw, "qw", torch.int8, (N, K))
    _like(sw, "sw", torch.float32, (N,))
    dx = _out(out, "out", torch.bfloat16, (M, K), dy.device)
    ws = _ws(workspace, workspace_bytes(OP_LINEAR_BWD_DX, M, N, K, mode), dy.device)
    _call("convrot_linear_bwd_dx", _ptr(dy), M, N, _ptr(qw), _ptr(sw), K, mode, _ptr(dx),
          _ptr(ws), ws.numel(), _stream())
    return dx


def dequant_weight_t(qw, sw, out=None):
    """Transient bf16 weight of the bf16 input gradient, transposed: [K, N]."""
    _req(qw, "qw", torch.int8, 2)
    N, K = qw.shape
    _like(sw, "sw", torch.float32, (N,))
    out = _out(out, "out", torch.bfloat16, (K, N), qw.device)
    _call("convrot_dequant_weight_t", _ptr(qw), _ptr(sw), N, K, _ptr(out), _stream())
    return out


def embedding_lookup(ids, qe, se, oob_count=None, out=None):
    """Quantized embedding lookup with row dequantization and inverse rotation."""
    _req(ids, "ids", torch.int32, 1)
    _req(qe, "qe", torch.int8, 2)
    _req(se, "se", torch.float32, 1)
    T = ids.shape[0]
    V, D = qe.shape
    _like(se, "se", torch.float32, (V,))
    if oob_count is not None:
        _like(oob_count, "oob_count", torch.int32, (1,))
    o = _out(out, "out", torch.bfloat16, (T, D), qe.device)
    _call("convrot_embedding_lookup", _ptr(ids), T, _ptr(qe), _ptr(se), V, D, _ptr(o),
          _ptr(oob_count), _stream())
    return o
