"""PyTorch modules over the C ABI: the frozen ConvRot INT8 Linear and Embedding.

The pages describe the layer from the trainer's side ("LoRA Training Guide for
MOSS-Image", section 7.1, ConvRot INT8; sd-scripts pull request 2461, Summary,
utils and wiring bullets):

- the frozen base weights are rotated and quantized per row on the GPU when the
  model is loaded, and the bf16 weight is dropped;
- the patched Linear takes the unrotated activation and returns the unrotated
  output, so a LoRA branch wrapped around it sees the ordinary input;
- the base is frozen, so its backward returns the input gradient only, through
  the transient bf16 dequantization (default) or the int8 GEMM;
- the token embedding is quantized in row chunks, and its lookup returns rows
  dequantized and rotated back.

Everything here is argument marshalling (reshapes to 2-D, dtype checks, buffer
bookkeeping): each computation is one of the library's entry points.
"""
from __future__ import annotations

import torch

from . import BLOCK, BWD_BF16, BWD_INT8, embedding_lookup, linear_bwd_dx, linear_fwd, quantize_weight

__all__ = ["ConvRotLinear", "ConvRotEmbedding", "convrot_linear"]

_MODES = {"bf16": BWD_BF16, "int8": BWD_INT8, BWD_BF16: BWD_BF16, BWD_INT8: BWD_INT8}


class _ConvRotLinearFn(torch.autograd.Function):
    """y = convrot_linear_fwd(x); grad_x = convrot_linear_bwd_dx(grad_y).

    The codes, scales and bias are frozen: they receive no gradient."""

    @staticmethod
    def forward(ctx, x2, qw, sw, bias, mode):
        ctx.save_for_backward(qw, sw)
        ctx.mode = mode
        return linear_fwd(x2, qw, sw, bias)

    @staticmethod
    def backward(ctx, gy):
        qw, sw = ctx.saved_tensors
        gx = None
        if ctx.needs_input_grad[0]:
            gx = linear_bwd_dx(gy.contiguous(), qw, sw, ctx.mode)
        return gx, None, None, None, None


def _check_act(x: torch.Tensor):
    # sd-scripts pull request 2461 lists, among its fixes, activations that were
    # cast to the int8 weight's dtype; the layer keeps bf16 activations and
    # refuses every other dtype instead of converting.
    if x.dtype != torch.bfloat16:
        raise TypeError(f"ConvRot INT8 layers take bf16 activations, got {x.dtype}")


def convrot_linear(x: torch.Tensor, qw: torch.Tensor, sw: torch.Tensor, bias=None,
                   bwd_mode="bf16") -> torch.Tensor:
    """Functional form of ConvRotLinear: x [..., K] bf16 -> y [..., N] bf16, with
    autograd through the input only."""
    _check_act(x)
    mode = _MODES[bwd_mode]
    K = qw.shape[1]
    if x.shape[-1] != K:
        raise ValueError(f"x has {x.shape[-1]} input features, the layer {K}")
    lead = x.shape[:-1]
    x2 = x.reshape(-1, K)
    if not x2.is_contiguous():
        x2 = x2.contiguous()
    y2 = _ConvRotLinearFn.apply(x2, qw, sw, bias, mode)
    return y2.reshape(*lead, qw.shape[0])


class ConvRotLinear(torch.nn.Module):
    """Frozen Linear with ConvRot INT8 weights: codes q_w [N, K] int8 and row
    scales s_w [N] fp32 in the rotated basis, optional bf16 bias [N].

    ``bwd_mode`` picks the input gradient: "bf16" (transient bf16 dequantization,
    the pages' default) or "int8" (the int8 GEMM)."""

    def __init__(self, qw: torch.Tensor, sw: torch.Tensor, bias=None, bwd_mode="bf16"):
        super().__init__()
        if bwd_mode not in _MODES:
            raise ValueError(f"bwd_mode must be 'bf16' or 'int8', got {bwd_mode!r}")
        if qw.dtype != torch.int8 or qw.dim() != 2 or qw.shape[1] % BLOCK:
            raise ValueError("qw must be int8 [N, K] with K a multiple of 128")
        if sw.dtype != torch.float32 or tuple(sw.shape) != (qw.shape[0],):
            raise ValueError("sw must be float32 [N]")
        if bias is not None and (bias.dtype != torch.bfloat16 or tuple(bias.shape) != (qw.shape[0],)):
            raise ValueError("bias must be bf16 [N]")
        self.bwd_mode = bwd_mode
        self.register_buffer("qw", qw)
        self.register_buffer("sw", sw)
        self.register_buffer("bias", bias)

    @property
    def in_features(self) -> int:
        return self.qw.shape[1]

    @property
    def out_features(self) -> int:
        return self.qw.shape[0]

    @classmethod
    def from_linear(cls, linear: torch.nn.Linear, bwd_mode="bf16") -> "ConvRotLinear":
        """Load-time conversion: the bf16 weight (on the GPU) is rotated and
        quantized per row by convrot_quantize_weight; the bias is kept in bf16."""
        w = linear.weight.detach()
        if w.dtype != torch.bfloat16:
            raise TypeError(f"the weight must be bf16, got {w.dtype}")
        qw, sw = quantize_weight(w.contiguous())
        b = linear.bias.detach().contiguous() if linear.bias is not None else None
        return cls(qw, sw, b, bwd_mode)

    def forward(self, x: torch.Tensor) -> torch.Tensor:
        return convrot_linear(x, self.qw, self.sw, self.bias, self.bwd_mode)

    def extra_repr(self) -> str:
        return (f"in_features={self.in_features}, out_features={self.out_features}, "
                f"bias={self.bias is not None}, bwd_mode={self.bwd_mode}")


class ConvRotEmbedding(torch.nn.Module):
    """Frozen token embedding stored as ConvRot INT8 rows: codes q_E [V, D] int8
    and row scales s_E [V] fp32 in the rotated basis.  The lookup returns
    bf16((s_E[id] * q_E[id]) R).

    An id outside [0, V) gives a zero row.  With ``check_ids`` the module also
    counts such ids on the GPU and raises after the lookup (one host
    synchronization per call), as torch.nn.Embedding would."""

    def __init__(self, qe: torch.Tensor, se: torch.Tensor, check_ids: bool = False):
        super().__init__()
        if qe.dtype != torch.int8 or qe.dim() != 2 or qe.shape[1] % BLOCK:
            raise ValueError("qe must be int8 [V, D] with D a multiple of 128")
        if se.dtype != torch.float32 or tuple(se.shape) != (qe.shape[0],):
            raise ValueError("se must be float32 [V]")
        self.check_ids = check_ids
        self.register_buffer("qe", qe)
        self.register_buffer("se", se)

    @property
    def num_embeddings(self) -> int:
        return self.qe.shape[0]

    @property
    def embedding_dim(self) -> int:
        return self.qe.shape[1]

    @classmethod
    def from_embedding(cls, emb: torch.nn.Embedding, chunk_rows: int = 8192,
                       check_ids: bool = False) -> "ConvRotEmbedding":
        """Load-time conversion, quantized in chunks of ``chunk_rows`` rows (the
        result is the same for any chunk size)."""
        w = emb.weight.detach()
        if w.dtype != torch.bfloat16:
            raise TypeError(f"the embedding must be bf16, got {w.dtype}")
        qe, se = quantize_weight(w.contiguous(), chunk_rows=chunk_rows)
        return cls(qe, se, check_ids)

    def forward(self, ids: torch.Tensor) -> torch.Tensor:
        if ids.dtype not in (torch.int32, torch.int64):
            raise TypeError(f"ids must be int32 or int64, got {ids.dtype}")
        flat = ids.reshape(-1)
        if flat.dtype != torch.int32:
            # int64 ids beyond the int32 range would wrap into [0, V) when
            # narrowed; clamping to [-1, V] first keeps every bad id out of range
            flat = flat.clamp(-1, self.num_embeddings).to(torch.int32)
        flat = flat.contiguous()
        oob = torch.zeros(1, dtype=torch.int32, device=flat.device) if self.check_ids else None
        out = embedding_lookup(flat, self.qe, self.se, oob)
        if oob is not None and int(oob.item()) != 0:
            raise IndexError(f"{int(oob.item())} token ids outside [0, {self.num_embeddings})")
        return out.reshape(*ids.shape, self.embedding_dim)

    def extra_repr(self) -> str:
        return f"{self.num_embeddings}, {self.embedding_dim}"
