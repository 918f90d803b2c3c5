"""Seeded synthetic inputs for the ConvRot INT8 linear workloads.

This module only draws random numbers and rounds them to bf16 bit patterns; it
holds none of the method's arithmetic.  Both the oracle and the GPU path are fed
from here, so the two sides always see the same bits.

Recipe (numpy ``Generator(PCG64(seed))``, one stream per tensor, seed =
1000 * base + index with x=0, W=1, W_down=2, dY=3, dY2=4, outlier choice=5,
ids=6, sequence lengths=7):
  * normals are drawn as float32 ``standard_normal`` times sigma, then rounded
    to bf16 (round half to even) on the bit pattern;
  * outlier channels: a seeded choice without replacement of ``n_out`` columns,
    multiplied by 50 before the bf16 rounding (4 columns for the tiny layer,
    round(1% of K) = 41 for K = 4096);
  * token ids are ``integers(0, V, T, int32)``;
  * packed variable-length batch: lengths uniform on [1024, 4096] drawn until
    the total reaches the token count, the last one truncated.

The five workloads (token batches shaped like a 1024x1024 DiT image at 16x
downscale = 4096 tokens, hidden size 4096, 42 blocks x 6 projections):
  tiny   x [64,256] (4 outlier cols), W [256,256]                       (fwd + dX)
  attn   x [4096,4096] (41 outlier cols), W [4096,4096]                 (fwd)
  mlp    x [4096,4096], W_up [16384,4096], W_down [4096,16384]; the down input
         is the bf16 GELU of the unquantized up projection; dY ~ N(0,1e-3)
  packed x [20480,4096], 252 weights [4096,4096] streamed; dY ~ N(0,1e-3)
  embed  E [248320,4096] ~ N(0,0.02) quantized in 8192-row chunks; 32768 ids
"""
from __future__ import annotations

import math

import numpy as np

SIGMA_W = 0.02
SIGMA_DY = 1e-3
OUTLIER_GAIN = 50.0

S_X, S_W, S_WDOWN, S_DY, S_DY2, S_OUT, S_IDS, S_SEQ = range(8)


def rng(base: int, index: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(1000 * base + index))


def f32_to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """Round float32 values to bf16 (nearest, ties to even) on the bit pattern."""
    a = np.ascontiguousarray(a, dtype=np.float32)
    u = a.view(np.uint32)
    lsb = (u >> np.uint32(16)) & np.uint32(1)
    r = (u + np.uint32(0x7FFF) + lsb) >> np.uint32(16)
    nan = np.isnan(a)
    out = r.astype(np.uint16)
    if nan.any():
        out[nan] = 0x7FC0
    return out


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    return (np.ascontiguousarray(b, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(
        np.float32)


def normal_bf16(shape, sigma: float, base: int, index: int, chunk: int = 1 << 24) -> np.ndarray:
    """bf16 bits of N(0, sigma) draws, generated in chunks to bound memory."""
    g = rng(base, index)
    n = int(np.prod(shape))
    out = np.empty(n, dtype=np.uint16)
    for i in range(0, n, chunk):
        m = min(chunk, n - i)
        v = g.standard_normal(m, dtype=np.float32)
        if sigma != 1.0:
            v *= np.float32(sigma)
        out[i:i + m] = f32_to_bf16_bits(v)
    return out.reshape(shape)


def outlier_columns(K: int, n_out: int, base: int) -> np.ndarray:
    return np.sort(rng(base, S_OUT).choice(K, size=n_out, replace=False)).astype(np.int64)


def activations(M: int, K: int, n_out: int, base: int = 0, index: int = S_X) -> np.ndarray:
    """x ~ N(0,1) with ``n_out`` whole columns scaled by 50 before bf16 rounding."""
    g = rng(base, index)
    cols = outlier_columns(K, n_out, base) if n_out else np.zeros(0, np.int64)
    out = np.empty((M, K), dtype=np.uint16)
    step = max(1, (1 << 24) // K)
    for r0 in range(0, M, step):
        r1 = min(M, r0 + step)
        v = g.standard_normal((r1 - r0, K), dtype=np.float32)
        if cols.size:
            v[:, cols] *= np.float32(OUTLIER_GAIN)
        out[r0:r1] = f32_to_bf16_bits(v)
    return out


def n_outliers(K: int) -> int:
    return int(round(0.01 * K))


def seqlens(total: int, base: int = 0, lo: int = 1024, hi: int = 4096) -> np.ndarray:
    g = rng(base, S_SEQ)
    out = []
    s = 0
    while s < total:
        L = int(g.integers(lo, hi + 1))
        L = min(L, total - s)
        out.append(L)
        s += L
    return np.asarray(out, dtype=np.int64)


def token_ids(T: int, V: int, base: int = 0) -> np.ndarray:
    return rng(base, S_IDS).integers(0, V, T, dtype=np.int32)


def gelu_erf_bf16(y_f32: np.ndarray) -> np.ndarray:
    """bf16 bits of the exact-erf GELU of float32 values (the MLP's down input)."""
    from scipy.special import erf
    y = np.asarray(y_f32, dtype=np.float64)
    g = 0.5 * y * (1.0 + erf(y / math.sqrt(2.0)))
    return f32_to_bf16_bits(g.astype(np.float32))


# --------------------------------------------------------------------------
# The five workloads
# --------------------------------------------------------------------------

def tiny(base: int = 0) -> dict:
    M, K, N = 64, 256, 256
    return dict(
        x=activations(M, K, 4, base),
        w=normal_bf16((N, K), SIGMA_W, base, S_W),
        dy=normal_bf16((M, N), SIGMA_DY, base, S_DY),
        M=M, K=K, N=N)


def attn(base: int = 0) -> dict:
    M = K = N = 4096
    return dict(x=activations(M, K, n_outliers(K), base),
                w=normal_bf16((N, K), SIGMA_W, base, S_W), M=M, K=K, N=N)


def mlp_weights(base: int = 0) -> dict:
    D, F = 4096, 16384
    return dict(w_up=normal_bf16((F, D), SIGMA_W, base, S_W),
                w_down=normal_bf16((D, F), SIGMA_W, base, S_WDOWN), D=D, F=F)


def mlp_down_input(x_bits: np.ndarray, w_up_bits: np.ndarray, matmul=None) -> np.ndarray:
    """Down-projection input: bf16 GELU(erf) of the unquantized up projection
    x * W_up^T evaluated in float32 (the generator must not depend on either
    implementation under test).  ``matmul`` may supply a float32 matmul."""
    xf = bf16_bits_to_f32(x_bits)
    wf = bf16_bits_to_f32(w_up_bits)
    y = matmul(xf, wf) if matmul is not None else xf @ wf.T
    return gelu_erf_bf16(np.asarray(y, dtype=np.float32))


def mlp_grads(M: int = 4096, base: int = 0) -> dict:
    D, F = 4096, 16384
    return dict(dy_down=normal_bf16((M, D), SIGMA_DY, base, S_DY),
                dy_up=normal_bf16((M, F), SIGMA_DY, base, S_DY2))


def packed(base: int = 0, layers: int = 252) -> dict:
    T, K, N = 20480, 4096, 4096
    return dict(seqlens=seqlens(T, base), x=activations(T, K, n_outliers(K), base),
                dy=normal_bf16((T, N), SIGMA_DY, base, S_DY), M=T, K=K, N=N, layers=layers)


def packed_weight(layer: int, base: int = 0, N: int = 4096, K: int = 4096) -> np.ndarray:
    """Fresh random weight of one of the streamed layers (its own seed stream)."""
    g = np.random.Generator(np.random.PCG64([1000 * base + S_W, layer]))
    out = np.empty((N, K), dtype=np.uint16)
    step = max(1, (1 << 24) // K)
    for r0 in range(0, N, step):
        r1 = min(N, r0 + step)
        v = g.standard_normal((r1 - r0, K), dtype=np.float32) * np.float32(SIGMA_W)
        out[r0:r1] = f32_to_bf16_bits(v)
    return out


def qkv_weights(base: int = 0, N: int = 4096, K: int = 4096) -> list:
    """The q, k and v projection weights that share one input (their own seed
    streams, disjoint from the streamed layers')."""
    return [packed_weight(1000 + j, base, N, K) for j in range(3)]


def lora_weights(K: int, N: int, R: int, base: int = 0) -> dict:
    """A trained-looking LoRA pair on its own seed streams: down A [R, K] and up
    B [N, R], both ~N(0, 0.02) in bf16 (an untrained up projection would be 0)."""
    g = np.random.Generator(np.random.PCG64([1000 * base + S_W, 2000 + R]))
    a = f32_to_bf16_bits(g.standard_normal((R, K), dtype=np.float32) * np.float32(SIGMA_W))
    b = f32_to_bf16_bits(g.standard_normal((N, R), dtype=np.float32) * np.float32(SIGMA_W))
    return dict(a=a, b=b)


EMBED_V, EMBED_D, EMBED_CHUNK, EMBED_T = 248320, 4096, 8192, 32768


def text_encoder_linear_shapes() -> list:
    """[rows, cols] of the text encoder's 200 quantized Linear layers, a stand-in:
    the pages give the count (200 Linear layers and the token embedding, about
    15.9 GB in bf16) and the hidden size 4096, not the layer shapes.  The stand-in
    follows the module list the pages name (8 full-attention layers with q/k/v/o,
    24 linear-attention layers with in_proj_qkv, in_proj_z and out_proj -- their
    32-output in_proj_a/b stay out of the 200 -- and 32 MLPs with gate/up/down)
    with widths chosen so that the 200 layers hold ~6.98 G parameters, the page's
    total less the 248320 x 4096 embedding."""
    D, F, QKV = 4096, 12288, 8192
    shapes = []
    for _ in range(8):
        shapes += [[D, D]] * 4                      # q, k, v, o
    for _ in range(24):
        shapes += [[QKV, D], [D, D], [D, D]]        # in_proj_qkv, in_proj_z, out_proj
    for _ in range(32):
        shapes += [[F, D], [F, D], [D, F]]          # gate, up, down
    return shapes


def embed_table(base: int = 0, V: int = EMBED_V, D: int = EMBED_D) -> np.ndarray:
    return normal_bf16((V, D), SIGMA_W, base, S_W)


def embed_ids(base: int = 0, T: int = EMBED_T, V: int = EMBED_V) -> np.ndarray:
    return token_ids(T, V, base)
