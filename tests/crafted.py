"""Crafted quantizer inputs shared by the CPU emulation tests and the GPU
parity tests (plain numpy: seeded draws and exact powers of two, none of the
method's arithmetic)."""
import numpy as np

import workloads as wl


def tiny_fold_rows(N: int, seed: int = 0):
    """dY rows whose folded maxima (s_w = 2^-20) sweep the subnormal binades of
    fp32 and the underflow to a zero scale:
      * N(0, 2^e) rows for e = -130 .. -105 (folded maxima ~2^-148 .. 2^-123);
      * rows whose maximum folds to j * 2^-142 = 128 j * 2^-149, j = 1 .. 63:
        a / 127 = j + j/127 rounds to j, so the maximum's quotient is exactly 128
        (the clamp's case), with random smaller elements beside it;
      * a row of 2^-120 everywhere (quotient 128 in every column) and rows whose
        maximum folds below 127 * 2^-150 (zero scale)."""
    g = np.random.default_rng(seed)
    rows = []
    for e in range(-130, -104):
        rows.append(g.standard_normal(N).astype(np.float32) * np.float32(2.0 ** e))
    for j in range(1, 64, 2):
        v = g.uniform(-1, 1, N).astype(np.float32) * np.float32(j * 2.0 ** -122)
        v[g.integers(N)] = np.float32(j * 2.0 ** -122)
        v[g.integers(N)] = np.float32(-j * 2.0 ** -122)
        rows.append(v)
    rows.append(np.full(N, 2.0 ** -120, np.float32))
    for e in (-124, -125, -127):
        rows.append(g.uniform(-1, 1, N).astype(np.float32) * np.float32(2.0 ** e))
    return wl.f32_to_bf16_bits(np.stack(rows)), np.full(N, 2.0 ** -20, np.float32)
