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


BF16_NAN, BF16_INF, BF16_NINF, BF16_MAX = 0x7FC0, 0x7F80, 0xFF80, 0x7F7F


def nonfinite_rows(K: int, seed: int = 0):
    """bf16 rows (K a multiple of 128) that are not finite after the rotation,
    each among ordinary N(0, 1) values, followed by one ordinary row:
      * a NaN input in the last block;
      * +inf in the first block; -inf in the middle;
      * +inf and -inf in one block (its sums are NaN);
      * a whole block of bf16's largest finite value (3.39e38): its rotated sum
        128 * 3.39e38 / sqrt(128) overflows fp32 to +inf;
      * every element NaN."""
    g = np.random.default_rng(seed)
    base = wl.f32_to_bf16_bits(g.standard_normal((7, K)).astype(np.float32))
    rows = base.copy()
    rows[0, K - 5] = BF16_NAN
    rows[1, 3] = BF16_INF
    rows[2, K // 2 + 7] = BF16_NINF
    rows[3, 10] = BF16_INF
    rows[3, 100] = BF16_NINF
    rows[4, 128:256 if K >= 256 else 128] = BF16_MAX
    if K < 256:
        rows[4, :128] = BF16_MAX
    rows[5, :] = BF16_NAN
    return rows  # row 6 stays ordinary


def nonfinite_fold_rows(N: int, seed: int = 0):
    """dY rows and column scales whose fold r = fl32(dY) * s_w is not finite in
    some column (NaN, +-inf inputs; a finite 2^100 times a column scale of 2^40,
    which overflows fp32), followed by one ordinary row."""
    g = np.random.default_rng(seed)
    dy = wl.f32_to_bf16_bits(g.standard_normal((5, N)).astype(np.float32))
    sw = np.full(N, 2.0 ** -3, np.float32)
    dy[0, N - 1] = BF16_NAN
    dy[1, 0] = BF16_INF
    dy[2, N // 3] = BF16_NINF
    dy[3, 7] = wl.f32_to_bf16_bits(np.float32([2.0 ** 100]))[0]
    sw[7] = np.float32(2.0 ** 40)
    return dy, sw  # row 4 stays ordinary (its column 7 folds to a finite value)


def crafted_rows(K: int) -> np.ndarray:
    """Rows that pin the quantizer's corner cases, tiled over all blocks of K."""
    def tile(entries, scale=1.0):
        v = np.zeros(K, dtype=np.float32)
        for b0 in range(0, K, 128):
            for i, val in entries.items():
                v[b0 + i] = val * scale
        return v
    rows = [
        np.zeros(K, np.float32),                          # all-zero row
        tile({0: -253.0, 1: -255.0}),                     # exact tie at 0.5
        tile({0: 3.0, 1: 1.0}),                           # exact tie at 63.5
        tile({0: -255.0, 1: -85.0}),                      # division vs reciprocal
        tile({0: 1.0}),                                   # e0
        tile({i: 1.0 for i in range(128)}),               # ones
        tile({1: 1.0}), tile({64: -1.0}),
        tile({0: 2.0 ** 20, 1: 2.0 ** -10, 77: -3.0}),    # wide but exact spread
        tile({3: 1e-32, 9: -2e-32}),                      # tiny scale (IEEE division path)
        tile({5: 1e36, 6: -3e35}),                        # huge scale (IEEE division path)
    ]
    return wl.f32_to_bf16_bits(np.stack(rows))
