"""Helpers shared by the GPU parity tests: host<->device transfer of bf16 bit
patterns and the comparison rules.

Comparison rules (the layer's parity bar):
  * int8 codes, fp32 scales and int32 accumulators: bit-exact;
  * bf16 outputs: per row, max |gpu - ref| <= 1e-2 * max |ref| (a row whose
    reference is all zero must be exactly zero).
"""
import numpy as np
import torch

import workloads as wl

ROW_TOL = 1e-2


def dev():
    return torch.device("cuda:0")


def bf16_to_dev(a: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).to(dev())


def to_dev(a: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a)).to(dev())


def bits(t: torch.Tensor) -> np.ndarray:
    return t.detach().cpu().contiguous().view(torch.int16).numpy().view(np.uint16)


def host(t: torch.Tensor) -> np.ndarray:
    return t.detach().cpu().numpy()


def assert_exact(gpu: np.ndarray, ref: np.ndarray, what: str):
    assert gpu.shape == ref.shape, (what, gpu.shape, ref.shape)
    if gpu.dtype == np.float32:
        g, r = gpu.view(np.uint32), ref.view(np.uint32)
    else:
        g, r = gpu, ref
    bad = np.argwhere(g != r)
    assert bad.size == 0, f"{what}: {len(bad)} mismatches, first at {bad[:5].tolist()}"


def row_errors(gpu_bits: np.ndarray, ref_bits: np.ndarray) -> np.ndarray:
    g = wl.bf16_bits_to_f32(gpu_bits).astype(np.float64)
    r = wl.bf16_bits_to_f32(ref_bits).astype(np.float64)
    err = np.max(np.abs(g - r), axis=1)
    scale = np.max(np.abs(r), axis=1)
    out = np.where(scale > 0, err / np.where(scale > 0, scale, 1.0), np.where(err > 0, np.inf, 0.0))
    return out


def assert_rows_close(gpu_bits: np.ndarray, ref_bits: np.ndarray, what: str, tol: float = ROW_TOL):
    assert gpu_bits.shape == ref_bits.shape, (what, gpu_bits.shape, ref_bits.shape)
    e = row_errors(gpu_bits, ref_bits)
    worst = int(np.argmax(e))
    assert np.all(e <= tol), f"{what}: row {worst} relative error {e[worst]:.3e} > {tol}"
    return float(e.max())
