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


def assert_fwd_elementwise(gpu_bits: np.ndarray, ref_bits: np.ndarray, what: str):
    """Forward outputs without bias, element by element: the GPU's fp32 chain
    fl32(fl32(fl32(acc) * s_w) * s_x) is within 3 * 2^-24 (relative) of the exact
    product, so after both sides round to bf16 they differ by at most one bf16
    ulp of the reference, i.e. |gpu - ref| <= 2^-7 * |ref|; an exact zero stays
    zero."""
    assert gpu_bits.shape == ref_bits.shape, (what, gpu_bits.shape, ref_bits.shape)
    g = wl.bf16_bits_to_f32(gpu_bits).astype(np.float64)
    r = wl.bf16_bits_to_f32(ref_bits).astype(np.float64)
    bad = np.argwhere(np.abs(g - r) > 2.0 ** -7 * np.abs(r) + 1e-37)
    assert bad.size == 0, (f"{what}: {len(bad)} elements beyond one bf16 ulp, first "
                           f"{bad[:3].tolist()}")


CANARY = 0x5A


class Guarded:
    """A device tensor with canary bands of ``band`` bytes on both sides, to
    catch writes past either end of an output.  ``t`` is the tensor handed to
    the kernels (16-byte aligned: the band is a multiple of 256 bytes)."""

    def __init__(self, shape, dtype, band: int = 4096):
        assert band % 256 == 0
        n = int(np.prod(shape)) if len(shape) else 1
        self.nbytes = n * torch.empty((), dtype=dtype).element_size()
        self.band = band
        self.raw = torch.full((band + self.nbytes + band,), CANARY, dtype=torch.uint8, device=dev())
        self.t = self.raw[band:band + self.nbytes].view(dtype).view(*shape)

    def check(self, what: str):
        torch.cuda.synchronize()
        lo = self.raw[:self.band]
        hi = self.raw[self.band + self.nbytes:]
        assert bool((lo == CANARY).all()), f"{what}: bytes before the buffer were written"
        assert bool((hi == CANARY).all()), f"{what}: bytes after the buffer were written"


def guarded_workspace(nbytes: int, band: int = 4096) -> Guarded:
    return Guarded((max(nbytes, 256),), torch.uint8, band)
