"""Host-side checks of the C ABI (no GPU needed): the library loads, exports every
symbol declared in include/convrot.h, and rejects bad arguments with the
documented status codes before anything is launched."""
import ctypes as C
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "convrot.h")


@pytest.fixture(scope="module")
def cr():
    import w8a8_rotated_int8_amd as cr
    if not os.path.exists(cr.library_path):
        from w8a8_rotated_int8_amd import build
        build.build()
    cr.lib()
    return cr


def declared_symbols():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"^\s*(?:int|size_t|const char\*)\s+(convrot_\w+)\s*\(", text, re.M)))


def test_header_declares_the_four_entry_points():
    syms = declared_symbols()
    for s in ("convrot_quantize_weight", "convrot_linear_fwd", "convrot_linear_bwd_dx",
              "convrot_embedding_lookup"):
        assert s in syms


def test_library_exports_every_declared_symbol(cr):
    L = C.CDLL(cr.library_path)
    syms = declared_symbols()
    assert len(syms) >= 11
    for s in syms:
        assert hasattr(L, s), s
    assert sorted(cr.EXPORTS) == syms


def test_status_strings(cr):
    for code in (0, -1, -2, -3, -4, -5, -6):
        assert cr.status_string(code) != "unknown status"
    assert cr.status_string(7) == "unknown status"


def test_workspace_sizes(cr):
    M, N, K = 4096, 4096, 4096
    assert cr.workspace_bytes(cr.OP_LINEAR_FWD, M, N, K) == M * K + 4 * M
    assert cr.workspace_bytes(cr.OP_LINEAR_BWD_DX, M, N, K, cr.BWD_INT8) == M * N + 4 * M
    assert cr.workspace_bytes(cr.OP_LINEAR_BWD_DX, M, N, K, cr.BWD_BF16) == 2 * N * K
    assert cr.workspace_bytes(cr.OP_LINEAR_FWD, 0, N, K) == 0
    assert cr.workspace_bytes(9, M, N, K) == 0
    # LoRA forward: the forward's q_x / s_x plus xa [M, R] bf16; R in {16, 32}
    for R in (16, 32):
        assert cr.workspace_bytes(cr.OP_LINEAR_FWD_LORA, M, N, K, R) == M * K + 4 * M + 2 * M * R
    assert cr.workspace_bytes(cr.OP_LINEAR_FWD_LORA, M, N, K, 8) == 0


# Fake, well-aligned, never-dereferenced device addresses: validation must reject
# these calls before any HIP call or launch.
A = C.c_void_p(1 << 20)
B = C.c_void_p(2 << 20)
Y = C.c_void_p(3 << 20)
WS = C.c_void_p(4 << 20)


def test_null_pointers_are_einval(cr):
    L = cr.lib()
    assert L.convrot_linear_fwd(None, 4, 128, B, B, 4, None, Y, WS, 1 << 20, None) == -1
    assert L.convrot_quantize_weight(None, 4, 128, 128, 0, B, Y, None) == -1
    assert L.convrot_embedding_lookup(None, 4, B, B, 10, 128, Y, None, None) == -1
    assert L.convrot_linear_bwd_dx(A, 4, 128, None, B, 128, 0, Y, WS, 1 << 20, None) == -1
    assert L.convrot_linear_fwd_lora(A, 4, 128, B, B, 4, None, None, B, 16, 1.0, Y, WS, 1 << 20,
                                     None) == -1


def test_bad_sizes_and_shapes(cr):
    L = cr.lib()
    assert L.convrot_linear_fwd(A, -1, 128, B, B, 4, None, Y, WS, 1 << 20, None) == -1
    assert L.convrot_linear_fwd(A, 4, 128, B, B, 0, None, Y, WS, 1 << 20, None) == -1
    assert L.convrot_linear_fwd(A, 4, 100, B, B, 4, None, Y, WS, 1 << 20, None) == -2
    assert L.convrot_linear_fwd(A, 4, 128 * 257, B, B, 4, None, Y, WS, 1 << 30, None) == -2
    assert L.convrot_quantize_weight(A, 4, 128, 64, 0, B, Y, None) == -2
    assert L.convrot_quantize_weight(A, 4, 130, 128, 0, B, Y, None) == -2
    assert L.convrot_embedding_lookup(A, 4, B, B, 10, 96, Y, None, None) == -2
    assert L.convrot_linear_bwd_dx(A, 4, 100, B, B, 128, 0, Y, WS, 1 << 20, None) == -2
    assert L.convrot_linear_bwd_dx(A, 4, 128, B, B, 128, 2, Y, WS, 1 << 20, None) == -1
    assert L.convrot_gemm_i8_i32(A, B, 4, 100, 128, 1, Y, None) == -2
    assert L.convrot_gemm_i8_i32(A, B, 4, 100, 128, 3, Y, None) == -1
    # LoRA rank must be 16 or 32; the workspace must hold q_x, s_x and xa
    assert L.convrot_linear_fwd_lora(A, 4, 128, B, B, 4, None, A, B, 8, 1.0, Y, WS, 1 << 20,
                                     None) == -2
    assert L.convrot_linear_fwd_lora(A, 4, 128, B, B, 4, None, A, B, 16, 1.0, Y, WS, 512,
                                     None) == -3


def test_empty_batch_is_a_no_op(cr):
    """A batch of 0 rows / tokens / ids enqueues nothing and touches no pointer
    (all NULL here, no stream, no GPU); the other sizes are still checked."""
    L = cr.lib()
    assert L.convrot_quantize_weight(None, 0, 256, 128, 0, None, None, None) == 0
    assert L.convrot_quantize_weight(None, 0, 256, 64, 0, None, None, None) == -2
    assert L.convrot_quantize_act(None, 0, 4096, None, None, None) == 0
    assert L.convrot_quantize_act(None, 0, 100, None, None, None) == -2
    assert L.convrot_bwd_quant_dy(None, 0, 4096, None, None, None, None) == 0
    assert L.convrot_linear_fwd(None, 0, 4096, None, None, 4096, None, None, None, 0, None) == 0
    assert L.convrot_linear_fwd(None, 0, 4000, None, None, 4096, None, None, None, 0, None) == -2
    assert L.convrot_linear_fwd(None, 0, 4096, None, None, 0, None, None, None, 0, None) == -1
    assert L.convrot_linear_fwd_lora(None, 0, 4096, None, None, 4096, None, None, None, 16, 1.0,
                                     None, None, 0, None) == 0
    assert L.convrot_linear_fwd_lora(None, 0, 4096, None, None, 4096, None, None, None, 8, 1.0,
                                     None, None, 0, None) == -2
    assert L.convrot_lora_down(None, 0, 4096, None, 32, None, None) == 0
    assert L.convrot_gemm_i8_bf16(None, None, None, None, 0, 256, 256, None, None, None) == 0
    assert L.convrot_gemm_i8_i32(None, None, 0, 256, 256, 1, None, None) == 0
    assert L.convrot_gemm_i8_i32(None, None, 0, 100, 256, 1, None, None) == -2
    for mode in (0, 1):
        assert L.convrot_linear_bwd_dx(None, 0, 4096, None, None, 4096, mode, None, None, 0,
                                       None) == 0
    assert L.convrot_linear_bwd_dx(None, 0, 4096, None, None, 4096, 2, None, None, 0, None) == -1
    assert L.convrot_embedding_lookup(None, 0, None, None, 10, 128, None, None, None) == 0
    assert L.convrot_embedding_lookup(None, 0, None, None, 10, 96, None, None, None) == -2
    for op, mode in ((cr.OP_LINEAR_FWD, 0), (cr.OP_LINEAR_FWD_LORA, 16),
                     (cr.OP_LINEAR_BWD_DX, cr.BWD_INT8)):
        assert cr.workspace_bytes(op, 0, 4096, 4096, mode) == 0


def test_misalignment_is_einval(cr):
    L = cr.lib()
    odd = C.c_void_p((1 << 20) + 2)
    assert L.convrot_linear_fwd(odd, 4, 128, B, B, 4, None, Y, WS, 1 << 20, None) == -1
    ws_odd = C.c_void_p((4 << 20) + 16)
    assert L.convrot_linear_fwd(A, 4, 128, B, B, 4, None, Y, ws_odd, 1 << 20, None) == -1


def test_workspace_too_small(cr):
    L = cr.lib()
    need = cr.workspace_bytes(cr.OP_LINEAR_FWD, 64, 256, 256)
    assert L.convrot_linear_fwd(A, 64, 256, B, B, 256, None, Y, WS, need - 1, None) == -3
    need = cr.workspace_bytes(cr.OP_LINEAR_BWD_DX, 64, 256, 256, cr.BWD_INT8)
    assert L.convrot_linear_bwd_dx(A, 64, 256, B, B, 256, 1, Y, WS, need - 1, None) == -3


def test_binding_fails_loudly_without_library(cr, monkeypatch, tmp_path):
    import importlib
    monkeypatch.setattr(cr, "_lib", None)
    monkeypatch.setattr(cr, "library_path", str(tmp_path / "missing.so"))
    with pytest.raises(ImportError):
        cr.lib()


def _odd(p, by=4):
    return C.c_void_p(p.value + by)


def test_every_pointer_alignment_is_checked(cr):
    """Each pointer the header promises 16-byte aligned is checked: the same
    call with one pointer moved by 4 bytes is CONVROT_EINVAL (and nothing is
    launched: the addresses are fake and there is no GPU)."""
    L = cr.lib()
    WS1 = 1 << 20
    # (function, args with each pointer a placeholder name)
    calls = {
        "convrot_quantize_weight": (["w", 64, 256, 128, 0, "q", "s", None], ["w", "q", "s"]),
        "convrot_quantize_act": (["x", 64, 256, "q", "s", None], ["x", "q", "s"]),
        "convrot_bwd_quant_dy": (["dy", 64, 256, "sw", "q", "s", None], ["dy", "sw", "q", "s"]),
        "convrot_gemm_i8_bf16": (["qx", "sx", "qw", "sw", 64, 256, 256, "bias", "y", None],
                                 ["qx", "sx", "qw", "sw", "bias", "y"]),
        "convrot_linear_fwd": (["x", 64, 256, "qw", "sw", 256, "bias", "y", "ws", WS1, None],
                               ["x", "qw", "sw", "bias", "y"]),
        "convrot_linear_fwd_noalloc": (["x", 64, 256, "qw", "sw", 256, "bias", "y", None],
                                       ["x", "qw", "sw", "bias", "y"]),
        "convrot_linear_fwd_lora": (["x", 64, 256, "qw", "sw", 256, "bias", "a", "b", 16, 1.0, "y",
                                     "ws", WS1, None], ["x", "qw", "sw", "bias", "a", "b", "y"]),
        "convrot_lora_down": (["x", 64, 256, "a", 16, "xa", None], ["x", "a", "xa"]),
        "convrot_gemm_i8_i32": (["a", "b", 64, 256, 256, 0, "acc", None], ["a", "b", "acc"]),
        "convrot_dequant_weight_t": (["qw", "sw", 256, 256, "wt", None], ["qw", "sw", "wt"]),
        "convrot_linear_bwd_dx": (["dy", 64, 256, "qw", "sw", 256, 1, "dx", "ws", WS1, None],
                                  ["dy", "qw", "sw", "dx"]),
        "convrot_embedding_lookup": (["ids", 64, "qe", "se", 1000, 256, "out", "oob", None],
                                     ["ids", "qe", "se", "out"]),
    }
    base = {}
    for i, name in enumerate(sorted({a for args, _ in calls.values() for a in args
                                     if isinstance(a, str)})):
        base[name] = C.c_void_p((i + 1) << 24)
    assert set(calls) | {"convrot_workspace_bytes", "convrot_status_string"} == set(cr.EXPORTS)
    for fn, (args, ptrs) in calls.items():
        f = getattr(L, fn)
        for moved in ptrs:
            real = [(_odd(base[a]) if a == moved else base[a]) if isinstance(a, str) else a
                    for a in args]
            assert f(*real) == -1, (fn, moved)
    # the workspace must be 256-byte aligned, the lookup's counter 4-byte aligned
    for fn in ("convrot_linear_fwd", "convrot_linear_fwd_lora", "convrot_linear_bwd_dx"):
        args, _ = calls[fn]
        real = [(_odd(base[a], 128) if a == "ws" else base[a]) if isinstance(a, str) else a
                for a in args]
        assert getattr(L, fn)(*real) == -1, fn
    args, _ = calls["convrot_embedding_lookup"]
    real = [(_odd(base[a], 2) if a == "oob" else base[a]) if isinstance(a, str) else a
            for a in args]
    assert L.convrot_embedding_lookup(*real) == -1


def test_size_limits(cr):
    """Row, column and id counts above 2^31 - 1, or tensors above 2^40 elements,
    are CONVROT_ESHAPE before any size arithmetic could overflow; the workspace
    query returns 0 for them."""
    L = cr.lib()
    big = (1 << 31)
    assert L.convrot_quantize_act(A, big, 128, B, Y, None) == -2
    assert L.convrot_quantize_act(A, (1 << 40) // 4096 + 1, 4096, B, Y, None) == -2
    assert L.convrot_linear_fwd(A, 64, 4096, B, B, big, None, Y, WS, 1 << 20, None) == -2
    assert L.convrot_gemm_i8_i32(A, B, 1 << 30, 1 << 30, 128, 0, Y, None) == -2
    assert L.convrot_embedding_lookup(A, big, B, B, 10, 128, Y, None, None) == -2
    assert L.convrot_linear_bwd_dx(A, 1 << 30, 1 << 20, B, B, 128, 0, Y, WS, 1 << 20, None) == -2
    assert cr.workspace_bytes(cr.OP_LINEAR_FWD, big, 128, 128) == 0
    assert cr.workspace_bytes(cr.OP_LINEAR_BWD_DX, 1 << 30, 1 << 30, 128, cr.BWD_BF16) == 0


def test_activations_must_be_bf16(cr, monkeypatch):
    """Activations and gradients keep their own dtype (bf16): the binding refuses
    any other dtype before reaching the C ABI, so nothing is enqueued.  This is the
    bug sd-scripts pull request 2461 lists first among the fixes of existing bugs:
    activations cast to the int8 weight's dtype."""
    import torch
    calls = []

    class Spy:
        def __getattr__(self, name):
            calls.append(name)
            raise AssertionError(f"reached the C ABI: {name}")

    monkeypatch.setattr(cr, "_lib", Spy())
    qw = torch.zeros((256, 256), dtype=torch.int8)
    sw = torch.ones(256, dtype=torch.float32)
    la = torch.zeros((16, 256), dtype=torch.bfloat16)
    lb = torch.zeros((256, 16), dtype=torch.bfloat16)
    for dt in (torch.int8, torch.float16, torch.float32, torch.uint8):
        x = torch.zeros((64, 256), dtype=dt)
        for fn in (lambda: cr.linear_fwd(x, qw, sw), lambda: cr.quantize_act(x),
                   lambda: cr.quantize_weight(x), lambda: cr.bwd_quant_dy(x, sw),
                   lambda: cr.linear_bwd_dx(x, qw, sw, cr.BWD_INT8),
                   lambda: cr.linear_bwd_dx(x, qw, sw, cr.BWD_BF16),
                   lambda: cr.linear_fwd_lora(x, qw, sw, la, lb, 1.0),
                   lambda: cr.lora_down(x, la)):
            with pytest.raises(TypeError):
                fn()
    assert calls == []


def test_noalloc_forward_host_checks(cr):
    """The allocation-free forward checks its arguments like the forward and
    refuses, on the host and before any HIP call, a call whose q_x, s_x and
    partials would not fit its static scratch."""
    L = cr.lib()
    f = L.convrot_linear_fwd_noalloc
    assert f(None, 4, 128, B, B, 4, None, Y, None) == -1
    assert f(A, 4, 100, B, B, 4, None, Y, None) == -2
    assert f(None, 0, 4096, None, None, 4096, None, None, None) == 0
    limit = cr.NOALLOC_SCRATCH_BYTES
    # 32768 x 4096 activations need 128 MiB of codes: over the 96 MiB scratch
    assert cr.workspace_bytes(cr.OP_LINEAR_FWD, 32768, 128, 4096) > limit
    assert f(A, 32768, 4096, B, B, 128, None, Y, None) == -6
    # 20480 x 4096 (the packed stream) still fits
    assert cr.workspace_bytes(cr.OP_LINEAR_FWD, 20480, 4096, 4096) <= limit
    m = re.search(r"#define CONVROT_NOALLOC_SCRATCH_BYTES \(\(size_t\)(\d+) << (\d+)\)",
                  open(HEADER).read())
    assert m and int(m.group(1)) << int(m.group(2)) == limit


def test_modules_refuse_before_the_c_abi(cr, monkeypatch):
    """The PyTorch modules check dtypes and shapes before any call reaches the
    library: a non-bf16 activation (the bug sd-scripts pull request 2461 fixed)
    and non-integer ids raise with nothing enqueued."""
    import torch
    from w8a8_rotated_int8_amd.nn import ConvRotEmbedding, ConvRotLinear

    class Spy:
        def __getattr__(self, name):
            raise AssertionError(f"reached the C ABI: {name}")

    monkeypatch.setattr(cr, "_lib", Spy())
    qw = torch.zeros((256, 384), dtype=torch.int8)
    sw = torch.ones(256, dtype=torch.float32)
    mod = ConvRotLinear(qw, sw, bwd_mode="int8")
    assert (mod.in_features, mod.out_features) == (384, 256)
    for dt in (torch.float16, torch.float32, torch.int8):
        with pytest.raises(TypeError):
            mod(torch.zeros((4, 384), dtype=dt))
    with pytest.raises(ValueError):
        mod(torch.zeros((4, 256), dtype=torch.bfloat16))  # wrong feature count
    with pytest.raises(ValueError):
        ConvRotLinear(qw, sw, bwd_mode="fp8")
    with pytest.raises(ValueError):
        ConvRotLinear(torch.zeros((256, 200), dtype=torch.int8), sw)  # K not a multiple of 128
    with pytest.raises(ValueError):
        ConvRotLinear(qw, sw, bias=torch.zeros(256, dtype=torch.float32))
    emb = ConvRotEmbedding(torch.zeros((10, 128), dtype=torch.int8), torch.ones(10))
    with pytest.raises(TypeError):
        emb(torch.zeros(3, dtype=torch.float32))
