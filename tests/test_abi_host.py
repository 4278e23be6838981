"""Host-only checks of the C-ABI library: it loads, exports every declared
symbol, carries the same NF4 table as the oracle, does the pages' storage
arithmetic, and rejects bad arguments on the host before any HIP call.

Storage figures ("Double quantization" and "Paged optimizers, and QLoRA end to
end", zerotofrontier.app PEFT page): 32/64 = 0.5 bits of constants per
parameter without double quantization; 8/64 + 32/(64*256) ~ 0.127 with it, a
saving of 0.373 bits (~3 GB at 65B); 4.127 bits ~ 0.516 bytes per weight;
65e9 * 4.127 / 8 ~ 33.5 GB for a 65B base.
"""
import ctypes
import os
import re

import numpy as np
import pytest
import torch

import bit_nf4_quantized_09_amd as nf4

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "qlora_nf4.h")


def _declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(nf4_\w+|qlora_\w+)\s*\(", text)))


def test_library_exports_every_declared_symbol():
    L = nf4.load_library()
    names = _declared_functions()
    assert names == sorted(["nf4_quantize", "nf4_double_quantize", "nf4_double_dequantize",
                            "nf4_dequantize", "qlora_linear_fwd", "qlora_linear_bwd",
                            "nf4_workspace_bytes", "nf4_storage_bytes", "nf4_codebook",
                            "nf4_last_error", "nf4_profile_next_fused", "nf4_adamw_step",
                            "nf4_adamw_step_paged", "nf4_quantize_codebook", "nf4_codebook_stats",
                            "qlora_linear_fwd_noalloc", "nf4_lowrank_svd", "nf4_loftq_init",
                            "nf4_double_quantize_batch", "nf4_double_quantize_batch_workspace_bytes"])
    for name in names:
        assert hasattr(L, name), name
    # and the C symbols are unmangled (extern "C")
    nm = os.popen("nm -D --defined-only %s" % nf4.lib_path()).read()
    for name in names:
        assert re.search(r"\bT %s\b" % name, nm), name


def test_codebook_matches_oracle(orc):
    lib_tab = np.array(nf4.nf4_codebook(), np.float32)
    assert np.array_equal(lib_tab.view(np.uint32), orc.nf4_codebook().view(np.uint32))


def test_storage_accounting_closed_forms():
    n = 64 * 256 * 1000
    codes, q, c2 = nf4.nf4_storage_bytes(n)
    assert codes == n // 2 and q == n // 64 and c2 == 4 * (n // 64 // 256)
    const_bits = 8.0 * (q + c2) / n
    assert abs(const_bits - (8 / 64 + 32 / (64 * 256))) < 1e-12
    assert round(const_bits, 3) == 0.127
    assert round(32 / 64 - const_bits, 3) == 0.373          # saving vs fp32 constants
    total_bits = 8.0 * (codes + q + c2) / n
    assert round(total_bits, 3) == 4.127
    assert round(total_bits / 8, 3) == 0.516
    n65 = 65 * 10 ** 9
    c, qq, cc = nf4.nf4_storage_bytes(n65)
    assert abs((c + qq + cc) / 1e9 - 33.5) < 0.1
    assert abs(n65 * (32 / 64 - const_bits) / 8 / 1e9 - 3.0) < 0.1   # "about 3 GB"
    # partial blocks round up
    assert nf4.nf4_storage_bytes(1) == (1, 1, 4)
    assert nf4.nf4_storage_bytes(65) == (33, 2, 4)
    assert nf4.nf4_storage_bytes(0) == (0, 0, 0)


def test_workspace_sizes():
    # double quantization keeps one float64 sum per 2048-constant chunk of the mean's tree
    assert nf4.nf4_workspace_bytes(nf4.NF4_OP_DOUBLE_QUANTIZE, 0, 0, 0, 0) == 0
    assert nf4.nf4_workspace_bytes(nf4.NF4_OP_DOUBLE_QUANTIZE, 0, 2048, 0, 0) == 8
    assert nf4.nf4_workspace_bytes(nf4.NF4_OP_DOUBLE_QUANTIZE, 0, 2049, 0, 0) == 2 * 8
    fwd = nf4.nf4_workspace_bytes(nf4.NF4_OP_LINEAR_FWD, 4096, 8192, 8192, 64)
    bwd = nf4.nf4_workspace_bytes(nf4.NF4_OP_LINEAR_BWD, 4096, 8192, 8192, 64)
    assert fwd >= 2 * 4096 * 64 * 2 and bwd >= 2 * 4096 * 64 * 2
    assert nf4.nf4_workspace_bytes(99, 1, 1, 1, 1) == 0
    # empty token batch: the backward still writes dA = dB = 0 through the slice buffer
    assert nf4.nf4_workspace_bytes(nf4.NF4_OP_LINEAR_FWD, 0, 256, 256, 8) >= 0
    assert nf4.nf4_workspace_bytes(nf4.NF4_OP_LINEAR_BWD, 0, 256, 256, 8) >= 256 * 8 * 4
    for M in (1, 16, 17, 300, 4096):
        for N, K in ((256, 256), (8192, 22016), (22016, 8192)):
            assert nf4.nf4_workspace_bytes(nf4.NF4_OP_LINEAR_BWD, M, N, K, 64) >= 2 * M * 64 * 2


# --- argument validation: every case below fails before any HIP call -------------

def test_quantize_rejects_bad_arguments():
    L = nf4.load_library()
    p = ctypes.c_void_p(4096)
    assert L.nf4_quantize(p, 0, 128, 32, p, p, None) == nf4.NF4_ERR_UNSUPPORTED
    assert b"blocksize" in L.nf4_last_error()
    assert L.nf4_quantize(p, 7, 128, 64, p, p, None) == nf4.NF4_ERR_ARG
    assert L.nf4_quantize(p, 0, -1, 64, p, p, None) == nf4.NF4_ERR_ARG
    assert L.nf4_quantize(None, 0, 128, 64, p, p, None) == nf4.NF4_ERR_ARG
    assert L.nf4_quantize(ctypes.c_void_p(4100), 0, 128, 64, p, p, None) == nf4.NF4_ERR_ARG
    assert b"aligned" in L.nf4_last_error()
    assert L.nf4_quantize(None, 0, 0, 64, None, None, None) == nf4.NF4_OK   # empty: nothing to do


def test_double_quantize_rejects_bad_arguments():
    L = nf4.load_library()
    p = ctypes.c_void_p(4096)
    assert L.nf4_double_quantize(p, 100, 128, p, p, p, None, 0, None) == nf4.NF4_ERR_UNSUPPORTED
    assert L.nf4_double_quantize(p, 100, 256, p, p, None, None, 0, None) == nf4.NF4_ERR_ARG
    # n1 > 0 needs a workspace (one float64 per 2048 constants)
    assert L.nf4_double_quantize(p, 100, 256, p, p, p, None, 0, None) == nf4.NF4_ERR_WORKSPACE
    assert L.nf4_double_quantize(p, 5000, 256, p, p, p, None, 0, None) == nf4.NF4_ERR_WORKSPACE
    assert L.nf4_double_quantize(p, 5000, 256, p, p, p, p, 8, None) == nf4.NF4_ERR_WORKSPACE
    assert L.nf4_double_dequantize(p, p, p, 10, 64, p, None) == nf4.NF4_ERR_UNSUPPORTED
    assert L.nf4_double_dequantize(None, p, p, 10, 256, p, None) == nf4.NF4_ERR_ARG


def _w(rows, cols, codes=4096):
    return nf4._Weight(codes, 4096, 4096, 4096, rows, cols)


def test_linear_rejects_bad_arguments():
    L = nf4.load_library()
    p = ctypes.c_void_p(4096)
    ws = ctypes.c_void_p(8192)
    fwd = L.qlora_linear_fwd
    good = _w(256, 256)
    assert fwd(None, p, 16, p, p, 8, 16.0, p, p, ws, 1 << 20, None) == nf4.NF4_ERR_ARG
    assert fwd(ctypes.byref(_w(256, 250)), p, 16, p, p, 8, 16.0, p, p, ws, 1 << 20, None) == nf4.NF4_ERR_UNSUPPORTED
    assert b"multiple of 64" in L.nf4_last_error()
    assert fwd(ctypes.byref(_w(250, 256)), p, 16, p, p, 8, 16.0, p, p, ws, 1 << 20, None) == nf4.NF4_ERR_UNSUPPORTED
    assert fwd(ctypes.byref(good), p, 16, p, p, 0, 16.0, p, p, ws, 1 << 20, None) == nf4.NF4_ERR_UNSUPPORTED
    assert fwd(ctypes.byref(good), p, 16, p, p, 12, 16.0, p, p, ws, 1 << 20, None) == nf4.NF4_ERR_UNSUPPORTED
    assert fwd(ctypes.byref(good), p, 16, p, p, 136, 16.0, p, p, ws, 1 << 20, None) == nf4.NF4_ERR_UNSUPPORTED
    assert fwd(ctypes.byref(good), p, 16, None, p, 8, 16.0, p, p, ws, 1 << 20, None) == nf4.NF4_ERR_ARG
    assert fwd(ctypes.byref(good), p, 16, p, p, 8, float("nan"), p, p, ws, 1 << 20, None) == nf4.NF4_ERR_ARG
    assert fwd(ctypes.byref(good), p, -1, p, p, 8, 16.0, p, p, ws, 1 << 20, None) == nf4.NF4_ERR_ARG
    assert fwd(ctypes.byref(good), p, 16, p, p, 8, 16.0, None, p, ws, 1 << 20, None) == nf4.NF4_ERR_ARG
    assert fwd(ctypes.byref(good), ctypes.c_void_p(4098), 16, p, p, 8, 16.0, p, p, ws, 1 << 20, None) == nf4.NF4_ERR_ARG
    assert fwd(ctypes.byref(good), p, 16, p, p, 8, 16.0, p, None, None, 0, None) == nf4.NF4_ERR_WORKSPACE
    assert fwd(ctypes.byref(good), p, 16, p, p, 8, 16.0, p, p, ctypes.c_void_p(8200), 1 << 20, None) == nf4.NF4_ERR_ARG
    assert fwd(ctypes.byref(_w(256, 256, codes=4104)), p, 16, p, p, 8, 16.0, p, p, ws, 1 << 20, None) == nf4.NF4_ERR_ARG
    assert fwd(ctypes.byref(good), p, 0, p, p, 8, 16.0, p, p, ws, 1 << 20, None) == nf4.NF4_OK  # M = 0
    # size limits (32-bit operand offsets, launch grid), before any device call
    assert fwd(ctypes.byref(_w(1 << 22, 64)), p, 16, p, p, 8, 16.0, p, p, ws, 1 << 20, None) == nf4.NF4_ERR_UNSUPPORTED
    assert b"below 2^22" in L.nf4_last_error()
    assert fwd(ctypes.byref(_w(64, 1 << 22)), p, 16, p, p, 8, 16.0, p, p, ws, 1 << 20, None) == nf4.NF4_ERR_UNSUPPORTED
    # the largest accepted N and K pass the shape checks, for every token count (they fail
    # later, on the workspace size, which this call gives as 16 bytes)
    for M in (1, 16, 17, 4096):
        assert fwd(ctypes.byref(_w(8, (1 << 22) - 64)), p, M, p, p, 8, 16.0, p, p, ws, 16, None) == nf4.NF4_ERR_WORKSPACE
        assert L.qlora_linear_bwd(ctypes.byref(_w((1 << 22) - 8, 64)), p, p, M, p, p, 8, 16.0, p, p, p, p, ws, 16,
                                  None) == nf4.NF4_ERR_WORKSPACE
    assert fwd(ctypes.byref(good), p, 1 << 23, p, p, 8, 16.0, p, p, ws, 1 << 20, None) == nf4.NF4_ERR_UNSUPPORTED
    wide = _w(1025 * 128, 64)       # (2^14 - 1) token tiles x 1025 feature tiles >= 2^24
    assert fwd(ctypes.byref(wide), p, (1 << 23) - 512, p, p, 8, 16.0, p, p, ws, 1 << 20, None) == nf4.NF4_ERR_UNSUPPORTED
    assert b"2^24 workgroups" in L.nf4_last_error()
    tall = _w(64, 1025 * 128)
    assert L.qlora_linear_bwd(ctypes.byref(tall), p, p, (1 << 23) - 512, p, p, 8, 16.0, p, p, p, p, ws,
                              1 << 20, None) == nf4.NF4_ERR_UNSUPPORTED
    bwd = L.qlora_linear_bwd
    assert bwd(ctypes.byref(good), p, p, 16, p, p, 8, 16.0, p, p, None, p, ws, 1 << 20, None) == nf4.NF4_ERR_ARG
    assert bwd(ctypes.byref(good), p, p, 16, p, p, 8, 16.0, None, p, p, p, ws, 16, None) == nf4.NF4_ERR_WORKSPACE
    assert bwd(ctypes.byref(good), None, p, 16, p, p, 8, 16.0, p, p, p, p, ws, 1 << 20, None) == nf4.NF4_ERR_ARG


def test_noalloc_forward_rejects_before_any_device_call():
    # the allocation-free forward checks the shape's workspace against its fixed 32 MiB
    # scratch on the host, before it looks up the scratch on a device
    L = nf4.load_library()
    p = ctypes.c_void_p(4096)
    f = L.qlora_linear_fwd_noalloc
    assert L.nf4_workspace_bytes(nf4.NF4_OP_LINEAR_FWD, 4096, 22016, 8192, 64) > (32 << 20)
    assert f(ctypes.byref(_w(22016, 8192)), p, 4096, p, p, 64, 16.0, p, p, None) == nf4.NF4_ERR_WORKSPACE
    assert b"33554432-byte scratch" in L.nf4_last_error()
    assert f(None, p, 16, p, p, 8, 16.0, p, p, None) == nf4.NF4_ERR_ARG
    assert f(ctypes.byref(_w(256, 250)), p, 16, p, p, 8, 16.0, p, p, None) == nf4.NF4_ERR_UNSUPPORTED
    assert f(ctypes.byref(_w(256, 256)), p, -1, p, p, 8, 16.0, p, p, None) == nf4.NF4_ERR_ARG


def test_dequantize_rejects_bad_arguments():
    L = nf4.load_library()
    p = ctypes.c_void_p(4096)
    assert L.nf4_dequantize(None, p, 0, None) == nf4.NF4_ERR_ARG
    assert L.nf4_dequantize(ctypes.byref(_w(4, 4)), p, 9, None) == nf4.NF4_ERR_ARG
    assert L.nf4_dequantize(ctypes.byref(_w(4, 4)), None, 0, None) == nf4.NF4_ERR_ARG
    assert L.nf4_dequantize(ctypes.byref(_w(-1, 4)), p, 0, None) == nf4.NF4_ERR_ARG
    assert L.nf4_dequantize(ctypes.byref(_w(1 << 40, 1 << 40)), p, 0, None) == nf4.NF4_ERR_ARG   # n overflows
    assert L.nf4_dequantize(ctypes.byref(_w(0, 4)), p, 0, None) == nf4.NF4_OK


def test_binding_fails_loudly_without_gpu_tensors():
    import torch
    with pytest.raises(ValueError):
        nf4.nf4_quantize(torch.zeros(64))


def test_adamw_rejects_bad_arguments():
    # checks happen on the host, before any HIP call
    L = nf4.load_library()
    p = ctypes.c_void_p(1 << 20)
    q = ctypes.c_void_p(2 << 20)
    m = ctypes.c_void_p(3 << 20)
    v = ctypes.c_void_p(4 << 20)
    step = L.nf4_adamw_step
    assert step(p, q, m, v, None, 0, 1e-4, 0.9, 0.999, 1e-8, 0.0, 1, None) == nf4.NF4_OK     # n == 0
    assert step(p, q, m, v, None, 64, 1e-4, 0.9, 0.999, 1e-8, 0.0, 0, None) == nf4.NF4_ERR_ARG  # step 0
    assert step(p, q, m, v, None, 64, 1e-4, 1.0, 0.999, 1e-8, 0.0, 1, None) == nf4.NF4_ERR_ARG  # beta1 = 1
    assert step(p, q, m, v, None, 64, 1e-4, 0.9, -0.1, 1e-8, 0.0, 1, None) == nf4.NF4_ERR_ARG  # beta2 < 0
    assert step(p, q, m, v, None, 64, 1e-4, 0.9, 0.999, 0.0, 0.0, 1, None) == nf4.NF4_ERR_ARG  # eps = 0
    assert step(p, q, m, v, None, 64, float("nan"), 0.9, 0.999, 1e-8, 0.0, 1, None) == nf4.NF4_ERR_ARG
    assert step(p, q, m, v, None, -1, 1e-4, 0.9, 0.999, 1e-8, 0.0, 1, None) == nf4.NF4_ERR_ARG
    assert step(None, q, m, v, None, 64, 1e-4, 0.9, 0.999, 1e-8, 0.0, 1, None) == nf4.NF4_ERR_ARG
    assert step(ctypes.c_void_p((1 << 20) + 4), q, m, v, None, 64, 1e-4, 0.9, 0.999, 1e-8, 0.0, 1,
                None) == nf4.NF4_ERR_ARG                                                      # misaligned
    assert step(p, q, m, v, ctypes.c_void_p((5 << 20) + 2), 64, 1e-4, 0.9, 0.999, 1e-8, 0.0, 1,
                None) == nf4.NF4_ERR_ARG                                                      # bf16 copy
    assert step(p, ctypes.c_void_p((1 << 20) + 128), m, v, None, 64, 1e-4, 0.9, 0.999, 1e-8, 0.0, 1,
                None) == nf4.NF4_ERR_ARG                                                      # overlap
    assert "overlap" in L.nf4_last_error().decode()
    paged = L.nf4_adamw_step_paged
    st = ctypes.c_void_p(8 << 20)
    assert paged(p, q, m, v, None, 64, 1e-4, 0.9, 0.999, 1e-8, 0.0, 1, st, 1024, None) == nf4.NF4_ERR_WORKSPACE
    assert paged(p, q, m, v, None, 64, 1e-4, 0.9, 0.999, 1e-8, 0.0, 1, None, 1 << 20, None) == nf4.NF4_ERR_ARG
    assert paged(p, q, m, v, None, 64, 1e-4, 0.9, 0.999, 1e-8, 0.0, 1, ctypes.c_void_p((8 << 20) + 16),
                 1 << 20, None) == nf4.NF4_ERR_ARG                                            # stage alignment


def test_codebook_entry_points_reject_bad_arguments():
    L = nf4.load_library()
    p = ctypes.c_void_p(1 << 20)
    lv = lambda xs: (ctypes.c_float * 16)(*xs)
    good = lv([k / 8 for k in range(-8, 8)])
    q = L.nf4_quantize_codebook
    assert q(p, 0, 0, 64, good, p, p, None) == nf4.NF4_OK                         # n == 0
    assert q(p, 0, 64, 32, good, p, p, None) == nf4.NF4_ERR_UNSUPPORTED           # blocksize
    assert q(p, 0, 64, 64, None, p, p, None) == nf4.NF4_ERR_ARG
    desc = lv([k / 8 for k in range(7, -9, -1)])
    assert q(p, 0, 64, 64, desc, p, p, None) == nf4.NF4_ERR_UNSUPPORTED            # not ascending
    # two midpoints inside one 1/32 bucket: levels 0, 0.01, 0.02 around the middle
    crowded = [k / 8 for k in range(-8, 0)] + [0.0, 0.01, 0.02] + [k / 8 for k in range(1, 6)]
    assert q(p, 0, 64, 64, lv(crowded), p, p, None) == nf4.NF4_ERR_UNSUPPORTED
    assert "bucket" in L.nf4_last_error().decode()
    # a symmetric table without a zero level puts a midpoint exactly at 0
    sym = [(k + 0.5) / 8 for k in range(-8, 8)]
    assert q(p, 0, 64, 64, lv(sym), p, p, None) == nf4.NF4_ERR_UNSUPPORTED
    assert "subnormal" in L.nf4_last_error().decode()
    st = L.nf4_codebook_stats
    assert nf4.nf4_workspace_bytes(nf4.NF4_OP_CODEBOOK_STATS, 0, 0, 0, 0) == 0
    wsb = nf4.nf4_workspace_bytes(nf4.NF4_OP_CODEBOOK_STATS, 0, 1 << 20, 0, 0)
    assert wsb > 0
    assert st(p, 0, 1 << 20, p, p, good, p, p, wsb - 8, None) == nf4.NF4_ERR_WORKSPACE
    assert st(p, 0, 1 << 20, p, p, None, p, p, wsb, None) == nf4.NF4_ERR_ARG
    assert st(p, 0, 1 << 20, p, p, good, None, p, wsb, None) == nf4.NF4_ERR_ARG


def test_binding_checks_tuple_sizes_before_the_device():
    # sizes and dtypes of the weight tuple are checked against its shape first, so a
    # mismatched tuple never reaches a kernel (CPU tensors: the size checks come first)
    u8, f32 = torch.uint8, torch.float32
    n = 4 * 64
    codes, q, c2, mean = torch.zeros(n // 2, dtype=u8), torch.zeros(4, dtype=u8), torch.zeros(1), torch.zeros(1)
    with pytest.raises(ValueError, match="codes must hold 128"):
        nf4.NF4Weight(codes[:100], q, c2, mean, (4, 64)).validate()
    with pytest.raises(ValueError, match="q must hold 4"):
        nf4.NF4Weight(codes, q[:3], c2, mean, (4, 64)).validate()
    with pytest.raises(ValueError, match="c2 must hold 1"):
        nf4.NF4Weight(codes, q, torch.zeros(2), mean, (4, 64)).validate()
    with pytest.raises(ValueError, match="mean must hold 1"):
        nf4.NF4Weight(codes, q, c2, mean.double(), (4, 64)).validate()
    with pytest.raises(ValueError, match="absmax must hold 4"):
        nf4.NF4Weight(codes, None, None, None, (4, 64), torch.zeros(5, dtype=f32)).validate()
    with pytest.raises(ValueError, match="absmax is missing"):
        nf4.NF4Weight(codes, None, None, None, (4, 64)).validate()
    with pytest.raises(ValueError, match="GPU tensor"):       # consistent, but on the host
        nf4.NF4Weight(codes, q, c2, mean, (4, 64)).validate()
    w = torch.zeros(n)
    with pytest.raises(ValueError, match="absmax must hold 4"):
        nf4.nf4_codebook_stats(w, codes, torch.zeros(3), nf4.nf4_codebook())
    with pytest.raises(ValueError, match="c2 must hold 1"):
        nf4.nf4_double_dequantize(q, torch.zeros(0), mean)


def test_lowrank_and_loftq_reject_bad_arguments():
    L = nf4.load_library()
    p = ctypes.c_void_p(4096)
    ws = ctypes.c_void_p(8192)
    svd = L.nf4_lowrank_svd
    big = 1 << 30
    assert svd(None, 256, 192, 8, 24, 2, p, p, p, p, ws, big, None) == nf4.NF4_ERR_ARG
    assert svd(p, 256, 192, 8, 4, 2, p, p, p, p, ws, big, None) == nf4.NF4_ERR_ARG          # l < r
    assert svd(p, 256, 192, 8, 97, 2, p, p, p, p, ws, big, None) == nf4.NF4_ERR_UNSUPPORTED  # l > 96
    assert svd(p, 16, 192, 8, 24, 2, p, p, p, p, ws, big, None) == nf4.NF4_ERR_ARG          # l > N
    assert svd(p, 256, 192, 8, 24, 17, p, p, p, p, ws, big, None) == nf4.NF4_ERR_ARG        # power_iters
    assert svd(p, 256, 192, 8, 24, 2, p, p, p, p, ws, 16, None) == nf4.NF4_ERR_WORKSPACE
    assert svd(p, 1 << 22, 192, 8, 24, 2, p, p, p, p, ws, big, None) == nf4.NF4_ERR_UNSUPPORTED
    lq = L.nf4_loftq_init
    assert lq(p, 256, 192, 8, 16.0, 3, 24, 2, p, p, p, p, p, p, p, p, ws, 16, None) == nf4.NF4_ERR_WORKSPACE
    assert lq(p, 256, 192, 8, 0.0, 3, 24, 2, p, p, p, p, p, p, p, p, ws, big, None) == nf4.NF4_ERR_ARG
    assert lq(p, 256, 192, 8, 16.0, 0, 24, 2, p, p, p, p, p, p, p, p, ws, big, None) == nf4.NF4_ERR_ARG
    assert lq(p, 256, 192, 8, 16.0, 3, 24, 2, p, p, p, p, p, None, p, p, ws, big, None) == nf4.NF4_ERR_ARG
    assert L.nf4_workspace_bytes(nf4.NF4_OP_LOFTQ, 24, 256, 192, 8) > 256 * 192 * 4
    assert L.nf4_workspace_bytes(nf4.NF4_OP_LOWRANK_SVD, 97, 256, 192, 8) == 0


def test_double_quantize_batch_host_checks():
    # sizes and argument checks of the batched double quantization, before any HIP call
    import ctypes
    L = nf4.load_library()
    n1 = (ctypes.c_int64 * 4)(1, 2048, 2049, 2048 * 2048)
    # one float64 chunk sum per 2048 constants of every tensor
    assert L.nf4_double_quantize_batch_workspace_bytes(4, n1) == 8 * (1 + 1 + 2 + 2048)
    assert L.nf4_double_quantize_batch_workspace_bytes(0, n1) == 0
    null = (ctypes.c_void_p * 1)(None)
    one = (ctypes.c_int64 * 1)(64)
    assert L.nf4_double_quantize_batch(0, None, None, None, None, None, None, 0, None) == 0
    assert L.nf4_double_quantize_batch(-1, null, one, null, null, null, None, 0, None) == nf4.NF4_ERR_ARG
    big = (ctypes.c_int64 * 1)(2048 * 2048 + 1)
    assert L.nf4_double_quantize_batch(1, null, big, null, null, null, None, 0, None) == nf4.NF4_ERR_UNSUPPORTED
    # NULL mean
    assert L.nf4_double_quantize_batch(1, null, one, null, null, null, None, 0, None) == nf4.NF4_ERR_ARG
    # a non-null but too small workspace is refused before anything runs
    fake = (ctypes.c_void_p * 1)(0x1000)
    assert L.nf4_double_quantize_batch(1, fake, one, fake, fake, fake, ctypes.c_void_p(0x1000), 4,
                                       None) == nf4.NF4_ERR_WORKSPACE
