"""The C ABI without a GPU: the library loads, exports every symbol the
header declares, computes its size helpers, and rejects invalid calls before
any HIP call (so nothing is enqueued and no device is needed)."""
import ctypes
import os
import re

import pytest

from block_scaled_precision_token_amd import ops

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "bsp.h")

if not os.path.exists(ops.LIB_PATH):
    pytest.skip("libbsp.so not built", allow_module_level=True)

L = ops.lib()
A = ctypes.c_void_p(1 << 20)        # a 16-byte aligned, never dereferenced address
MIS = ctypes.c_void_p((1 << 20) + 4)  # misaligned


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(bsp_[a-z0-9_]+)\s*\(", text)))


def test_every_declared_symbol_is_exported():
    names = declared_functions()
    assert len(names) >= 13
    for n in names:
        assert hasattr(L, n), n
    assert set(names) == set(ops.EXPORTED)


def test_version_and_status_strings():
    assert L.bsp_version() == 100
    for s in range(8):
        assert len(L.bsp_status_string(s)) > 0
    assert L.bsp_status_string(99) == b"unknown status"


def test_size_helpers():
    c, s, o = ctypes.c_size_t(), ctypes.c_size_t(), ctypes.c_size_t()
    assert L.bsp_nvfp4_sizes(8192, 2048, 1, ctypes.byref(c), ctypes.byref(s), ctypes.byref(o)) == 0
    assert (c.value, s.value, o.value) == (8192 * 1024, 8192 * 128, 8192)
    assert L.bsp_nvfp4_sizes(8192, 2040, 1, ctypes.byref(c), ctypes.byref(s), ctypes.byref(o)) == 2
    assert L.bsp_mxfp8_sizes(4096, 7168, ctypes.byref(c), ctypes.byref(s)) == 0
    assert (c.value, s.value) == (4096 * 7168, 4096 * 224)
    assert L.bsp_mxfp8_grouped_cols(100, 4) == 256          # roundup256(100 + 31*4)
    assert L.bsp_mxfp8_grouped_cols(36864, 257) == 45056    # rows of the copy start on 128-byte lines
    # tile list + counters (256-byte aligned), then block-major scale planes:
    # blocks padded to whole K stages plus one stage (128 K values, 8 NVFP4
    # blocks, in the forward form; 64 in the weight-gradient form), rows
    # padded to 256
    def up(x, a):
        return (x + a - 1) // a * a
    head = up((512 + 128 + 16) * 8, 256)
    nbp = up(2048 // 16, 8) + 8
    a_plane = nbp * ((65536 + 255) // 256 + 128) * 256
    b_plane = 128 * nbp * up(1536, 256)
    assert L.bsp_gemm_workspace_size(0, 0, 65536, 1536, 2048, 128) == head + up(a_plane, 256) + up(b_plane, 256)
    nbp = up(7168 // 32, 4) + 4
    head = up(((36864 + 127) // 128 + 257 + 16) * 8, 256)
    a_plane = nbp * ((36864 + 255) // 256 + 257) * 256
    assert L.bsp_gemm_workspace_size(1, 0, 36864, 4096, 7168, 257) == head + up(a_plane, 256) + 257 * nbp * 4096
    # unknown modes size to 0
    assert L.bsp_gemm_workspace_size(0, 3, 65536, 1536, 2048, 128) == 0
    assert L.bsp_gemm_workspace_size(0, 7, 65536, 1536, 2048, 128) == 0
    head = up((258 + 16) * 8 + 257 * 4, 256)           # + the expert order
    nbp = 37120 // 32 + 2
    assert L.bsp_gemm_workspace_size(1, 2, 4096, 7168, 37120, 257) == head + nbp * 4096 + nbp * 7168
    assert L.bsp_gemm_workspace_size(7, 0, 64, 64, 64, 1) == 0
    assert L.bsp_requant_workspace_size(16384) == 8 * 4
    assert L.bsp_requant_workspace_size(16) == 4
    assert L.bsp_requant_workspace_size(1 << 30) == 1024 * 4
    assert L.bsp_requant_workspace_size(0) == 0


def test_nvfp4_rejects_bad_arguments():
    q = L.bsp_quantize_nvfp4_per_token
    assert q(None, 4, 32, 32, 1, A, A, A, 0, None) == 1
    assert q(A, 4, 30, 32, 1, A, A, A, 0, None) == 2        # K % 16
    assert q(A, 4, 32, 16, 1, A, A, A, 0, None) == 2        # ldx < K
    assert q(A, 4, 32, 32, 3, A, A, A, 0, None) == 2        # rows_per_scale does not divide M
    assert q(A, 0, 32, 32, 1, A, A, A, 0, None) == 2
    assert q(MIS, 4, 32, 32, 1, A, A, A, 0, None) == 3
    assert q(A, 4, 32, 36, 1, A, A, A, 0, None) == 3        # ldx % 8
    assert q(A, 4, 32, 32, 1, A, A, A, 0x80, None) == 1     # unknown flag


def test_mxfp8_rejects_bad_arguments():
    q = L.bsp_quantize_mxfp8
    # (x, x_rows, K, ldx, gather, M, batch, codes_row, scales_row, codes_colT, scales_colT, ld_colT, offsets, G,
    #  flags, stream)
    assert q(A, 64, 64, 64, None, 64, 1, None, None, None, None, 0, None, 0, 0, None) == 1   # nothing requested
    assert q(A, 64, 64, 64, None, 64, 1, A, None, None, None, 0, None, 0, 0, None) == 1      # codes without scales
    assert q(A, 64, 48, 64, None, 64, 1, A, A, None, None, 0, None, 0, 0, None) == 2         # K % 32
    assert q(A, 48, 64, 64, None, 48, 1, None, None, A, A, 48, None, 0, 0, None) == 2        # ungrouped M % 32
    assert q(A, 100, 64, 64, None, 100, 1, None, None, A, A, 192, A, 4, 0, None) == 2        # ld_colT < bound 224
    assert q(A, 64, 64, 64, None, 64, 1, A, A, None, None, 0, A, 2, 0, None) == 1            # groups need the column copy
    assert q(A, 64, 64, 64, None, 64, 1, A, A, None, None, 0, None, 0, 1, None) == 1         # flags
    assert q(A, 64, 64, 64, None, 32, 1, A, A, None, None, 0, None, 0, 0, None) == 2         # M != x_rows without gather
    assert q(A, 64, 64, 64, MIS, 32, 1, A, A, None, None, 0, None, 0, 0, None) == 3          # misaligned gather
    assert q(A, 64, 64, 64, None, 64, 0, A, A, None, None, 0, None, 0, 0, None) == 2         # batch < 1
    assert q(A, 64, 64, 64, A, 64, 2, A, A, None, None, 0, None, 0, 0, None) == 4            # batch with gather


def test_dequantize_and_requant_reject_bad_arguments():
    d = L.bsp_dequantize
    assert d(2, A, A, A, 4, 32, 1, A, 0, None) == 1
    assert d(0, A, A, None, 4, 32, 1, A, 0, None) == 1      # NVFP4 needs outer
    assert d(1, A, A, None, 4, 48, 1, A, 0, None) == 2
    assert d(1, A, A, None, 4, 64, 1, A, 5, None) == 1
    r = L.bsp_requant_transpose_sr
    assert r(A, A, A, 24, 32, A, A, A, 0, 2, A, 4096, None) == 2      # M % 16
    assert r(A, A, A, 32, 32, A, A, A, 0, 2, None, 0, None) == 5      # workspace
    assert r(A, A, A, 32, 32, A, A, A, 0, 4, A, 4096, None) == 1      # flags


def test_gemm_rejects_bad_arguments():
    g = L.bsp_moe_grouped_gemm_blockscaled
    ws = 1 << 16
    # NVFP4 needs both outer scales; MXFP8 takes none
    assert g(0, 0, A, A, None, None, 64, A, 2, 64, 64, 64, A, A, A, A, 0, 64, A, ws, None) == 1
    assert g(1, 0, A, A, A, None, 64, A, 2, 64, 64, 64, A, A, None, A, 0, 64, A, ws, None) == 1
    # the weight-gradient form takes no gather
    assert g(0, 2, A, A, A, A, 64, A, 2, 64, 64, 64, A, A, A, A, 0, 64, A, ws, None) == 1
    assert g(1, 0, A, A, None, None, 64, A, 2, 64, 64, 48, A, A, None, A, 0, 64, A, ws, None) == 2
    # both formats fetch operand rows in 16-byte pieces: K % 32 == 0
    assert g(0, 0, A, A, A, None, 64, A, 2, 64, 64, 48, A, A, A, A, 0, 64, A, ws, None) == 2
    # 32-bit limits: A codes of 2^32 bytes or more
    assert g(1, 0, A, A, None, A, 1 << 22, A, 2, 64, 64, 1024, A, A, None, A, 0, 64, A, ws, None) == 2
    assert g(1, 0, A, A, None, None, 64, A, 2, 64, 64, 64, A, A, None, A, 0, 32, A, ws, None) == 2   # ldc < N
    assert g(1, 0, A, A, None, None, 64, A, 2, 64, 64, 64, A, A, None, A, 0, 64, A, 8, None) == 5
    assert g(1, 0, A, A, None, None, 32, A, 2, 64, 64, 64, A, A, None, A, 0, 64, A, ws, None) == 2   # a_rows != M
    # modes 3 and 4 are unknown
    assert g(1, 3, A, A, None, None, 64, A, 2, 64, 128, 64, A, A, None, A, 1, 128, A, ws, None) == 1
    assert g(1, 4, A, A, None, None, 64, A, 2, 64, 128, 64, A, A, None, A, 1, 128, A, ws, None) == 1


def test_tiled_gemm_rejects_unknown_tile():
    g = L.bsp_moe_grouped_gemm_blockscaled_tiled
    ws = 1 << 16
    for tile in (64, 192, -1, 512):
        assert g(1, 0, A, A, None, None, 64, A, 2, 64, 64, 64, A, A, None, A, 0, 64, A, ws, tile, None) == 1
    b = L.bsp_moe_grouped_gemm_bf16_tiled
    assert b(0, A, 64, A, 64, None, 64, A, 2, 64, 64, 64, A, 0, 64, A, ws, 100, None) == 1


def test_noalloc_gemm_checks_before_any_hip_call():
    g = L.bsp_moe_grouped_gemm_blockscaled_noalloc
    # the same argument errors as the workspace form
    assert g(0, 0, A, A, None, None, 64, A, 2, 64, 64, 64, A, A, A, A, 0, 64, None) == 1
    assert g(1, 0, A, A, None, None, 64, A, 2, 64, 64, 48, A, A, None, A, 0, 64, None) == 2
    assert g(1, 0, A, A, None, None, 64, A, 2, 64, 64, 64, A, A, None, A, 0, 32, None) == 2
    assert g(1, 0, MIS, A, None, None, 64, A, 2, 64, 64, 64, A, A, None, A, 0, 64, None) == 3
    # a valid problem whose workspace exceeds the static scratch: the DeepSeek-V3
    # gate/up forward GEMM of 257 experts (about 249 MiB) is refused, nothing enqueued
    need = L.bsp_gemm_workspace_size(1, 0, 36864, 4096, 7168, 257)
    assert need > ops.GEMM_SCRATCH_BYTES
    assert g(1, 0, A, A, None, A, 4096, A, 257, 36864, 4096, 7168, A, A, None, A, 1, 4096, None) == 7
    assert L.bsp_status_string(7) != b"unknown status"
    # the Qwen3-30B-A3B-shaped expert GEMMs fit
    assert L.bsp_gemm_workspace_size(0, 0, 65536, 1536, 2048, 128) <= ops.GEMM_SCRATCH_BYTES
    assert L.bsp_gemm_workspace_size(0, 0, 65536, 2048, 768, 128) <= ops.GEMM_SCRATCH_BYTES


def test_bf16_gemm_workspace_and_bad_arguments():
    def up(x, a):
        return (x + a - 1) // a * a
    ws = L.bsp_gemm_bf16_workspace_size
    assert ws(0, 65536, 2048, 768, 128) == up(((65536 + 127) // 128 + 128 + 16) * 8, 256)
    assert ws(1, 65536, 2048, 768, 128) == ws(0, 65536, 2048, 768, 128)
    assert ws(2, 2048, 768, 65536, 128) == 512       # the weight-gradient form: the expert order
    assert ws(5, 64, 64, 64, 1) == 0 and ws(0, 0, 64, 64, 1) == 0
    g = L.bsp_moe_grouped_gemm_bf16
    W = 1 << 16
    # (mode, a, lda, b, ldb, gather, src_rows, off, G, M, N, K, c, c_dtype, ldc, ws, ws_bytes, stream)
    assert g(3, A, 64, A, 64, None, 64, A, 2, 64, 64, 64, A, 0, 64, A, W, None) == 1        # unknown mode
    assert g(0, None, 64, A, 64, None, 64, A, 2, 64, 64, 64, A, 0, 64, A, W, None) == 1     # null operand
    assert g(0, A, 64, A, 64, None, 64, A, 2, 64, 64, 60, A, 0, 64, A, W, None) == 2        # K % 8
    assert g(0, A, 64, A, 64, None, 32, A, 2, 64, 64, 64, A, 0, 64, A, W, None) == 2        # src_rows != M
    assert g(1, A, 64, A, 64, None, 64, A, 2, 64, 60, 64, A, 0, 64, A, W, None) == 2        # DGRAD N % 8
    assert g(1, A, 64, A, 32, None, 64, A, 2, 64, 64, 64, A, 0, 64, A, W, None) == 2        # DGRAD ldb < N
    assert g(2, A, 64, A, 64, None, 100, A, 2, 64, 64, 64, A, 0, 64, A, W, None) == 2       # src_rows != K
    assert g(2, A, 60, A, 64, None, 64, A, 2, 60, 64, 64, A, 0, 64, A, W, None) == 2        # WGRAD M % 8
    assert g(2, A, 64, A, 64, None, 64, A, 2, 64, 64, 64, A, 0, 64, None, 0, None) == 5     # WGRAD workspace
    assert g(0, A, 64, A, 64, None, 64, A, 2, 64, 64, 64, A, 0, 64, A, 8, None) == 5        # workspace too small
    assert g(0, A, 64, A, 64, None, 64, A, 2, 64, 64, 64, A, 0, 64, None, 0, None) == 5     # workspace missing
    assert g(0, A, 68, A, 64, None, 64, A, 2, 64, 64, 64, A, 0, 64, A, W, None) == 3        # lda % 8
    assert g(0, MIS, 64, A, 64, None, 64, A, 2, 64, 64, 64, A, 0, 64, A, W, None) == 3      # misaligned
    # 32-bit limits: A of 2^32 bytes or more
    assert g(0, A, 1024, A, 1024, A, 1 << 21, A, 2, 64, 64, 1024, A, 0, 64, A, W, None) == 2


def test_requant_batched_workspace_and_bad_arguments():
    ws = L.bsp_requant_batched_workspace_size
    assert ws(128, 2048, 2048) == 128 * 4           # one outer scale per expert: one partial each
    assert ws(1, 16384, 1) == L.bsp_requant_workspace_size(16384)
    assert ws(4, 8192, 1) == 4 * 4 * 4
    assert ws(2, 256, 512) == 2 * 4                 # one scale over two tensors
    assert ws(2, 256, 96) == 0 and ws(0, 256, 1) == 0
    r = L.bsp_requant_transpose_sr_batched
    W = 1 << 16
    # (codes, scales, outer, rps, E, M, K, codesT, scalesT, outerT, seed, flags, ws, ws_bytes, stream)
    assert r(A, A, A, 64, 2, 64, 64, A, A, A, 0, 0x4, A, W, None) == 1          # unknown flag
    assert r(A, A, None, 64, 2, 64, 64, A, A, A, 0, 0, A, W, None) == 1         # null outer
    assert r(A, A, A, 64, 2, 60, 64, A, A, A, 0, 0, A, W, None) == 2            # M % 16
    assert r(A, A, A, 48, 2, 64, 64, A, A, A, 0, 0, A, W, None) == 2            # rps neither divides nor spans M
    assert r(A, A, A, 64, 70000, 64, 64, A, A, A, 0, 0, A, W, None) == 2        # too many tensors
    assert r(A, A, A, 1, 2, 64, 64, A, A, A, 0, 0, A, 4, None) == 5             # workspace too small
    assert r(MIS, A, A, 64, 2, 64, 64, A, A, A, 0, 0, A, W, None) == 3          # misaligned


def test_requant_grouped_bad_arguments():
    r = L.bsp_requant_transpose_sr_grouped
    # (codes, scales, outer, src_rows, gather, off, G, R, K, codesT, scalesT, ldT, outerT, seed, flags, stream)
    assert r(A, A, A, 64, None, A, 2, 64, 64, A, A, 128, A, 0, 0x4, None) == 1        # unknown flag
    assert r(A, A, A, 64, None, None, 2, 64, 64, A, A, 128, A, 0, 0, None) == 1       # null offsets
    assert r(A, A, A, 64, None, A, 0, 64, 64, A, A, 128, A, 0, 0, None) == 2          # G < 1
    assert r(A, A, A, 64, None, A, 4096, 64, 64, A, A, 1 << 20, A, 0, 0, None) == 2   # G > 2048
    assert r(A, A, A, 64, None, A, 2, 64, 40, A, A, 128, A, 0, 0, None) == 2          # K % 16
    assert r(A, A, A, 50, None, A, 2, 64, 64, A, A, 128, A, 0, 0, None) == 2          # src_rows != R
    assert r(A, A, A, 64, None, A, 2, 64, 64, A, A, 96, A, 0, 0, None) == 2           # ldT < grouped cols
    assert r(A, A, A, 64, None, A, 2, 64, 64, A, A, 144, A, 0, 0, None) == 2          # ldT % 32
    assert r(A, A, A, 64, MIS, A, 2, 64, 64, A, A, 128, A, 0, 0, None) == 3           # misaligned gather


def test_nvfp4_variants_reject_bad_arguments():
    r = L.bsp_quantize_nvfp4_rht
    assert r(A, 64, 64, 64, 0x10000, A, A, A, 0, None) == 1       # signs past 16 bits
    assert r(A, 64, 64, 64, 0x1234, A, A, A, 0x2, None) == 1      # unknown flag
    assert r(A, 64, 16384, 16384, 1, A, A, A, 0, None) == 2       # rows longer than 8192
    assert r(A, 64, 72, 64, 1, A, A, A, 0, None) == 2             # ldx < K
    assert r(A, 64, 64, 68, 1, A, A, A, 0, None) == 3             # ldx % 8
    d = L.bsp_quantize_nvfp4_2d
    assert d(A, 40, 64, 64, A, A, A, None) == 2                   # M % 16
    assert d(A, 64, 40, 64, A, A, A, None) == 2                   # K % 16
    assert d(None, 64, 64, 64, A, A, A, None) == 1
    assert d(MIS, 64, 64, 64, A, A, A, None) == 3


def test_python_binding_fails_loudly_without_device_tensors():
    import torch
    with pytest.raises(ValueError):
        ops.quantize_nvfp4_per_token(torch.zeros(4, 32, dtype=torch.bfloat16))
