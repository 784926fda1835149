"""The Python binding's argument checks, without a GPU.

Every tensor argument must reach the library as a pointer to device memory of
the right dtype, contiguous and large enough; a host tensor, a wrong integer
width for the offsets or the gather, or an undersized output would otherwise
become a bad address inside a kernel.  Here CPU tensors stand in for device
tensors (ops.DEVICE_TYPE rebound to "cpu") and the library is replaced by a
stub that fails the test if it is ever reached, so every case must be rejected
with ValueError before any pointer is passed on.
"""
import pytest
import torch

from block_scaled_precision_token_amd import ops


class _NoLibrary:
    def __getattr__(self, name):
        if name.endswith("_size") or name.endswith("_cols"):
            return lambda *a: 1 << 10          # size helpers: any small value
        raise AssertionError(f"library call {name} reached with invalid arguments")


@pytest.fixture(autouse=True)
def cpu_as_device(monkeypatch):
    monkeypatch.setattr(ops, "DEVICE_TYPE", "cpu")
    monkeypatch.setattr(ops, "_lib_raw", lambda: _NoLibrary())
    monkeypatch.setattr(ops, "_stream", lambda dev: None)


def u8(*s):
    return torch.zeros(s, dtype=torch.uint8)


def f32(*s):
    return torch.zeros(s, dtype=torch.float32)


def bf(*s):
    return torch.zeros(s, dtype=torch.bfloat16)


def i64(*s):
    return torch.zeros(s, dtype=torch.int64)


def i32(*s):
    return torch.zeros(s, dtype=torch.int32)


def rejects(fn, *a, match=None, **k):
    with pytest.raises(ValueError, match=match):
        fn(*a, **k)


def test_host_tensor_is_rejected_when_device_expected(monkeypatch):
    monkeypatch.setattr(ops, "DEVICE_TYPE", "cuda")
    rejects(ops.quantize_nvfp4_per_token, bf(4, 32), match="device tensor")


def test_quantize_nvfp4_outputs():
    x = bf(4, 32)
    rejects(ops.quantize_nvfp4_per_token, x.float(), match="bfloat16")
    rejects(ops.quantize_nvfp4_per_token, x, out=(u8(4, 15), u8(4, 2), f32(4)), match="codes")
    rejects(ops.quantize_nvfp4_per_token, x, out=(u8(4, 16), u8(4, 1), f32(4)), match="scales")
    rejects(ops.quantize_nvfp4_per_token, x, out=(u8(4, 16), u8(4, 2), f32(3)), match="outer")
    rejects(ops.quantize_nvfp4_per_token, x, out=(u8(4, 16), u8(4, 2), i32(4)), match="dtype")
    rejects(ops.quantize_nvfp4_per_token, x, out=(u8(16, 4).t(), u8(4, 2), f32(4)), match="contiguous")
    rejects(ops.quantize_nvfp4_rht, x, 5, out=(u8(4, 16), u8(4, 2), f32(2)), match="outer")
    rejects(ops.quantize_nvfp4_2d, bf(16, 32), out=(u8(16, 16), u8(1, 1), f32(1)), match="scales")


def test_quantize_mxfp8_every_tensor():
    x = bf(64, 64)
    rejects(ops.quantize_mxfp8, x, row_gather=i64(64), match="row_gather")
    rejects(ops.quantize_mxfp8, x, colwise=True, group_offsets=i32(3), match="group_offsets")
    rejects(ops.quantize_mxfp8, x, colwise=True, group_offsets=i64(1), match="group_offsets")
    rejects(ops.quantize_mxfp8, x, out={"codes_row": u8(63, 64), "scales_row": u8(64, 2)}, match="codes_row")
    rejects(ops.quantize_mxfp8, x, out={"codes_row": u8(64, 64), "scales_row": u8(64, 1)}, match="scales_row")
    rejects(ops.quantize_mxfp8, x, out={"codes_row": u8(64, 64), "scales_row": None}, match="scales_row")
    rejects(ops.quantize_mxfp8, x, rowwise=False, out={"codes_colT": u8(63, 64), "scales_colT": u8(64, 2)},
            match="codes_colT")
    rejects(ops.quantize_mxfp8, x, rowwise=False, out={"codes_colT": u8(64, 64), "scales_colT": u8(64, 1)},
            match="scales_colT")
    # a stacked input: every output carries the batch
    rejects(ops.quantize_mxfp8, bf(3, 64, 64), out={"codes_row": u8(2, 64, 64), "scales_row": u8(3, 64, 2)},
            match="codes_row")


def test_dequantize_operands_and_output():
    c, s, g = u8(8, 16), u8(8, 2), f32(8)
    rejects(ops.dequantize, ops.FMT_NVFP4, c, u8(8, 1), g, match="scales")
    rejects(ops.dequantize, ops.FMT_NVFP4, c, s, None, match="outer")
    rejects(ops.dequantize, ops.FMT_NVFP4, c, s, f32(7), match="outer")
    rejects(ops.dequantize, ops.FMT_NVFP4, c, s, g, out=f32(8, 31), match="out")
    rejects(ops.dequantize, ops.FMT_NVFP4, c, s, g, out=i32(8, 32), match="dtype")
    rejects(ops.dequantize, ops.FMT_MXFP8, u8(8, 32), u8(8, 0), match="scales")


def test_requant_operands_outputs_workspace():
    c, s, g = u8(32, 16), u8(32, 2), f32(32)
    rejects(ops.requant_transpose_sr, c, u8(32, 1), g, match="scales")
    rejects(ops.requant_transpose_sr, c, s, f32(31), match="outer")
    rejects(ops.requant_transpose_sr, c, s, g, out=(u8(32, 15), u8(32, 2), f32(1)), match="codesT")
    rejects(ops.requant_transpose_sr, c, s, g, out=(u8(32, 16), u8(32, 2), f32(0)), match="outerT")
    rejects(ops.requant_transpose_sr, c, s, g, workspace=u8(3), match="workspace")
    rejects(ops.requant_transpose_sr_batched, c, s, f32(2), 2, 16, out=(u8(64, 8), u8(64, 1), f32(1)),
            match="outerT")
    off = i64(3)
    rejects(ops.requant_transpose_sr_grouped, c, s, g, off.int(), 32, match="group_offsets")
    rejects(ops.requant_transpose_sr_grouped, c, s, g, off, 32, gather=i64(32), match="gather")
    rejects(ops.requant_transpose_sr_grouped, c, s, g, off, 32, gather=i32(31), match="gather")
    rejects(ops.requant_transpose_sr_grouped, c, s, g, off, 32, ldT=96, out=(u8(32, 47), u8(32, 6), f32(2)),
            match="codesT")


def test_blockscaled_gemm_every_tensor():
    G, M, N, K = 2, 40, 64, 64
    off = i64(G + 1)
    a, as_ = u8(M, K // 2), u8(M, K // 16)
    b, bs = u8(G * N, K // 2), u8(G * N, K // 16)
    ag, bg = f32(M), f32(G)
    gm = ops.moe_grouped_gemm_blockscaled
    kw = dict(a_outer=ag, b_outer=bg)
    args = (ops.FMT_NVFP4, ops.GEMM_FPROP)
    rejects(gm, *args, a, as_, b, bs, off.int(), N, K, **kw, match="group_offsets")
    rejects(gm, *args, a, as_, b, bs, off, N, K + 32, **kw, match="a_codes")
    rejects(gm, *args, a, u8(M, 3), b, bs, off, N, K, **kw, match="a_scales")
    rejects(gm, *args, a, as_, u8(G * N - 1, K // 2), bs, off, N, K, **kw, match="b_codes")
    rejects(gm, *args, a, as_, b, u8(G * N, 3), off, N, K, **kw, match="b_scales")
    rejects(gm, *args, a, as_, b, bs, off, N, K, a_outer=f32(M - 1), b_outer=bg, match="a_outer")
    rejects(gm, *args, a, as_, b, bs, off, N, K, a_outer=ag, b_outer=None, match="b_outer")
    rejects(gm, *args, a, as_, b, bs, off, N, K, a_gather=i64(M), **kw, match="a_gather")
    rejects(gm, *args, a, as_, b, bs, off, N, K, M=M + 5, a_gather=i32(M), **kw, match="a_gather")
    rejects(gm, *args, a, as_, b, bs, off, N, K, out=f32(M, N - 1), **kw, match="out")
    rejects(gm, *args, a, as_, b, bs, off, N, K, out=torch.zeros(M, N, dtype=torch.float16), **kw, match="dtype")
    rejects(gm, *args, a, as_, b, bs, off, N, K, workspace=u8(3), **kw, match="workspace")
    # MXFP8 takes no outer scales
    rejects(gm, ops.FMT_MXFP8, ops.GEMM_FPROP, u8(M, K), u8(M, 2), u8(G * N, K), u8(G * N, 2), off, N, K,
            a_outer=ag, match="outer")
    # weight gradient: C [G, M, N]
    rejects(gm, ops.FMT_MXFP8, ops.GEMM_WGRAD, u8(M, K), u8(M, 2), u8(N, K), u8(N, 2), off, N, K, M=M,
            out=f32(1, M, N), match="out")


def test_bf16_gemm_every_tensor():
    G, M, N, K = 2, 40, 64, 32
    off = i64(G + 1)
    gm = ops.moe_grouped_gemm_bf16
    rejects(gm, ops.GEMM_FPROP, f32(M, K), bf(G * N, K), off, N, K, match="bfloat16|dtype")
    rejects(gm, ops.GEMM_FPROP, bf(M, K), bf(G * N - 1, K), off, N, K, match="b")
    rejects(gm, ops.GEMM_FPROP, bf(M, K), bf(G * N, K), off.int(), N, K, match="group_offsets")
    rejects(gm, ops.GEMM_FPROP, bf(M, K), bf(G * N, K), off, N, K, gather=i32(M - 1), M=M, match="gather")
    rejects(gm, ops.GEMM_DGRAD, bf(M, K), bf(G * K - 1, N), off, N, K, match="b")
    rejects(gm, ops.GEMM_WGRAD, bf(M, K), bf(M, N), off, N, M + 1, match="rows")
    rejects(gm, ops.GEMM_WGRAD, bf(M, K), bf(M, N), off, N, M, out=f32(G, K, N - 8), match="out")
    rejects(gm, ops.GEMM_FPROP, bf(M, K), bf(G * N, K), off, N, K, workspace=i32(4), match="workspace")


def test_swiglu_quantize_outputs():
    h13 = f32(8, 64)
    rejects(ops.swiglu_quantize, h13.to(torch.float16), match="dtype")
    rejects(ops.swiglu_quantize, h13, fmt=-1, out=(bf(8, 31), None, None, None), match="h")
    rejects(ops.swiglu_quantize, h13, fmt=ops.FMT_NVFP4, out=(None, u8(8, 15), u8(8, 2), f32(8)), match="codes")
    rejects(ops.swiglu_quantize, h13, fmt=ops.FMT_NVFP4, out=(None, u8(8, 16), u8(8, 2), None), match="outer")
    rejects(ops.swiglu_quantize, h13, fmt=ops.FMT_MXFP8, out=(None, u8(8, 32), u8(8, 0), None), match="scales")
