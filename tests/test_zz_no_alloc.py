"""The allocation-free grouped GEMM (bsp_moe_grouped_gemm_blockscaled_noalloc)
through the C ABI: its output must equal the workspace form's output bit for
bit (same kernels, same launch; only the workspace's address differs) and
meet the GEMM bound against the oracle, on consecutive calls whose second
problem is smaller than the first, so that anything the first call left in the
shared static scratch would show up in the second."""
import numpy as np
import pytest
import torch

import oracle
from block_scaled_precision_token_amd import ops, synth
from tests.gpu_util import assert_gemm_close, host, to_dev

pytestmark = pytest.mark.gpu


def offsets(counts):
    off = np.zeros(len(counts) + 1, np.int64)
    np.cumsum(counts, out=off[1:])
    return off


def rowgroup_case(fmt, T, K, N, counts, seed):
    off = offsets(counts)
    src = np.random.default_rng(seed).integers(0, T, int(off[-1])).astype(np.int32)
    x = synth.activations(seed + 1, T, K)
    w = synth.weights(seed + 2, len(counts), N, K)
    if fmt == ops.FMT_NVFP4:
        ac, as_, ag = oracle.quantize_nvfp4(x, mode46=True)
        bc, bs, bg = oracle.quantize_nvfp4(w, rows_per_scale=N)
    else:
        (ac, as_), (bc, bs) = oracle.quantize_mxfp8_rowwise(x), oracle.quantize_mxfp8_rowwise(w)
        ag = bg = None
    return off, src, (ac, as_, ag, bc, bs, bg)


def run_both(fmt, mode, N, K, off, src, q, out_dtype=torch.float32):
    ac, as_, ag, bc, bs, bg = q
    args = (fmt, mode, to_dev(ac), to_dev(as_), to_dev(bc), to_dev(bs), to_dev(off), N, K)
    kw = dict(a_outer=None if ag is None else to_dev(ag), b_outer=None if bg is None else to_dev(bg),
              a_gather=None if src is None else to_dev(src))
    ref = ops.moe_grouped_gemm_blockscaled(*args, out_dtype=out_dtype, **kw)
    out = torch.full_like(ref, float("nan"))
    ops.moe_grouped_gemm_blockscaled_noalloc(*args, out=out, **kw)
    torch.cuda.synchronize()
    got = host(out)
    assert np.array_equal(got.view(np.uint8), host(ref).view(np.uint8)), "noalloc differs from the workspace form"
    return got


@pytest.mark.parametrize("fmt", [ops.FMT_NVFP4, ops.FMT_MXFP8])
def test_noalloc_forward_two_calls_second_smaller(fmt):
    # call 1: 6 groups, 900 routed rows; call 2: 3 groups, 70 rows, shorter K and N
    for T, K, N, counts, seed in [(600, 512, 384, [300, 0, 129, 1, 270, 200], 11), (40, 64, 96, [10, 0, 60], 12)]:
        off, src, q = rowgroup_case(fmt, T, K, N, counts, seed)
        got = run_both(fmt, ops.GEMM_FPROP, N, K, off, src, q)
        ac, as_, ag, bc, bs, bg = q
        ref, refabs = oracle.gemm_rowgroup(fmt, ac, as_, ag, src, off, N, K, bc, bs, bg)
        assert_gemm_close(got, ref, refabs)


def test_noalloc_weight_gradient_then_smaller_forward():
    # the weight-gradient form's scratch layout (padded starts, expert order, scale planes), then a small forward
    counts = [50, 0, 64, 1, 100, 37]
    off = offsets(counts)
    R, G, NA, NB = int(off[-1]), len(counts), 160, 96
    dy = synth.activations(21, R, NA)
    h = synth.activations(22, R, NB)
    ld = ops.mxfp8_grouped_cols(R, G)
    ac, as_ = oracle.quantize_mxfp8_colwise(dy, off, ldT=ld)
    bc, bs = oracle.quantize_mxfp8_colwise(h, off, ldT=ld)
    args = (ops.FMT_MXFP8, ops.GEMM_WGRAD, to_dev(ac), to_dev(as_), to_dev(bc), to_dev(bs), to_dev(off), NB, ld)
    ref = ops.moe_grouped_gemm_blockscaled(*args, M=NA)
    out = torch.full_like(ref, float("nan"))
    ops.moe_grouped_gemm_blockscaled_noalloc(*args, M=NA, out=out)
    got = host(out)
    assert np.array_equal(got.view(np.uint8), host(ref).view(np.uint8))
    sel = np.array([[g, n] for g in range(G) for n in range(NA)], np.int64)
    r, rabs = oracle.gemm_wgrad(ac, as_, bc, bs, off, sel)
    assert_gemm_close(got.reshape(G * NA, NB), r, rabs)
    off2, src2, q2 = rowgroup_case(ops.FMT_NVFP4, 30, 96, 64, [7, 23], 23)
    got2 = run_both(ops.FMT_NVFP4, ops.GEMM_FPROP, 64, 96, off2, src2, q2, out_dtype=torch.bfloat16)
    ac2, as2, ag2, bc2, bs2, bg2 = q2
    r2, rabs2 = oracle.gemm_rowgroup(ops.FMT_NVFP4, ac2, as2, ag2, src2, off2, 64, 96, bc2, bs2, bg2)
    assert_gemm_close(synth.f32_from_bf16_bits(got2), r2, rabs2, bf16=True)


def test_noalloc_rejects_problems_beyond_the_scratch():
    # a valid call whose workspace exceeds the static scratch is refused before any launch
    G, N, K = 257, 4096, 7168
    need = ops.gemm_workspace_size(ops.FMT_MXFP8, ops.GEMM_FPROP, 36864, N, K, G)
    assert need > ops.GEMM_SCRATCH_BYTES
    dev = torch.device("cuda:0")
    off = torch.zeros(G + 1, dtype=torch.int64, device=dev)
    a = torch.empty((36864, K), dtype=torch.uint8, device=dev)
    a_s = torch.empty((36864, K // 32), dtype=torch.uint8, device=dev)
    b = torch.empty((G * N, K), dtype=torch.uint8, device=dev)          # never read: nothing is launched
    b_s = torch.empty((G * N, K // 32), dtype=torch.uint8, device=dev)
    out = torch.empty((36864, N), dtype=torch.bfloat16, device=dev)
    with pytest.raises(ops.BspError, match="SCRATCH_LIMIT"):
        ops.moe_grouped_gemm_blockscaled_noalloc(ops.FMT_MXFP8, ops.GEMM_FPROP, a, a_s, b, b_s, off, N, K, out=out)
