"""GPU parity of the quantize / dequantize / requant / SwiGLU kernels with the
CPU oracle: codes, scales and outer scales bit-exact, through the C ABI.

Shapes span several tiles with ragged tails and include the full sizes of the
synthetic workloads (256x2048 round trip, 8192x2048 MXFP8 activations, the
128 expert weights 2048x768, 16384x2048 requant), plus edge tensors: zeros,
negative zeros, bf16 maximum, bf16 subnormals, single outliers and values on
rounding midpoints.
"""
import numpy as np
import pytest
import torch

import oracle
from block_scaled_precision_token_amd import ops, synth
from tests.gpu_util import DEV, assert_bytes_equal, assert_swiglu_close, host, to_dev, to_dev_bf16

pytestmark = pytest.mark.gpu


def edge_tensor(M, K, seed=0):
    """Rows of edge cases followed by random rows."""
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((M, K)).astype(np.float32)
    if M >= 8:
        x[0] = 0.0
        x[1] = -0.0
        x[2] = 3.3895313892515355e38 * np.sign(rng.standard_normal(K))
        x[3] = 1e-39 * rng.standard_normal(K)                   # bf16 subnormals
        x[4] = 0.0
        x[4, K // 2] = 1000.0                                    # single outlier
        # exact E2M1 midpoints under outer scale 1 (2688 in the first block)
        mids = np.array([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0, 6.0], np.float32)
        x[5] = np.resize(np.concatenate([mids, -mids]) * 448.0 / 6.0 * 6.0 / 448.0, K)
        x[5, 0] = 2688.0
        # E4M3 midpoint block maxima: block amax / 6 lands between two E4M3 values
        x[6] = np.resize(np.array([6 * 8.5, 1, 2, 3], np.float32), K)
        x[6, 0] = 2688.0
        x[7] = rng.standard_normal(K) * 1e-30
    return synth.bf16_bits_from_f32(x)


# ---------------------------------------------------------------------------
# NVFP4
# ---------------------------------------------------------------------------

# K spans every lanes-per-row choice of the per-token kernel (16-value blocks
# per row: 1, 25, 3, 48, 63, 96, 128, 97, 160, 448; 13 and 21 rows leave the
# two-rows-per-wavefront form a partial last pair) and the scope kernel (8208)
@pytest.mark.parametrize("M,K", [(1, 16), (19, 400), (37, 48), (130, 768), (66, 1008), (45, 1536), (256, 2048),
                                 (13, 2048), (21, 1552), (11, 2560), (33, 7168), (9, 8208)])
@pytest.mark.parametrize("mode46", [False, True])
def test_nvfp4_per_token_parity(M, K, mode46):
    x = edge_tensor(M, K, seed=M * 31 + K)
    c, s, g = ops.quantize_nvfp4_per_token(to_dev_bf16(x), mode46=mode46)
    rc, rs, rg = oracle.quantize_nvfp4(x, mode46=mode46)
    assert_bytes_equal(host(g), rg, "outer")
    assert_bytes_equal(host(s), rs, "scales")
    assert_bytes_equal(host(c), rc, "codes")


def test_nvfp4_round_trip_config_outliers():
    # 256 x 2048 activations, N(0,1) with 0.1% outliers x50
    x = synth.activations(20261201, 256, 2048)
    for m46 in (False, True):
        c, s, g = ops.quantize_nvfp4_per_token(to_dev_bf16(x), mode46=m46)
        rc, rs, rg = oracle.quantize_nvfp4(x, mode46=m46)
        assert_bytes_equal(host(c), rc, "codes")
        assert_bytes_equal(host(s), rs, "scales")
        assert_bytes_equal(host(g), rg, "outer")


@pytest.mark.parametrize("E,N,K", [(3, 48, 64), (4, 768, 2048), (2, 100, 32)])
def test_nvfp4_per_expert_scope(E, N, K):
    w = synth.weights(7 + N, E, N, K)
    w[3, 5] = synth.bf16_bits_from_f32(np.float32([3.0]))[0]
    c, s, g = ops.quantize_nvfp4_per_token(to_dev_bf16(w), rows_per_scale=N)
    rc, rs, rg = oracle.quantize_nvfp4(w, rows_per_scale=N)
    assert_bytes_equal(host(g), rg, "outer")
    assert_bytes_equal(host(s), rs, "scales")
    assert_bytes_equal(host(c), rc, "codes")


def test_nvfp4_per_tensor_scope_and_row_stride():
    x = synth.activations(55, 64, 160)
    big = np.zeros((64, 200), np.uint16)
    big[:, :160] = x
    xd = to_dev_bf16(big)[:, :160]
    c, s, g = ops.quantize_nvfp4_per_token(xd, rows_per_scale=64, mode46=True)
    rc, rs, rg = oracle.quantize_nvfp4(x, rows_per_scale=64, mode46=True)
    assert_bytes_equal(host(g), rg, "outer")
    assert_bytes_equal(host(c), rc, "codes")
    assert_bytes_equal(host(s), rs, "scales")


def test_nvfp4_batch_invariance_on_device():
    x = synth.activations(77, 64, 512)
    y = x.copy()
    y[1:] = synth.activations(78, 63, 512)
    a = ops.quantize_nvfp4_per_token(to_dev_bf16(x), mode46=True)
    b = ops.quantize_nvfp4_per_token(to_dev_bf16(y[:1]), mode46=True)   # M = 1 vs M = 64
    assert_bytes_equal(host(a[0])[0], host(b[0])[0], "codes row 0")
    assert_bytes_equal(host(a[1])[0], host(b[1])[0], "scales row 0")


# ---------------------------------------------------------------------------
# MXFP8
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("M,K", [(32, 32), (96, 96), (160, 192), (8192, 2048)])
def test_mxfp8_row_and_col_parity(M, K):
    if M == 8192:
        x = synth.activations(20261202, M, K, row_log10_range=(-3, 2))
    else:
        x = edge_tensor(M, K, seed=M + K)
    q = ops.quantize_mxfp8(to_dev_bf16(x), rowwise=True, colwise=True)
    rc, rs = oracle.quantize_mxfp8_rowwise(x)
    tc, ts = oracle.quantize_mxfp8_colwise(x)
    assert_bytes_equal(host(q["scales_row"]), rs, "row scales")
    assert_bytes_equal(host(q["codes_row"]), rc, "row codes")
    assert_bytes_equal(host(q["scales_colT"]), ts, "col scales")
    assert_bytes_equal(host(q["codes_colT"]), tc, "col codes")


def test_mxfp8_colwise_only_and_rowwise_only():
    x = edge_tensor(64, 128, seed=3)
    q = ops.quantize_mxfp8(to_dev_bf16(x), rowwise=False, colwise=True)
    tc, ts = oracle.quantize_mxfp8_colwise(x)
    assert_bytes_equal(host(q["codes_colT"]), tc, "col codes")
    assert_bytes_equal(host(q["scales_colT"]), ts, "col scales")
    q = ops.quantize_mxfp8(to_dev_bf16(x), rowwise=True, colwise=False)
    rc, rs = oracle.quantize_mxfp8_rowwise(x)
    assert_bytes_equal(host(q["codes_row"]), rc, "row codes")
    assert_bytes_equal(host(q["scales_row"]), rs, "row scales")


def test_mxfp8_expert_weights_full_size():
    # 128 expert weights of 2048 x 768 (blocks along 768), one launch over [262144, 768]
    w = synth.weights(20261203, 128, 2048, 768)
    q = ops.quantize_mxfp8(to_dev_bf16(w), rowwise=True)
    rc, rs = oracle.quantize_mxfp8_rowwise(w)
    assert_bytes_equal(host(q["scales_row"]), rs, "scales")
    assert_bytes_equal(host(q["codes_row"]), rc, "codes")


@pytest.mark.parametrize("counts", [[5, 0, 35, 60], [1, 31, 32, 33, 0, 0, 64, 200], [0, 0, 7]])
def test_mxfp8_grouped_columnwise(counts):
    off = np.zeros(len(counts) + 1, np.int64)
    np.cumsum(counts, out=off[1:])
    M = int(off[-1])
    x = synth.activations(sum(counts), M, 96)
    G = len(counts)
    ld = ops.mxfp8_grouped_cols(M, G)
    q = ops.quantize_mxfp8(to_dev_bf16(x), rowwise=True, colwise=True, group_offsets=to_dev(off))
    P = oracle.padded_offsets(off)
    tc, ts = oracle.quantize_mxfp8_colwise(x, off, ldT=ld)
    used = int(P[-1])
    assert_bytes_equal(host(q["codes_colT"])[:, :used], tc[:, :used], "grouped col codes")
    assert_bytes_equal(host(q["scales_colT"])[:, :used // 32], ts[:, :used // 32], "grouped col scales")
    rc, rs = oracle.quantize_mxfp8_rowwise(x)
    assert_bytes_equal(host(q["codes_row"]), rc, "row codes")


@pytest.mark.parametrize("grouped", [False, True])
def test_mxfp8_with_row_gather(grouped):
    T, R = 50, 96
    x = synth.activations(91, T, 64)
    rng = np.random.default_rng(92)
    src = rng.integers(0, T, R).astype(np.int32)
    xg = x[src]
    if grouped:
        off = np.array([0, 10, 10, 70, 96], np.int64)
        q = ops.quantize_mxfp8(to_dev_bf16(x), rowwise=True, colwise=True, group_offsets=to_dev(off),
                               row_gather=to_dev(src))
        ld = q["codes_colT"].shape[1]
        tc, ts = oracle.quantize_mxfp8_colwise(xg, off, ldT=ld)
        used = int(oracle.padded_offsets(off)[-1])
        assert_bytes_equal(host(q["codes_colT"])[:, :used], tc[:, :used], "gathered grouped col codes")
        assert_bytes_equal(host(q["scales_colT"])[:, :used // 32], ts[:, :used // 32], "gathered grouped col scales")
    else:
        q = ops.quantize_mxfp8(to_dev_bf16(x), rowwise=True, colwise=True, row_gather=to_dev(src))
        tc, ts = oracle.quantize_mxfp8_colwise(xg)
        assert_bytes_equal(host(q["codes_colT"]), tc, "gathered col codes")
        assert_bytes_equal(host(q["scales_colT"]), ts, "gathered col scales")
    rc, rs = oracle.quantize_mxfp8_rowwise(xg)
    assert_bytes_equal(host(q["codes_row"]), rc, "gathered row codes")
    assert_bytes_equal(host(q["scales_row"]), rs, "gathered row scales")
    # rowwise-only kernel with a gather
    q = ops.quantize_mxfp8(to_dev_bf16(x), rowwise=True, colwise=False, row_gather=to_dev(src))
    assert_bytes_equal(host(q["codes_row"]), rc, "gathered row-only codes")


@pytest.mark.parametrize("rowwise", [True, False])
def test_mxfp8_batched_per_expert_columnwise(rowwise):
    # stacked expert weights [E, N, K]: one launch, per-expert columnwise copies
    E, N, K = 3, 96, 64
    w = synth.weights(93, E, N, K)
    q = ops.quantize_mxfp8(to_dev_bf16(w).reshape(E, N, K), rowwise=rowwise, colwise=True)
    for e in range(E):
        tc, ts = oracle.quantize_mxfp8_colwise(w[e * N:(e + 1) * N])
        assert_bytes_equal(host(q["codes_colT"][e]), tc, f"expert {e} col codes")
        assert_bytes_equal(host(q["scales_colT"][e]), ts, f"expert {e} col scales")
        if rowwise:
            rc, rs = oracle.quantize_mxfp8_rowwise(w[e * N:(e + 1) * N])
            assert_bytes_equal(host(q["codes_row"][e]), rc, f"expert {e} row codes")
            assert_bytes_equal(host(q["scales_row"][e]), rs, f"expert {e} row scales")


# ---------------------------------------------------------------------------
# dequantize
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("out_dtype", [torch.float32, torch.bfloat16])
def test_dequantize_parity(out_dtype):
    x = edge_tensor(48, 224, seed=9)
    rc, rs, rg = oracle.quantize_nvfp4(x, mode46=True)
    f = ops.dequantize(ops.FMT_NVFP4, to_dev(rc), to_dev(rs), to_dev(rg), out_dtype=out_dtype)
    rf, rb = oracle.dequantize_nvfp4(rc, rs, rg)
    assert_bytes_equal(host(f), rf if out_dtype == torch.float32 else rb, "nvfp4 dequant")
    mc, ms = oracle.quantize_mxfp8_rowwise(x)
    f = ops.dequantize(ops.FMT_MXFP8, to_dev(mc), to_dev(ms), out_dtype=out_dtype)
    rf, rb = oracle.dequantize_mxfp8(mc, ms)
    assert_bytes_equal(host(f), rf if out_dtype == torch.float32 else rb, "mxfp8 dequant")


@pytest.mark.parametrize("E,N,K", [(3, 32, 64), (8, 256, 2048)])
@pytest.mark.parametrize("out_dtype", [torch.float32, torch.bfloat16])
def test_dequantize_per_expert_scope(E, N, K, out_dtype):
    w = synth.weights(31 + K, E, N, K)
    rc, rs, rg = oracle.quantize_nvfp4(w, rows_per_scale=N)
    f = ops.dequantize(ops.FMT_NVFP4, to_dev(rc), to_dev(rs), to_dev(rg), rows_per_scale=N, out_dtype=out_dtype)
    rf, rb = oracle.dequantize_nvfp4(rc, rs, rg, rows_per_scale=N)
    assert_bytes_equal(host(f), rf if out_dtype == torch.float32 else rb, "dequant per expert")


# ---------------------------------------------------------------------------
# requant + SR
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("M,K", [(16, 16), (48, 80), (272, 144), (528, 272), (768, 384), (2048, 512),
                                 (16384, 2048)])
@pytest.mark.parametrize("sr", [True, False])
def test_requant_parity(M, K, sr):
    x = synth.activations(20261203 + M, M, K)
    rc, rs, rg = oracle.quantize_nvfp4(x)
    seed = 0x5EED + M
    ct, st, gt = ops.requant_transpose_sr(to_dev(rc), to_dev(rs), to_dev(rg), seed=seed, sr=sr)
    rct, rst, rgt = oracle.requant_transpose_sr(rc, rs, rg, seed=seed, use_sr=sr)
    assert_bytes_equal(host(gt), rgt, "outerT")
    assert_bytes_equal(host(st), rst, "scalesT")
    assert_bytes_equal(host(ct), rct, "codesT")


@pytest.mark.parametrize("M,K", [(272, 144), (512, 256)])
@pytest.mark.parametrize("sr", [True, False])
def test_requant_arbitrary_operands(M, K, sr):
    """Codes, scales and outer scales drawn directly rather than produced by
    the quantizer: every code, negative and subnormal E4M3 scales, zero and
    tiny outer scales (flushed blocks), and values v up to 9 after the
    rescale, so that every rounding branch is taken."""
    rng = np.random.default_rng(20261210 + M)
    rc = rng.integers(0, 256, size=(M, K // 2), dtype=np.uint8)
    rs = rng.integers(0, 256, size=(M, K // 16), dtype=np.uint8)
    rs[(rs & 0x7F) == 0x7F] = 0x3F          # E4M3FN has no 0x7F / 0xFF value
    rg = (10.0 ** rng.uniform(-3, 3, size=M)).astype(np.float32)
    rg[::37] = 0.0
    rg[5] = 1e-37
    seed = 0xC0FFEE + M
    ct, st, gt = ops.requant_transpose_sr(to_dev(rc), to_dev(rs), to_dev(rg), seed=seed, sr=sr)
    rct, rst, rgt = oracle.requant_transpose_sr(rc, rs, rg, seed=seed, use_sr=sr)
    assert_bytes_equal(host(gt), rgt, "outerT")
    assert_bytes_equal(host(st), rst, "scalesT")
    assert_bytes_equal(host(ct), rct, "codesT")


def test_requant_worked_example_on_device():
    x = np.zeros((16, 32), np.float32)
    x[0, 0] = 2688.0
    x[0, 16] = -54.0
    x[0, 17] = 5.4
    x[1, 0] = 2688.0
    x[1, 17] = 12.0
    xb = synth.bf16_bits_from_f32(x)
    c, s, g = ops.quantize_nvfp4_per_token(to_dev_bf16(xb))
    ups = 0
    n = 256
    for seed in range(n):
        ct, st, gt = ops.requant_transpose_sr(c, s, g, seed=seed, sr=True)
        code = int(host(ct)[17, 0] & 15)
        assert code in (4, 5)
        ups += code == 5
    # P(3) = 1/4 exactly per element draw; 256 draws within 5 sigma
    assert abs(ups / n - 0.25) < 5 * np.sqrt(0.25 * 0.75 / n)
    ct, st, gt = ops.requant_transpose_sr(c, s, g, sr=False)
    assert int(host(ct)[17, 0] & 15) == 4 and int(host(st)[17, 0]) == 0x40   # element 2, scale 2


@pytest.mark.parametrize("E,M,K,rps", [(3, 272, 144, 272), (4, 512, 256, 1), (2, 256, 2048, 512),
                                        (128, 48, 32, 48)])
@pytest.mark.parametrize("sr", [True, False])
def test_requant_batched_parity(E, M, K, rps, sr):
    """Per-expert tensors requantized on their own (own G_e; SR bits indexed in
    the stacked output), against the oracle: per-expert weight scales
    (rps = M), per-row scales (rps = 1) and one scale over two tensors."""
    w = synth.weights(20261215 + M, E, M, K)
    if rps == 1:
        rc, rs, rg = oracle.quantize_nvfp4(w)
    else:
        rc, rs, rg = oracle.quantize_nvfp4(w, rows_per_scale=rps)
    seed = 0xBA7C + E
    ct, st, gt = ops.requant_transpose_sr_batched(to_dev(rc), to_dev(rs), to_dev(rg), E, rps, seed=seed, sr=sr)
    rct, rst, rgt = oracle.requant_transpose_sr_batched(rc, rs, rg, E, rps, seed=seed, use_sr=sr)
    assert_bytes_equal(host(gt)[:E], rgt, "outerT")
    assert_bytes_equal(host(st), rst, "scalesT")
    assert_bytes_equal(host(ct), rct, "codesT")


GROUPED_RQ_CASES = [
    # (source rows, K, rows per group, gather)
    (40, 64, [21, 0, 39, 33], True),
    (300, 272, [129, 0, 128, 1, 142, 31, 32], True),
    (256, 2048, [64, 64, 0, 128], False),
    (8192, 2048, None, True),          # Qwen3-shaped: 65,536 routed rows of 8192 tokens, 128 experts
]


@pytest.mark.parametrize("T,K,counts,gathered", GROUPED_RQ_CASES)
@pytest.mark.parametrize("sr", [True, False])
def test_requant_grouped_parity(T, K, counts, gathered, sr):
    """Token-blocked operands of the 4-bit weight gradient: rows of each group
    (through the routing map, bad indices read as zeros), each group
    requantized with its own G_g into 32-padded columns; bit-exact against the
    oracle, columns past the padded total untouched."""
    if counts is None:
        off, src = synth.route_topk(20261205, T, 128, 8, synth.zipf_bias(20261204, 128))
    else:
        off = np.concatenate([[0], np.cumsum(counts)]).astype(np.int64)
        rng = np.random.default_rng(T + K)
        src = rng.integers(0, T, int(off[-1])).astype(np.int32)
        if src.size > 8:
            src[2] = -1
            src[src.size // 2] = T + 5
    R = int(off[-1])
    if not gathered:
        src = None
        T = R
    x = synth.activations(20261216 + K, T, K)
    rc, rs, rg = oracle.quantize_nvfp4(x, mode46=True)
    G = off.size - 1
    ldT = ops.mxfp8_grouped_cols(R, G) + 32
    seed = 0x6A0B + K
    ct, st, gt = ops.requant_transpose_sr_grouped(to_dev(rc), to_dev(rs), to_dev(rg), to_dev(off), R, ldT=ldT,
                                                  gather=None if src is None else to_dev(src), seed=seed, sr=sr)
    rct, rst, rgt = oracle.requant_transpose_sr_grouped(rc, rs, rg, src, off, ldT, seed=seed, use_sr=sr)
    assert_bytes_equal(host(gt)[:G], rgt, "outerT")
    assert_bytes_equal(host(st), rst, "scalesT")
    assert_bytes_equal(host(ct), rct, "codesT")


@pytest.mark.parametrize("M,K", [(64, 2048), (37, 4096), (8, 16), (16, 8192), (24, 768), (13, 1536)])
@pytest.mark.parametrize("m46", [False, True])
def test_nvfp4_rht_parity(M, K, m46):
    x = synth.activations(20261222 + K, M, K)
    signs = 0x9C35 ^ K
    c, s, g = ops.quantize_nvfp4_rht(to_dev_bf16(x), signs, mode46=m46)
    rc, rs, rg = oracle.quantize_nvfp4_rht(x, signs, mode46=m46)
    assert_bytes_equal(host(g), rg, "outer")
    assert_bytes_equal(host(s), rs, "scales")
    assert_bytes_equal(host(c), rc, "codes")


@pytest.mark.parametrize("M,K", [(64, 2048), (48, 272), (16, 16), (256, 7168)])
def test_nvfp4_2d_parity(M, K):
    x = synth.activations(20261223 + K, M, K)
    c, s, g = ops.quantize_nvfp4_2d(to_dev_bf16(x))
    rc, rs, rg = oracle.quantize_nvfp4_2d(x)
    assert_bytes_equal(host(g)[:1], rg, "outer")
    assert_bytes_equal(host(s), rs, "scales")
    assert_bytes_equal(host(c), rc, "codes")


def test_nvfp4_2d_outlier_tile_on_device():
    # the pages' example: one large value among 256 flattens the other 255
    x = np.full((16, 32), 0.75, np.float32)
    x[0, 0] = 2688.0
    c, s, g = ops.quantize_nvfp4_2d(to_dev_bf16(synth.bf16_bits_from_f32(x)))
    c = host(c)
    mags = np.stack([c & 7, (c >> 4) & 7], axis=-1).reshape(16, 32)
    assert mags[0, 0] == 7 and np.count_nonzero(mags[:, :16]) == 1 and np.count_nonzero(mags[:, 16:]) == 256


# ---------------------------------------------------------------------------
# SwiGLU + quantize
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("R,I", [(5, 32), (37, 480), (19, 640), (130, 768), (21, 992), (7, 1280), (44, 1536),
                                 (17, 2048), (9, 4096)])
@pytest.mark.parametrize("fmt,m46", [(-1, False), (0, True), (0, False), (1, False)])
@pytest.mark.parametrize("in_dtype", ["f32", "bf16"])
def test_swiglu_quantize_parity(R, I, fmt, m46, in_dtype):
    h13 = synth.fp32_matrix(R * 7 + I, R, 2 * I, std=2.5)
    # gate values at and past the ends of exp's range (exp(-z) is inf from
    # z = -89 and 0 from z = 104), signed zeros, large magnitudes
    h13[0, :16] = [0.0, -0.0, 90.0, -120.0, 89.0, -89.0, 104.0, -104.0, 88.5, -103.5, 1e4, -1e4,
                   -88.75, 103.75, 0.5, -0.5]
    if in_dtype == "bf16":
        hb = synth.bf16_bits_from_f32(h13)
        h13 = synth.f32_from_bf16_bits(hb)
        dev_in = to_dev_bf16(hb)
    else:
        dev_in = to_dev(h13)
    h, c, s, g = ops.swiglu_quantize(dev_in, fmt=fmt, mode46=m46, return_h=True)
    # stage 1: h within one bf16 unit of the oracle's binary64 SwiGLU
    hd = host(h)
    assert_swiglu_close(hd, h13)
    # stage 2: the device's own h quantized bit for bit as the oracle quantizes it
    if fmt == 0:
        rc, rs, rg = oracle.quantize_nvfp4(hd, mode46=m46)
        assert_bytes_equal(host(g), rg, "outer")
        assert_bytes_equal(host(s), rs, "scales")
        assert_bytes_equal(host(c), rc, "codes")
    elif fmt == 1:
        rc, rs = oracle.quantize_mxfp8_rowwise(hd)
        assert_bytes_equal(host(s), rs, "scales")
        assert_bytes_equal(host(c), rc, "codes")
