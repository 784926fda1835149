"""GPU parity of the exact kernel configurations that the timed workload steps
run, at their full sizes, through the C ABI: each call below is the call the
step makes (same entry point, same flags, same shapes and routing), checked
byte for byte against the oracle -- in full where the oracle finishes in a
few seconds, else on sampled experts and groups (largest, smallest, the
shared expert and random ones) -- plus small cases that reach the same code
branches cheaply:

  - DeepSeek-V3-shaped MXFP8 step: the batched rowwise + per-expert
    columnwise quantization of the 257 experts' W13 [4096, 7168] and W2
    [7168, 2048]; X rowwise; the grouped columnwise copy of X read through
    the routing map (257 groups); the rowwise + grouped columnwise copies of
    h, dY and dH13;
  - more than 256 groups (the padded group starts are computed over several
    groups per thread): grouped MXFP8 and grouped requant with 257 and 300
    groups, empty groups, with and without a gather;
  - per-token NVFP4 of rows with 1537..2048 values once M > 8188 (one row per
    wavefront), both modes, at the 4-bit backward's 65,536 x 2048;
  - rowwise-only MXFP8 of tensors of at least 2^26 values (the tile kernel
    without its column pass; smaller ones take the lane-per-block kernel):
    the MXFP8 quantization workload's 128 expert weights [2048, 768], and a
    gathered rowwise copy of 65,536 routed rows of 2048;
  - the Qwen3-shaped NVFP4 down GEMM and the 4-bit backward's NVFP4 data- and
    weight-gradient GEMMs at full size on sampled rows and groups.
"""
import numpy as np
import pytest
import torch

import oracle
from block_scaled_precision_token_amd import ops, synth
from tests.gpu_util import DEV, assert_bytes_equal, assert_gemm_close, host, to_dev, to_dev_bf16

pytestmark = pytest.mark.gpu


def bits(t):
    """bf16 device tensor -> host uint16 bits."""
    return host(t)


def ragged_groups(G, seed, max_rows=40, empty_every=7):
    rng = np.random.default_rng(seed)
    counts = rng.integers(0, max_rows + 1, G)
    counts[::empty_every] = 0
    counts[1] = 32
    counts[2] = 33
    off = np.zeros(G + 1, np.int64)
    np.cumsum(counts, out=off[1:])
    return off


# ---------------------------------------------------------------------------
# more than 256 groups
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("G", [257, 300])
@pytest.mark.parametrize("gathered", [False, True])
@pytest.mark.parametrize("rowwise", [False, True])
def test_mxfp8_grouped_many_groups(G, gathered, rowwise):
    off = ragged_groups(G, G + 11)
    R = int(off[-1])
    K = 96
    if gathered:
        T = 500
        x = synth.activations(G + 12, T, K)
        src = np.random.default_rng(G).integers(0, T, R).astype(np.int32)
        src[3] = -1                                 # out-of-range entries read as zero rows
        src[R // 2] = T + 7
        xg = np.where((src >= 0) & (src < T), 1, 0)[:, None] * x[np.clip(src, 0, T - 1)]
        xg = xg.astype(np.uint16)
        q = ops.quantize_mxfp8(to_dev_bf16(x), rowwise, True, group_offsets=to_dev(off), row_gather=to_dev(src))
    else:
        xg = synth.activations(G + 12, R, K)
        q = ops.quantize_mxfp8(to_dev_bf16(xg), rowwise, True, group_offsets=to_dev(off))
    ld = q["codes_colT"].shape[1]
    assert ld == ops.mxfp8_grouped_cols(R, G)
    used = int(oracle.padded_offsets(off)[-1])
    tc, ts = oracle.quantize_mxfp8_colwise(xg, off, ldT=ld)
    assert_bytes_equal(host(q["codes_colT"])[:, :used], tc[:, :used], "grouped col codes")
    assert_bytes_equal(host(q["scales_colT"])[:, :used // 32], ts[:, :used // 32], "grouped col scales")
    if rowwise:
        rc, rs = oracle.quantize_mxfp8_rowwise(xg)
        assert_bytes_equal(host(q["codes_row"]), rc, "row codes")
        assert_bytes_equal(host(q["scales_row"]), rs, "row scales")


@pytest.mark.parametrize("G", [257, 300])
@pytest.mark.parametrize("gathered", [False, True])
def test_requant_grouped_many_groups(G, gathered):
    off = ragged_groups(G, G + 21)
    R = int(off[-1])
    K = 80
    if gathered:
        T = 600
        src = np.random.default_rng(G + 1).integers(0, T, R).astype(np.int32)
        src[5] = -2
    else:
        T, src = R, None
    x = synth.activations(G + 22, T, K)
    rc, rs, rg = oracle.quantize_nvfp4(x, mode46=True)
    ldT = ops.mxfp8_grouped_cols(R, G) + 64
    for sr in (True, False):
        ct, st, gt = ops.requant_transpose_sr_grouped(to_dev(rc), to_dev(rs), to_dev(rg), to_dev(off), R, ldT=ldT,
                                                      gather=None if src is None else to_dev(src), seed=G, sr=sr)
        rct, rst, rgt = oracle.requant_transpose_sr_grouped(rc, rs, rg, src, off, ldT, seed=G, use_sr=sr)
        assert_bytes_equal(host(gt)[:G], rgt, "outerT")
        assert_bytes_equal(host(st), rst, "scalesT")
        assert_bytes_equal(host(ct), rct, "codesT")


# ---------------------------------------------------------------------------
# per-token NVFP4, K in (1536, 2048], more than 8188 rows
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("M,K", [(8196, 1552), (8196, 2048), (65536, 2048)])
@pytest.mark.parametrize("mode46", [False, True])
def test_nvfp4_per_token_one_row_per_wavefront(M, K, mode46):
    xd = synth.device_activations(M + K + mode46, M, K, device=DEV)
    xd[7] = 0                                          # a zero row: g = 0
    x = bits(xd)
    c, s, g = ops.quantize_nvfp4_per_token(xd, mode46=mode46)
    rc, rs, rg = oracle.quantize_nvfp4(x, mode46=mode46)
    assert_bytes_equal(host(g), rg, "outer")
    assert_bytes_equal(host(s), rs, "scales")
    assert_bytes_equal(host(c), rc, "codes")


# ---------------------------------------------------------------------------
# DeepSeek-V3-shaped MXFP8 quantization, as the timed step calls it
# ---------------------------------------------------------------------------

T_D, H_D, I_D, E_D, TOPK_D = 4096, 7168, 2048, 256, 8
N13_D = 2 * I_D
SEED = 20261301


def test_mxfp8_rowwise_only_large_batched_weights():
    E, N, K = 128, 2048, 768        # the MXFP8 quantization workload's weights: 2^27.6 values
    w = synth.device_weights(SEED + 41, E, N, K, device=DEV)
    q = ops.quantize_mxfp8(w.view(E, N, K), True, False)
    for e in (0, 1, 63, 127):
        rc, rs = oracle.quantize_mxfp8_rowwise(bits(w[e * N:(e + 1) * N]))
        assert_bytes_equal(host(q["codes_row"][e]), rc, f"expert {e} row codes")
        assert_bytes_equal(host(q["scales_row"][e]), rs, f"expert {e} row scales")


def test_mxfp8_rowwise_only_large_gathered():
    T, K, R = 8192, 2048, 65536     # 2^27 gathered values
    x = synth.device_activations(SEED + 42, T, K, device=DEV)
    rng = np.random.default_rng(SEED + 43)
    src = rng.integers(0, T, R).astype(np.int32)
    src[::1000] = -1                # out-of-range indices read as zero rows
    src[7] = T
    q = ops.quantize_mxfp8(x, True, False, row_gather=to_dev(src))
    xh = bits(x)
    rows = np.r_[0:64, 7, 1000, 2000, R - 64:R, rng.integers(0, R, 256)]
    xs = np.where(((src[rows] >= 0) & (src[rows] < T))[:, None], xh[np.clip(src[rows], 0, T - 1)], 0).astype(np.uint16)
    rc, rs = oracle.quantize_mxfp8_rowwise(xs)
    assert_bytes_equal(host(q["codes_row"])[rows], rc, "gathered row codes")
    assert_bytes_equal(host(q["scales_row"])[rows], rs, "gathered row scales")


@pytest.fixture(scope="module")
def dsv3():
    off, src = synth.route_topk(SEED, T_D, E_D, TOPK_D, synth.zipf_bias(SEED + 1, E_D, 1.1, uniform_mix=0.5),
                                shared_expert=True)
    counts = np.diff(off)
    rng = np.random.default_rng(SEED + 2)
    sampled = sorted({int(np.argmax(counts[:-1])), int(np.argmin(counts[:-1])), E_D,
                      *rng.integers(0, E_D, 2).tolist()})
    return off, src, sampled


@pytest.mark.parametrize("which,N,K", [("w13", N13_D, H_D), ("w2", H_D, I_D)])
def test_dsv3_weights_row_col_sampled_experts(dsv3, which, N, K):
    _, _, sampled = dsv3
    G = E_D + 1
    w = synth.device_weights(SEED + 3 + (which == "w2"), G, N, K, device=DEV)
    q = ops.quantize_mxfp8(w.view(G, N, K), True, True)
    for e in sampled:
        we = bits(w[e * N:(e + 1) * N])
        rc, rs = oracle.quantize_mxfp8_rowwise(we)
        assert_bytes_equal(host(q["codes_row"][e]), rc, f"{which} expert {e} row codes")
        assert_bytes_equal(host(q["scales_row"][e]), rs, f"{which} expert {e} row scales")
        tc, ts = oracle.quantize_mxfp8_colwise(we)
        assert_bytes_equal(host(q["codes_colT"][e]), tc, f"{which} expert {e} col codes")
        assert_bytes_equal(host(q["scales_colT"][e]), ts, f"{which} expert {e} col scales")


def test_dsv3_x_rowwise_and_gathered_grouped_columnwise(dsv3):
    off, src, _ = dsv3
    R, G = int(off[-1]), E_D + 1
    x = synth.device_activations(SEED + 5, T_D, H_D, device=DEV)
    xh = bits(x)
    q = ops.quantize_mxfp8(x, True, False)
    rc, rs = oracle.quantize_mxfp8_rowwise(xh)
    assert_bytes_equal(host(q["codes_row"]), rc, "x row codes")
    assert_bytes_equal(host(q["scales_row"]), rs, "x row scales")
    del rc
    qg = ops.quantize_mxfp8(x, False, True, group_offsets=to_dev(off), row_gather=to_dev(src))
    ld = qg["codes_colT"].shape[1]
    used = int(oracle.padded_offsets(off)[-1])
    tc, ts = oracle.quantize_mxfp8_colwise(xh[src], off, ldT=ld)
    assert_bytes_equal(host(qg["scales_colT"])[:, :used // 32], ts[:, :used // 32], "x grouped col scales")
    assert_bytes_equal(host(qg["codes_colT"])[:, :used], tc[:, :used], "x grouped col codes")


@pytest.mark.parametrize("which,K", [("h", I_D), ("dy", H_D), ("dh13", N13_D)])
def test_dsv3_routed_rows_row_and_grouped_col(dsv3, which, K):
    off, _, _ = dsv3
    R = int(off[-1])
    a = synth.device_activations(SEED + 6 + K, R, K, device=DEV, std=0.5 if which == "h" else 1.0)
    q = ops.quantize_mxfp8(a, True, True, group_offsets=to_dev(off))
    ah = bits(a)
    del a
    rc, rs = oracle.quantize_mxfp8_rowwise(ah)
    assert_bytes_equal(host(q["scales_row"]), rs, f"{which} row scales")
    assert_bytes_equal(host(q["codes_row"]), rc, f"{which} row codes")
    del rc
    ld = q["codes_colT"].shape[1]
    used = int(oracle.padded_offsets(off)[-1])
    tc, ts = oracle.quantize_mxfp8_colwise(ah, off, ldT=ld)
    assert_bytes_equal(host(q["scales_colT"])[:, :used // 32], ts[:, :used // 32], f"{which} grouped col scales")
    assert_bytes_equal(host(q["codes_colT"])[:, :used], tc[:, :used], f"{which} grouped col codes")


# ---------------------------------------------------------------------------
# Qwen3-shaped NVFP4 GEMMs at full size
# ---------------------------------------------------------------------------

T_Q, E_Q, TOPK_Q, H_Q, I_Q = 8192, 128, 8, 2048, 768
N13_Q = 2 * I_Q


@pytest.fixture(scope="module")
def qwen3():
    off, src = synth.route_topk(SEED + 20, T_Q, E_Q, TOPK_Q, synth.zipf_bias(SEED + 21, E_Q))
    return off, src


def sample_rows(off, n, seed):
    rng = np.random.default_rng(seed)
    big = int(np.argmax(np.diff(off)))
    return np.unique(np.concatenate([rng.integers(0, off[-1], n), [0, off[-1] - 1, off[big], off[big + 1] - 1]]))


def test_qwen3_nvfp4_down_gemm_sampled_rows(qwen3):
    # Y = h W2_e^T: h [65536, 768] per-token NVFP4 (4/6), W2 128 x [2048, 768] per expert
    off, _ = qwen3
    R = int(off[-1])
    h = bits(synth.device_activations(SEED + 22, R, I_Q, device=DEV, std=0.5))
    ac, as_, ag = oracle.quantize_nvfp4(h, mode46=True)
    w2 = bits(synth.device_weights(SEED + 23, E_Q, H_Q, I_Q, device=DEV))
    bc, bs, bg = oracle.quantize_nvfp4(w2, rows_per_scale=H_Q)
    del w2
    y = ops.moe_grouped_gemm_blockscaled(ops.FMT_NVFP4, ops.GEMM_FPROP, to_dev(ac), to_dev(as_), to_dev(bc),
                                         to_dev(bs), to_dev(off), H_Q, I_Q, a_outer=to_dev(ag), b_outer=to_dev(bg),
                                         out_dtype=torch.bfloat16)
    rows = sample_rows(off, 48, 3)
    ref, refabs = oracle.gemm_rowgroup(oracle.FMT_NVFP4, ac, as_, ag, None, off, H_Q, I_Q, bc, bs, bg, rows=rows)
    got = synth.f32_from_bf16_bits(host(y)[rows])
    assert_gemm_close(got, ref, refabs, bf16=True)


def test_qwen3_nvfp4_4bit_dgrad_sampled_rows(qwen3):
    # dX = dH13 W13_e with W13 requantized (SR) per expert on the device, as the 4-bit backward step does
    off, _ = qwen3
    R = int(off[-1])
    w13 = bits(synth.device_weights(SEED + 24, E_Q, N13_Q, H_Q, device=DEV))
    wc, ws, wg = oracle.quantize_nvfp4(w13, rows_per_scale=N13_Q)
    del w13
    bct, bst, bgt = ops.requant_transpose_sr_batched(to_dev(wc), to_dev(ws), to_dev(wg), E_Q, N13_Q, seed=2, sr=True)
    rct, rst, rgt = oracle.requant_transpose_sr_batched(wc, ws, wg, E_Q, N13_Q, seed=2, use_sr=True)
    assert_bytes_equal(host(bgt)[:E_Q], rgt, "W13 requant outerT")
    assert_bytes_equal(host(bst), rst, "W13 requant scalesT")
    assert_bytes_equal(host(bct), rct, "W13 requant codesT")
    del wc, ws
    dh = bits(synth.device_activations(SEED + 25, R, N13_Q, device=DEV))
    ac, as_, ag = oracle.quantize_nvfp4(dh)
    del dh
    dx = ops.moe_grouped_gemm_blockscaled(ops.FMT_NVFP4, ops.GEMM_DGRAD, to_dev(ac), to_dev(as_), bct, bst,
                                          to_dev(off), H_Q, N13_Q, a_outer=to_dev(ag), b_outer=bgt,
                                          out_dtype=torch.bfloat16)
    rows = sample_rows(off, 48, 4)
    ref, refabs = oracle.gemm_rowgroup(oracle.FMT_NVFP4, ac, as_, ag, None, off, H_Q, N13_Q, rct, rst, rgt, rows=rows)
    got = synth.f32_from_bf16_bits(host(dx)[rows])
    assert_gemm_close(got, ref, refabs, bf16=True)


def test_qwen3_nvfp4_4bit_wgrad_sampled_groups(qwen3):
    # dW13_e = dH13_e^T X_e, both grouped-requantized (SR) on the device, X through the routing map
    off, src = qwen3
    R = int(off[-1])
    G = E_Q
    dh = bits(synth.device_activations(SEED + 26, R, N13_Q, device=DEV))
    x = bits(synth.device_activations(SEED + 27, T_Q, H_Q, device=DEV))
    dc, ds, dg = oracle.quantize_nvfp4(dh)
    xc, xs, xg = oracle.quantize_nvfp4(x, mode46=True)
    del dh, x
    ld = ops.mxfp8_grouped_cols(R, G)
    offd = to_dev(off)
    a = ops.requant_transpose_sr_grouped(to_dev(dc), to_dev(ds), to_dev(dg), offd, R, ldT=ld, seed=5, sr=True)
    b = ops.requant_transpose_sr_grouped(to_dev(xc), to_dev(xs), to_dev(xg), offd, R, ldT=ld, gather=to_dev(src),
                                         seed=6, sr=True)
    ra = oracle.requant_transpose_sr_grouped(dc, ds, dg, None, off, ld, seed=5, use_sr=True)
    rb = oracle.requant_transpose_sr_grouped(xc, xs, xg, src, off, ld, seed=6, use_sr=True)
    for got, ref, what in zip(a + b, ra + rb, ("dH13 codesT", "dH13 scalesT", "dH13 outerT", "X codesT",
                                               "X scalesT", "X outerT")):
        assert_bytes_equal(host(got)[:ref.shape[0]], ref, what)
    dw = ops.moe_grouped_gemm_blockscaled(ops.FMT_NVFP4, ops.GEMM_WGRAD, a[0], a[1], b[0], b[1], offd, H_Q, ld,
                                          M=N13_Q, a_outer=a[2], b_outer=b[2], out_dtype=torch.bfloat16)
    counts = np.diff(off)
    groups = sorted({int(np.argmax(counts)), int(np.argmin(counts)), 0, G - 1})
    rng = np.random.default_rng(7)
    sel = np.array([[g, m] for g in groups
                    for m in np.unique(np.concatenate([rng.integers(0, N13_Q, 5), [0, N13_Q - 1]]))], np.int64)
    ref, refabs = oracle.gemm_wgrad_nvfp4(ra[0], ra[1], ra[2], rb[0], rb[1], rb[2], off, sel)
    dwh = host(dw)
    got = synth.f32_from_bf16_bits(np.stack([dwh[g, m] for g, m in sel]))
    assert_gemm_close(got, ref, refabs, bf16=True)
