"""GPU parity of the block-scaled grouped GEMM with the binary64 oracle on
identical quantized operands (made by the oracle), through the C ABI.

Bound: max |C - R| / sum_k |A B| <= 1e-3 and max |C - R| / max |R| <= 1e-3
(f32 output); bf16 output adds its own 2^-9 relative rounding.  Cases cover
ragged and empty groups, gathers, N and K tails, all three modes, and the
full Qwen3-shaped (NVFP4) and DeepSeek-V3-shaped (MXFP8) workloads on sampled
rows.
"""
import functools

import numpy as np
import pytest
import torch

import oracle
from block_scaled_precision_token_amd import ops, synth
from tests.gpu_util import DEV, assert_bytes_equal, assert_gemm_close, host, to_dev


_GEMM = ops.moe_grouped_gemm_blockscaled


@pytest.fixture(params=["auto", "128", "256"], autouse=True)
def gemm_tile(request, monkeypatch):
    """Run every GEMM case with the library's tile choice and with each tile
    edge pinned through the tiled entry point (tile = 128 or 256)."""
    if request.param != "auto":
        monkeypatch.setattr(ops, "moe_grouped_gemm_blockscaled", functools.partial(_GEMM, tile=int(request.param)))
    return request.param

pytestmark = pytest.mark.gpu


def offsets(counts):
    off = np.zeros(len(counts) + 1, np.int64)
    np.cumsum(counts, out=off[1:])
    return off


CASES = [
    # (tokens, K, N, group sizes of the gathered rows)
    (40, 64, 96, [10, 0, 1, 29, 40]),
    (200, 160, 130, [129, 0, 128, 1, 142]),
    (64, 96, 64, [64, 64]),
    (40, 32, 96, [3, 37]),
    (300, 2048, 256, [300, 37, 5, 258]),
]


def make_rows(T, counts, seed):
    rng = np.random.default_rng(seed)
    off = offsets(counts)
    src = rng.integers(0, T, int(off[-1])).astype(np.int32)
    return off, src


@pytest.mark.parametrize("T,K,N,counts", CASES)
@pytest.mark.parametrize("out_dtype", [torch.float32, torch.bfloat16])
def test_nvfp4_fprop_gather(T, K, N, counts, out_dtype):
    G = len(counts)
    off, src = make_rows(T, counts, T + K)
    x = synth.activations(K + 1, T, K)
    w = synth.weights(K + 2, G, N, K)
    ac, as_, ag = oracle.quantize_nvfp4(x, mode46=True)
    bc, bs, bg = oracle.quantize_nvfp4(w, rows_per_scale=N)
    c = ops.moe_grouped_gemm_blockscaled(ops.FMT_NVFP4, ops.GEMM_FPROP, to_dev(ac), to_dev(as_), to_dev(bc),
                                         to_dev(bs), to_dev(off), N, K, a_outer=to_dev(ag), b_outer=to_dev(bg),
                                         a_gather=to_dev(src), out_dtype=out_dtype)
    ref, refabs = oracle.gemm_rowgroup(oracle.FMT_NVFP4, ac, as_, ag, src, off, N, K, bc, bs, bg)
    got = host(c.float())
    assert_gemm_close(got, ref, refabs, bf16=out_dtype == torch.bfloat16)


@pytest.mark.parametrize("T,K,N,counts", CASES)
def test_mxfp8_fprop_gather(T, K, N, counts):
    if K % 32:
        pytest.skip("MXFP8 needs K % 32 == 0")
    G = len(counts)
    off, src = make_rows(T, counts, T + 3 * K)
    x = synth.activations(K + 5, T, K)
    w = synth.weights(K + 6, G, N, K)
    ac, as_ = oracle.quantize_mxfp8_rowwise(x)
    bc, bs = oracle.quantize_mxfp8_rowwise(w)
    c = ops.moe_grouped_gemm_blockscaled(ops.FMT_MXFP8, ops.GEMM_FPROP, to_dev(ac), to_dev(as_), to_dev(bc),
                                         to_dev(bs), to_dev(off), N, K, a_gather=to_dev(src))
    ref, refabs = oracle.gemm_rowgroup(oracle.FMT_MXFP8, ac, as_, None, src, off, N, K, bc, bs, None)
    assert_gemm_close(host(c), ref, refabs)


def test_mxfp8_dgrad_uses_columnwise_weight_copy():
    # dX = dY W: W_e [N, K] stored rowwise along K; its columnwise copy [K, N]
    # has blocks along N, the reduction dim of dgrad.
    G, N, Kf, R = 3, 96, 128, 150
    counts = [50, 64, 36]
    off = offsets(counts)
    w = synth.weights(41, G, N, Kf)
    dy = synth.activations(42, R, N)
    dyc, dys = oracle.quantize_mxfp8_rowwise(dy)
    wtc = np.zeros((G, Kf, N), np.uint8)
    wts = np.zeros((G, Kf, N // 32), np.uint8)
    for e in range(G):
        wtc[e], wts[e] = oracle.quantize_mxfp8_colwise(w[e * N:(e + 1) * N])
    c = ops.moe_grouped_gemm_blockscaled(ops.FMT_MXFP8, ops.GEMM_DGRAD, to_dev(dyc), to_dev(dys),
                                         to_dev(wtc.reshape(G * Kf, N)), to_dev(wts.reshape(G * Kf, N // 32)),
                                         to_dev(off), Kf, N)
    ref, refabs = oracle.gemm_rowgroup(oracle.FMT_MXFP8, dyc, dys, None, None, off, Kf, N,
                                       wtc.reshape(G * Kf, N), wts.reshape(G * Kf, N // 32), None)
    assert_gemm_close(host(c), ref, refabs)


@pytest.mark.parametrize("counts", [[50, 0, 64, 1, 100], [33, 200]])
@pytest.mark.parametrize("out_dtype", [torch.float32, torch.bfloat16])
def test_mxfp8_wgrad_grouped_columnwise(counts, out_dtype):
    # dW_e = dY_e^T h_e over the tokens of group e, from grouped columnwise copies
    off = offsets(counts)
    R = int(off[-1])
    NA, NB = 160, 96
    G = len(counts)
    dy = synth.activations(51, R, NA)
    h = synth.activations(52, R, NB)
    ld = ops.mxfp8_grouped_cols(R, G)
    ac, as_ = oracle.quantize_mxfp8_colwise(dy, off, ldT=ld)
    bc, bs = oracle.quantize_mxfp8_colwise(h, off, ldT=ld)
    c = ops.moe_grouped_gemm_blockscaled(ops.FMT_MXFP8, ops.GEMM_WGRAD, to_dev(ac), to_dev(as_), to_dev(bc),
                                         to_dev(bs), to_dev(off), NB, ld, M=NA, out_dtype=out_dtype)
    sel = np.array([[g, n] for g in range(G) for n in range(NA)], np.int64)
    ref, refabs = oracle.gemm_wgrad(ac, as_, bc, bs, off, sel)
    got = host(c.float()).reshape(G * NA, NB)
    assert_gemm_close(got, ref, refabs, bf16=out_dtype == torch.bfloat16)


def test_wgrad_from_device_grouped_quantizer():
    # the weight-gradient GEMM consuming columnwise copies made on the device
    counts = [70, 3, 0, 90]
    off = offsets(counts)
    R = int(off[-1])
    dy = synth.activations(61, R, 128)
    h = synth.activations(62, R, 64)
    offd = to_dev(off)
    from tests.gpu_util import to_dev_bf16
    qa = ops.quantize_mxfp8(to_dev_bf16(dy), rowwise=False, colwise=True, group_offsets=offd)
    qb = ops.quantize_mxfp8(to_dev_bf16(h), rowwise=False, colwise=True, group_offsets=offd)
    ld = qa["codes_colT"].shape[1]
    c = ops.moe_grouped_gemm_blockscaled(ops.FMT_MXFP8, ops.GEMM_WGRAD, qa["codes_colT"], qa["scales_colT"],
                                         qb["codes_colT"], qb["scales_colT"], offd, 64, ld, M=128)
    ac, as_ = oracle.quantize_mxfp8_colwise(dy, off, ldT=ld)
    bc, bs = oracle.quantize_mxfp8_colwise(h, off, ldT=ld)
    sel = np.array([[g, n] for g in range(4) for n in range(128)], np.int64)
    ref, refabs = oracle.gemm_wgrad(ac, as_, bc, bs, off, sel)
    assert_gemm_close(host(c).reshape(4 * 128, 64), ref, refabs)


def test_qwen3_shaped_nvfp4_gate_up_sampled_rows():
    # 8192 tokens, top-8 of 128 experts (Zipf load), hidden 2048 -> gate/up 1536
    T, E, k, H, N = 8192, 128, 8, 2048, 1536
    off, src = synth.route_topk(20261205, T, E, k, synth.zipf_bias(20261204, E))
    x = synth.activations(20261206, T, H)
    ac, as_, ag = oracle.quantize_nvfp4(x, mode46=True)
    # weights on the device (tensor of 128 x 1536 x 2048), quantized by the oracle per expert
    w = synth.weights(20261207, E, N, H)
    bc, bs, bg = oracle.quantize_nvfp4(w, rows_per_scale=N)
    del w
    c = ops.moe_grouped_gemm_blockscaled(ops.FMT_NVFP4, ops.GEMM_FPROP, to_dev(ac), to_dev(as_), to_dev(bc),
                                         to_dev(bs), to_dev(off), N, H, a_outer=to_dev(ag), b_outer=to_dev(bg),
                                         a_gather=to_dev(src))
    rng = np.random.default_rng(0)
    counts = np.diff(off)
    big = int(np.argmax(counts))
    rows = np.unique(np.concatenate([rng.integers(0, off[-1], 48), [0, off[-1] - 1, off[big], off[big + 1] - 1]]))
    ref, refabs = oracle.gemm_rowgroup(oracle.FMT_NVFP4, ac, as_, ag, src, off, N, H, bc, bs, bg, rows=rows)
    got = host(c)[rows]
    assert_gemm_close(got, ref, refabs)


@pytest.mark.parametrize("sr", [True, False])
def test_nvfp4_dgrad_on_requantized_weights(sr):
    # The 4-bit backward's data gradient: dX = dY W_e with the forward's NVFP4
    # weight copy W_e [N, Kf] dequantized, transposed and requantized on the
    # device (16-blocks along N, the reduction dim of dgrad; per-expert G_e).
    G, N, Kf = 3, 96, 160
    counts = [50, 0, 77]
    off = offsets(counts)
    R = int(off[-1])
    w = synth.weights(43, G, N, Kf)
    wc, ws, wg = oracle.quantize_nvfp4(w, rows_per_scale=N)
    bct, bst, bgt = ops.requant_transpose_sr_batched(to_dev(wc), to_dev(ws), to_dev(wg), G, N, seed=99, sr=sr)
    rct, rst, rgt = oracle.requant_transpose_sr_batched(wc, ws, wg, G, N, seed=99, use_sr=sr)
    np.testing.assert_array_equal(host(bct), rct)
    dy = synth.activations(44, R, N)
    ac, as_, ag = oracle.quantize_nvfp4(dy)
    c = ops.moe_grouped_gemm_blockscaled(ops.FMT_NVFP4, ops.GEMM_DGRAD, to_dev(ac), to_dev(as_), bct, bst,
                                         to_dev(off), Kf, N, a_outer=to_dev(ag), b_outer=bgt)
    ref, refabs = oracle.gemm_rowgroup(oracle.FMT_NVFP4, ac, as_, ag, None, off, Kf, N, rct, rst, rgt)
    assert_gemm_close(host(c), ref, refabs)


@pytest.mark.parametrize("counts", [[50, 0, 64, 1, 100], [33, 200, 7]])
@pytest.mark.parametrize("sr", [True, False])
def test_nvfp4_wgrad_on_grouped_requantized_operands(counts, sr):
    # The 4-bit backward's weight gradient: dW_e = dY_e^T X_e, both operands
    # requantized on the device from rowwise per-token NVFP4 into token-blocked
    # grouped copies (X through the routing map), one outer scale per group.
    G = len(counts)
    off = offsets(counts)
    R = int(off[-1])
    T, NA, NB = 90, 160, 96
    rng = np.random.default_rng(R)
    src = rng.integers(0, T, R).astype(np.int32)
    dy = synth.activations(53, R, NA)
    x = synth.activations(54, T, NB)
    dyc, dys, dyg = oracle.quantize_nvfp4(dy)
    xc, xs, xg = oracle.quantize_nvfp4(x, mode46=True)
    ld = ops.mxfp8_grouped_cols(R, G)
    offd = to_dev(off)
    a = ops.requant_transpose_sr_grouped(to_dev(dyc), to_dev(dys), to_dev(dyg), offd, R, ldT=ld, seed=3, sr=sr)
    b = ops.requant_transpose_sr_grouped(to_dev(xc), to_dev(xs), to_dev(xg), offd, R, ldT=ld, gather=to_dev(src),
                                         seed=4, sr=sr)
    ra = oracle.requant_transpose_sr_grouped(dyc, dys, dyg, None, off, ld, seed=3, use_sr=sr)
    rb = oracle.requant_transpose_sr_grouped(xc, xs, xg, src, off, ld, seed=4, use_sr=sr)
    for got, ref in zip(a + b, ra + rb):
        np.testing.assert_array_equal(host(got)[:ref.shape[0]], ref)
    c = ops.moe_grouped_gemm_blockscaled(ops.FMT_NVFP4, ops.GEMM_WGRAD, a[0], a[1], b[0], b[1], offd, NB, ld, M=NA,
                                         a_outer=a[2], b_outer=b[2])
    sel = np.array([[g, n] for g in range(G) for n in range(NA)], np.int64)
    ref, refabs = oracle.gemm_wgrad_nvfp4(ra[0], ra[1], ra[2], rb[0], rb[1], rb[2], off, sel)
    assert_gemm_close(host(c).reshape(G * NA, NB), ref, refabs)


# --- the DeepSeek-V3-shaped MXFP8 GEMMs at full size, sampled ---------------
# 4096 tokens, hidden 7168, expert intermediate 2048, top-8 of 256 routed
# experts plus one shared expert (36,864 rows), as in the timed step.  The
# weights (7.5 G values per projection) are generated and quantized on the
# device with the step's own calls; the sampled experts' device codes and
# scales are first checked byte for byte against the oracle's quantization of
# the same bf16 values, and only rows (or weight-gradient groups) of those
# experts are checked, so every checked output depends on operands the oracle
# has confirmed.

T_D, H_D, I_D, E_D, TOPK_D = 4096, 7168, 2048, 256, 8
N13_D = 2 * I_D


@pytest.fixture(scope="module")
def dsv3_routing():
    off, src = synth.route_topk(20261210, T_D, E_D, TOPK_D, synth.zipf_bias(20261209, E_D, 1.1, uniform_mix=0.5),
                                shared_expert=True)
    counts = np.diff(off)
    rng = np.random.default_rng(20261211)
    sampled = sorted({int(np.argmax(counts[:-1])), int(np.argmin(counts[:-1])), E_D,
                      *rng.integers(0, E_D, 2).tolist()})
    rows = {}
    for e in sampled:
        lo, hi = int(off[e]), int(off[e + 1])
        rows[e] = np.unique(np.concatenate([[lo, hi - 1], rng.integers(lo, hi, 3)]))
    return off, src, sampled, rows


def host_bits(t):
    return t.view(torch.int16).cpu().numpy().view(np.uint16)


def test_dsv3_shaped_mxfp8_gate_up_sampled(dsv3_routing, gemm_tile):
    if gemm_tile != "auto":
        pytest.skip("full size: the library's tile choice only (the one bench.py times)")
    off, src, sampled, rows = dsv3_routing
    G, R = E_D + 1, int(off[-1])
    x = synth.activations(20261212, T_D, H_D)
    ac, as_ = oracle.quantize_mxfp8_rowwise(x)
    w13 = synth.device_weights(20261213, G, N13_D, H_D, device=DEV)
    wq = ops.quantize_mxfp8(w13.view(G, N13_D, H_D), True, True)
    bc, bs = {}, {}
    for e in sampled:
        bc[e], bs[e] = oracle.quantize_mxfp8_rowwise(host_bits(w13[e * N13_D:(e + 1) * N13_D]))
        assert_bytes_equal(host(wq["codes_row"][e]), bc[e], f"W13 expert {e} row codes")
        assert_bytes_equal(host(wq["scales_row"][e]), bs[e], f"W13 expert {e} row scales")
    del w13
    h13 = ops.moe_grouped_gemm_blockscaled(ops.FMT_MXFP8, ops.GEMM_FPROP, to_dev(ac), to_dev(as_),
                                           wq["codes_row"], wq["scales_row"], to_dev(off), N13_D, H_D, M=R,
                                           a_gather=to_dev(src), out_dtype=torch.bfloat16)
    got = host(h13.float())
    for e in sampled:
        sel = rows[e]
        ref, refabs = oracle.gemm_rowgroup(oracle.FMT_MXFP8, ac, as_, None, src[sel], np.array([0, sel.size]),
                                           N13_D, H_D, bc[e], bs[e], None)
        assert_gemm_close(got[sel], ref, refabs, bf16=True)


def test_dsv3_shaped_mxfp8_dgrad_gate_up_sampled(dsv3_routing, gemm_tile):
    if gemm_tile != "auto":
        pytest.skip("full size: the library's tile choice only (the one bench.py times)")
    # dX = dH13 W13_e through W13's columnwise copy [H, 2I] per expert
    off, src, sampled, rows = dsv3_routing
    G, R = E_D + 1, int(off[-1])
    dh = synth.device_activations(20261214, R, N13_D, device=DEV)
    dq = ops.quantize_mxfp8(dh, True, True, group_offsets=to_dev(off))
    w13 = synth.device_weights(20261215, G, N13_D, H_D, device=DEV)
    wq = ops.quantize_mxfp8(w13.view(G, N13_D, H_D), True, True)
    bc, bs, ac, as_ = {}, {}, {}, {}
    for e in sampled:
        bc[e], bs[e] = oracle.quantize_mxfp8_colwise(host_bits(w13[e * N13_D:(e + 1) * N13_D]))
        assert_bytes_equal(host(wq["codes_colT"][e]), bc[e], f"W13 expert {e} col codes")
        assert_bytes_equal(host(wq["scales_colT"][e]), bs[e], f"W13 expert {e} col scales")
        sel = torch.from_numpy(rows[e]).to(DEV)
        ac[e], as_[e] = oracle.quantize_mxfp8_rowwise(host_bits(dh[sel]))
        assert_bytes_equal(host(dq["codes_row"][sel]), ac[e], f"dH13 rows of expert {e}")
        assert_bytes_equal(host(dq["scales_row"][sel]), as_[e], f"dH13 row scales of expert {e}")
    del w13, dh
    dx = ops.moe_grouped_gemm_blockscaled(ops.FMT_MXFP8, ops.GEMM_DGRAD, dq["codes_row"], dq["scales_row"],
                                          wq["codes_colT"], wq["scales_colT"], to_dev(off), H_D, N13_D, M=R,
                                          out_dtype=torch.bfloat16)
    got = host(dx.float())
    for e in sampled:
        ref, refabs = oracle.gemm_rowgroup(oracle.FMT_MXFP8, ac[e], as_[e], None, None,
                                           np.array([0, rows[e].size]), H_D, N13_D, bc[e], bs[e], None)
        assert_gemm_close(got[rows[e]], ref, refabs, bf16=True)


def test_dsv3_shaped_mxfp8_wgrad_gate_up_sampled(dsv3_routing, gemm_tile):
    if gemm_tile != "auto":
        pytest.skip("full size: the library's tile choice only (the one bench.py times)")
    # dW13_e = dH13_e^T X_e over the routed rows of expert e, both operands in
    # their grouped columnwise copies (X read through the routing map)
    off, src, sampled, rows = dsv3_routing
    G, R = E_D + 1, int(off[-1])
    offd = to_dev(off)
    dh = synth.device_activations(20261216, R, N13_D, device=DEV)
    x = synth.device_activations(20261217, T_D, H_D, device=DEV)
    qa = ops.quantize_mxfp8(dh, True, True, group_offsets=offd)
    qb = ops.quantize_mxfp8(x, False, True, group_offsets=offd, row_gather=to_dev(src))
    P = oracle.padded_offsets(off)
    ref_ops = {}
    for e in sampled:
        lo, hi = int(off[e]), int(off[e + 1])
        one = np.array([0, hi - lo], np.int64)   # one group: padded to 32 rows like the grouped copies
        a_e = oracle.quantize_mxfp8_colwise(host_bits(dh[lo:hi]), one)
        b_e = oracle.quantize_mxfp8_colwise(host_bits(x[torch.from_numpy(src[lo:hi].astype(np.int64)).to(DEV)]), one)
        w = a_e[0].shape[1]                      # the group's 32-padded width
        assert_bytes_equal(host(qa["codes_colT"][:, P[e]:P[e] + w]), a_e[0], f"dH13 group {e} col codes")
        assert_bytes_equal(host(qa["scales_colT"][:, P[e] // 32:(P[e] + w) // 32]), a_e[1], f"dH13 group {e} scales")
        assert_bytes_equal(host(qb["codes_colT"][:, P[e]:P[e] + w]), b_e[0], f"X group {e} col codes")
        assert_bytes_equal(host(qb["scales_colT"][:, P[e] // 32:(P[e] + w) // 32]), b_e[1], f"X group {e} scales")
        ref_ops[e] = (a_e, b_e, hi - lo)
    del dh, x
    ld = qa["codes_colT"].shape[1]
    dw = ops.moe_grouped_gemm_blockscaled(ops.FMT_MXFP8, ops.GEMM_WGRAD, qa["codes_colT"], qa["scales_colT"],
                                          qb["codes_colT"], qb["scales_colT"], offd, H_D, ld, M=N13_D,
                                          out_dtype=torch.bfloat16)
    rng = np.random.default_rng(20261218)
    for e in sampled:
        (ac, as_), (bc, bs), n = ref_ops[e]
        ms = np.unique(np.concatenate([[0, N13_D - 1], rng.integers(0, N13_D, 4)]))
        sel = np.stack([np.zeros_like(ms), ms], 1)
        ref, refabs = oracle.gemm_wgrad(ac, as_, bc, bs, np.array([0, n]), sel)
        assert_gemm_close(host(dw[e].float())[ms], ref, refabs, bf16=True)
