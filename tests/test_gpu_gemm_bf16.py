"""GPU parity of the BF16 grouped GEMM -- the backward GEMMs of the NVFP4 MoE
layer in either mode (original or dequantized operands) -- with the binary64
oracle on identical bf16 operands, through the C ABI.

Bound as for the block-scaled GEMM: max |C - R| / sum_k |A B| <= 1e-3 and
max |C - R| / max |R| <= 1e-3 (f32 output; bf16 output adds its own 2^-9
relative rounding).  Cases cover ragged and empty groups, gathers with
out-of-range entries, N, M and K tails (K a multiple of 8 but not of the
32-value stage), all three forms, both tile edges, and the full
Qwen3-30B-A3B-shaped backward GEMMs on sampled rows.
"""
import functools

import numpy as np
import pytest
import torch

import oracle
from block_scaled_precision_token_amd import ops, synth
from tests.gpu_util import DEV, assert_gemm_close, host, to_dev, to_dev_bf16

pytestmark = pytest.mark.gpu


_GEMM = ops.moe_grouped_gemm_bf16


@pytest.fixture(params=["auto", "128", "256"], autouse=True)
def gemm_tile(request, monkeypatch):
    """Every case with the library's tile choice and with each tile edge
    pinned through the tiled entry point."""
    if request.param != "auto":
        monkeypatch.setattr(ops, "moe_grouped_gemm_bf16", functools.partial(_GEMM, tile=int(request.param)))
    return request.param


def offsets(counts):
    off = np.zeros(len(counts) + 1, np.int64)
    np.cumsum(counts, out=off[1:])
    return off


def gathered_rows(T, counts, seed, bad=True):
    rng = np.random.default_rng(seed)
    off = offsets(counts)
    src = rng.integers(0, T, int(off[-1])).astype(np.int32)
    if bad and src.size > 8:
        src[1] = -1          # out-of-range indices read as zero rows
        src[src.size // 2] = T
    return off, src


ROW_CASES = [
    # (source rows, K, N, rows of C per group)
    (40, 64, 96, [10, 0, 1, 29, 40]),
    (200, 200, 136, [129, 0, 128, 1, 142]),     # K = 6 stages + 8, N tail
    (64, 96, 64, [64, 64]),
    (40, 8, 96, [3, 37]),                       # a single partial stage
    (300, 2056, 264, [300, 37, 5, 258]),
]


@pytest.mark.parametrize("T,K,N,counts", ROW_CASES)
@pytest.mark.parametrize("out_dtype", [torch.float32, torch.bfloat16])
def test_bf16_fprop_gather(T, K, N, counts, out_dtype):
    G = len(counts)
    off, src = gathered_rows(T, counts, T + K)
    x = synth.activations(K + 11, T, K)
    w = synth.weights(K + 12, G, N, K)                       # [G * N, K]
    c = ops.moe_grouped_gemm_bf16(ops.GEMM_FPROP, to_dev_bf16(x), to_dev_bf16(w), to_dev(off), N, K,
                                  gather=to_dev(src), out_dtype=out_dtype)
    ref, refabs = oracle.gemm_bf16_rowgroup(oracle.GEMM_FPROP, x, w, src, off, N, K)
    assert_gemm_close(host(c.float()), ref, refabs, bf16=out_dtype == torch.bfloat16)


@pytest.mark.parametrize("T,K,N,counts", ROW_CASES)
@pytest.mark.parametrize("gather", [True, False])
def test_bf16_dgrad_takes_weight_as_stored(T, K, N, counts, gather):
    # dX = dY W_e with W_e [K, N] as the forward stores it (out x in)
    G = len(counts)
    off, src = gathered_rows(T, counts, T + 2 * K)
    R = int(off[-1])
    dy = synth.activations(K + 13, T if gather else R, K)
    w = synth.weights(K + 14, G, K, N)                       # [G * K, N]
    c = ops.moe_grouped_gemm_bf16(ops.GEMM_DGRAD, to_dev_bf16(dy), to_dev_bf16(w), to_dev(off), N, K,
                                  gather=to_dev(src) if gather else None)
    ref, refabs = oracle.gemm_bf16_rowgroup(oracle.GEMM_DGRAD, dy, w, src if gather else None, off, N, K)
    assert_gemm_close(host(c), ref, refabs)


WG_CASES = [
    # (M, N, source rows of B, rows per group)
    (64, 96, 50, [10, 0, 33, 57]),
    (136, 264, 300, [300, 1, 0, 31, 258]),
    (256, 512, 128, [64, 64]),
    (24, 40, 20, [5]),
    (96, 64, 40, [0, 0]),                       # no rows at all: C is zero
]


@pytest.mark.parametrize("M,N,T,counts", WG_CASES)
@pytest.mark.parametrize("out_dtype", [torch.float32, torch.bfloat16])
def test_bf16_wgrad_gather(M, N, T, counts, out_dtype):
    # dW_e = dY_e^T X[src] over the rows of group e, X read through the gather
    G = len(counts)
    off, src = gathered_rows(T, counts, M + N)
    R = max(int(off[-1]), 1)
    dy = synth.activations(M + 15, R, M)
    x = synth.activations(N + 16, T, N)
    srcd = to_dev(src) if src.size else to_dev(np.zeros(1, np.int32))
    c = ops.moe_grouped_gemm_bf16(ops.GEMM_WGRAD, to_dev_bf16(dy), to_dev_bf16(x), to_dev(off), N, R,
                                  gather=srcd, out_dtype=out_dtype)
    sel = np.array([[g, m] for g in range(G) for m in range(M)], np.int64)
    ref, refabs = oracle.gemm_bf16_wgrad(dy, x, src if src.size else None, off, sel)
    got = host(c.float()).reshape(G * M, N)
    assert_gemm_close(got, ref, refabs, bf16=out_dtype == torch.bfloat16)


def test_bf16_wgrad_without_gather():
    counts = [70, 3, 0, 90]
    off = offsets(counts)
    R = int(off[-1])
    M, N = 128, 72
    dy = synth.activations(71, R, M)
    h = synth.activations(72, R, N)
    c = ops.moe_grouped_gemm_bf16(ops.GEMM_WGRAD, to_dev_bf16(dy), to_dev_bf16(h), to_dev(off), N, R)
    sel = np.array([[g, m] for g in range(4) for m in range(M)], np.int64)
    ref, refabs = oracle.gemm_bf16_wgrad(dy, h, None, off, sel)
    assert_gemm_close(host(c).reshape(4 * M, N), ref, refabs)
    assert not host(c)[2].any()                              # the empty group's gradient is zero


def test_bf16_leading_dimensions_and_ldc():
    # operands and output inside wider buffers (lda, ldb, ldc > the logical width)
    counts = [40, 24]
    off = offsets(counts)
    R, K, N = 64, 72, 40
    x = synth.activations(81, R, K + 24)
    w = synth.weights(82, 2, K, N + 8)
    out = torch.full((R, N + 24), 7.0, dtype=torch.float32, device=DEV)
    ops.moe_grouped_gemm_bf16(ops.GEMM_DGRAD, to_dev_bf16(x)[:, :K], to_dev_bf16(w), to_dev(off), N, K, out=out)
    xs = np.ascontiguousarray(x[:, :K])
    ws = np.ascontiguousarray(w.reshape(2, K, N + 8)[:, :, :N]).reshape(2 * K, N)
    ref, refabs = oracle.gemm_bf16_rowgroup(oracle.GEMM_DGRAD, xs, ws, None, off, N, K)
    got = host(out)
    assert_gemm_close(got[:, :N], ref, refabs)
    assert np.all(got[:, N:] == 7.0)                         # columns past N untouched


# --- the Qwen3-30B-A3B-shaped backward GEMMs at full size, sampled -----------

T_Q, E_Q, TOPK_Q, H_Q, I_Q = 8192, 128, 8, 2048, 768


def _qwen3_routing():
    return synth.route_topk(20261205, T_Q, E_Q, TOPK_Q, synth.zipf_bias(20261204, E_Q))


def _sample_rows(off, n, seed):
    rng = np.random.default_rng(seed)
    big = int(np.argmax(np.diff(off)))
    return np.unique(np.concatenate([rng.integers(0, off[-1], n), [0, off[-1] - 1, off[big], off[big + 1] - 1]]))


def test_qwen3_shaped_dgrad_sampled_rows():
    # dX_routed = dH13 W13_e: [65536, 1536] x W13_e [1536, 2048] -> [65536, 2048]
    off, src = _qwen3_routing()
    R = int(off[-1])
    dh = synth.device_activations(20261301, R, 2 * I_Q, device=DEV)
    w13 = synth.device_weights(20261302, E_Q, 2 * I_Q, H_Q, device=DEV)
    c = ops.moe_grouped_gemm_bf16(ops.GEMM_DGRAD, dh, w13, to_dev(off), H_Q, 2 * I_Q)
    rows = _sample_rows(off, 40, 1)
    got = host(c)[rows]
    dh_h = host(dh)
    for e in np.unique(np.searchsorted(off, rows, side="right") - 1):
        sel = rows[(rows >= off[e]) & (rows < off[e + 1])]
        w_e = host(w13[e * 2 * I_Q:(e + 1) * 2 * I_Q])
        ref, refabs = oracle.gemm_bf16_rowgroup(oracle.GEMM_DGRAD, dh_h[sel], w_e, None,
                                                np.array([0, sel.size]), H_Q, 2 * I_Q)
        assert_gemm_close(got[np.isin(rows, sel)], ref, refabs)


def test_qwen3_shaped_wgrad_sampled_groups():
    # dW13_e = dH13_e^T X[src]: 128 experts x [1536, 2048], X gathered through the routing map
    off, src = _qwen3_routing()
    R = int(off[-1])
    dh = synth.device_activations(20261303, R, 2 * I_Q, device=DEV)
    x = synth.device_activations(20261304, T_Q, H_Q, device=DEV)
    c = ops.moe_grouped_gemm_bf16(ops.GEMM_WGRAD, dh, x, to_dev(off), H_Q, R, gather=to_dev(src),
                                  out_dtype=torch.bfloat16)
    counts = np.diff(off)
    groups = sorted({int(np.argmax(counts)), int(np.argmin(counts)), 0, E_Q - 1})
    x_h = host(x)
    dh_h = host(dh)
    rng = np.random.default_rng(2)
    for g in groups:
        ms = np.unique(np.concatenate([rng.integers(0, 2 * I_Q, 6), [0, 2 * I_Q - 1]]))
        lo, hi = int(off[g]), int(off[g + 1])
        sel = np.stack([np.zeros_like(ms), ms], 1)
        ref, refabs = oracle.gemm_bf16_wgrad(dh_h[lo:hi], x_h, src[lo:hi], np.array([0, hi - lo]), sel)
        got = host(c[g]).view(np.uint16)[ms]
        got = synth.f32_from_bf16_bits(got)
        assert_gemm_close(got, ref, refabs, bf16=True)
