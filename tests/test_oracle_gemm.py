"""Pins of the oracle's grouped GEMM reference and SwiGLU.

GEMM: numpy float64 matmul (a library routine) on operands decoded
independently (the pages' E2M1 value set, torch's float8 and bfloat16
decodes), and identity-weight cases whose result is known in closed form.
SwiGLU: the explicit f32 exp against numpy's exp (within 2 ulp), the silu
formula in float64, and exact special values.
"""
import numpy as np
import torch

import oracle
from block_scaled_precision_token_amd import synth
from tests.conftest import read_golden

E2M1 = np.array([float(v) for v in read_golden("e2m1_value_set.txt")["values"].split()])


def e4m3_vals(codes):
    return torch.from_numpy(np.ascontiguousarray(codes, np.uint8)).view(torch.float8_e4m3fn).double().numpy()


def nvfp4_exact(codes, scales, outer, rows_per_scale=1):
    M, K = codes.shape[0], codes.shape[1] * 2
    q = np.empty((M, K), np.uint8)
    q[:, 0::2] = codes & 15
    q[:, 1::2] = codes >> 4
    v = np.where(q & 8, -E2M1[q & 7], E2M1[q & 7])
    s = e4m3_vals(scales.reshape(-1)).reshape(M, K // 16).repeat(16, axis=1)
    g = np.repeat(outer.astype(np.float64), rows_per_scale)[:, None]
    return v * s * g


def mxfp8_exact(codes, scales):
    M, K = codes.shape
    v = e4m3_vals(codes.reshape(-1)).reshape(M, K)
    return v * np.exp2(scales.astype(np.float64) - 127).repeat(32, axis=1)


def routing(T, E, k, seed):
    bias = synth.zipf_bias(seed, E)
    return synth.route_topk(seed + 1, T, E, k, bias)


def test_nvfp4_fprop_with_gather_matches_float64_matmul():
    T, E, k, N, K = 48, 4, 2, 40, 64
    off, src = routing(T, E, k, 3)
    x = synth.activations(4, T, K)
    w = synth.weights(5, E, N, K)
    ac, as_, ag = oracle.quantize_nvfp4(x, mode46=True)
    bc, bs, bg = oracle.quantize_nvfp4(w, rows_per_scale=N)
    c, cabs = oracle.gemm_rowgroup(oracle.FMT_NVFP4, ac, as_, ag, src, off, N, K, bc, bs, bg)
    A = nvfp4_exact(ac, as_, ag)
    B = nvfp4_exact(bc, bs, bg, rows_per_scale=N)
    for e in range(E):
        rows = np.arange(off[e], off[e + 1])
        ref = A[src[rows]] @ B[e * N:(e + 1) * N].T
        np.testing.assert_allclose(c[rows], ref, rtol=1e-12, atol=1e-12 * np.abs(ref).max())
        refabs = np.abs(A[src[rows]]) @ np.abs(B[e * N:(e + 1) * N]).T
        np.testing.assert_allclose(cabs[rows], refabs, rtol=1e-12)


def test_mxfp8_fprop_and_row_subset():
    T, E, k, N, K = 40, 3, 2, 32, 96
    off, src = routing(T, E, k, 6)
    x = synth.activations(7, T, K)
    w = synth.weights(8, E, N, K)
    ac, as_ = oracle.quantize_mxfp8_rowwise(x)
    bc, bs = oracle.quantize_mxfp8_rowwise(w)
    rows = np.array([0, 5, int(off[1]), int(off[-1]) - 1], np.int64)
    c, _ = oracle.gemm_rowgroup(oracle.FMT_MXFP8, ac, as_, None, src, off, N, K, bc, bs, None, rows=rows)
    A = mxfp8_exact(ac, as_)
    B = mxfp8_exact(bc, bs)
    for i, r in enumerate(rows):
        e = int(np.searchsorted(off, r, side="right") - 1)
        ref = B[e * N:(e + 1) * N] @ A[src[r]]
        np.testing.assert_allclose(c[i], ref, rtol=1e-12, atol=1e-12 * np.abs(ref).max())


def test_identity_weights_closed_form():
    # B_e = c_e * I with c_e an exact power of two: C = A * c_e exactly
    T, E, K = 32, 2, 64
    off = np.array([0, 20, 32], np.int64)
    x = synth.activations(9, T, K)
    ac, as_ = oracle.quantize_mxfp8_rowwise(x)
    eye = np.zeros((E * K, K), np.float32)
    for e in range(E):
        eye[e * K:(e + 1) * K] = np.eye(K, dtype=np.float32) * (2.0 ** (e - 1))
    bc, bs = oracle.quantize_mxfp8_rowwise(synth.bf16_bits_from_f32(eye))
    c, _ = oracle.gemm_rowgroup(oracle.FMT_MXFP8, ac, as_, None, None, off, K, K, bc, bs, None)
    A = mxfp8_exact(ac, as_)
    for e in range(E):
        np.testing.assert_array_equal(c[off[e]:off[e + 1]], A[off[e]:off[e + 1]] * 2.0 ** (e - 1))


def test_wgrad_matches_float64_matmul_per_group():
    T, E, k, NA, NB = 50, 4, 2, 64, 32
    off, src = routing(T, E, k, 10)
    R = int(off[-1])
    dy = synth.activations(11, R, NA)
    h = synth.activations(12, R, NB)
    ac, as_ = oracle.quantize_mxfp8_colwise(dy, off)
    bc, bs = oracle.quantize_mxfp8_colwise(h, off)
    P = oracle.padded_offsets(off)
    sel = np.array([[g, n] for g in range(E) for n in (0, 7, NA - 1)], np.int64)
    c, cabs = oracle.gemm_wgrad(ac, as_, bc, bs, off, sel)
    A = mxfp8_exact(ac, as_)
    B = mxfp8_exact(bc, bs)
    for i, (g, n) in enumerate(sel):
        ref = B[:, P[g]:P[g + 1]] @ A[n, P[g]:P[g + 1]]
        np.testing.assert_allclose(c[i], ref, rtol=1e-12, atol=1e-12 * np.abs(ref).max())
        # padded columns are zero, so the unpadded group gives the same result
        n_g = off[g + 1] - off[g]
        ref2 = B[:, P[g]:P[g] + n_g] @ A[n, P[g]:P[g] + n_g]
        np.testing.assert_allclose(c[i], ref2, rtol=1e-12, atol=1e-12 * np.abs(ref).max())


def bf16_vals(bits):
    t = torch.from_numpy(np.ascontiguousarray(bits, np.uint16).view(np.int16))
    return t.view(torch.bfloat16).double().numpy()


def test_bf16_fprop_and_dgrad_match_float64_matmul():
    T, E, k, N, K = 40, 3, 2, 24, 56
    off, src = routing(T, E, k, 13)
    x = synth.activations(14, T, K)
    w_fp = synth.weights(15, E, N, K)                        # forward-form B [E, N, K]
    w_dg = synth.weights(16, E, K, N)                        # data-gradient form B [E, K, N]
    A = bf16_vals(x)
    src = src.copy()
    src[3] = -1                                              # out-of-range gathers read as zero rows
    src[7] = T
    c0, cabs0 = oracle.gemm_bf16_rowgroup(oracle.GEMM_FPROP, x, w_fp.reshape(E * N, K), src, off, N, K)
    c1, _ = oracle.gemm_bf16_rowgroup(oracle.GEMM_DGRAD, x, w_dg.reshape(E * K, N), src, off, N, K)
    B0 = bf16_vals(w_fp.reshape(E, N, K))
    B1 = bf16_vals(w_dg.reshape(E, K, N))
    for r in range(int(off[-1])):
        e = int(np.searchsorted(off, r, side="right") - 1)
        t = src[r]
        a = A[t] if 0 <= t < T else np.zeros(K)
        ref0 = B0[e] @ a
        ref1 = a @ B1[e]
        np.testing.assert_allclose(c0[r], ref0, rtol=1e-12, atol=1e-12 * max(np.abs(ref0).max(), 1e-300))
        np.testing.assert_allclose(c1[r], ref1, rtol=1e-12, atol=1e-12 * max(np.abs(ref1).max(), 1e-300))
        np.testing.assert_allclose(cabs0[r], np.abs(B0[e]) @ np.abs(a), rtol=1e-12)
    assert not c0[3].any() and not c1[7].any()
    # the two forms agree when B_e of one is the transpose of the other's
    wt = np.ascontiguousarray(w_fp.reshape(E, N, K).transpose(0, 2, 1)).reshape(E * K, N)
    c2, _ = oracle.gemm_bf16_rowgroup(oracle.GEMM_DGRAD, x, wt, src, off, N, K, rows=np.array([0, 9, 20]))
    np.testing.assert_array_equal(c2, c0[[0, 9, 20]])


def test_bf16_wgrad_matches_float64_matmul_per_group():
    T, E, k, M, N = 30, 4, 2, 40, 24
    off, src = routing(T, E, k, 17)
    R = int(off[-1])
    dy = synth.activations(18, R, M)                         # A: group rows in routed order
    x = synth.activations(19, T, N)                          # B: gathered by the routing map
    src = src.copy()
    src[2] = -5
    sel = np.array([[g, m] for g in range(E) for m in (0, 11, M - 1)], np.int64)
    c, cabs = oracle.gemm_bf16_wgrad(dy, x, src, off, sel)
    A = bf16_vals(dy)
    X = bf16_vals(x)
    Xg = np.where((src >= 0)[:, None], X[np.clip(src, 0, T - 1)], 0.0)
    for i, (g, m) in enumerate(sel):
        rows = slice(off[g], off[g + 1])
        ref = A[rows, m] @ Xg[rows]
        np.testing.assert_allclose(c[i], ref, rtol=1e-12, atol=1e-12 * max(np.abs(ref).max(), 1e-300))
        np.testing.assert_allclose(cabs[i], np.abs(A[rows, m]) @ np.abs(Xg[rows]), rtol=1e-12)
    # without a gather, B's rows are the group rows themselves
    xr = synth.activations(20, R, N)
    c3, _ = oracle.gemm_bf16_wgrad(dy, xr, None, off, sel[:3])
    ref3 = A[off[0]:off[1]].T @ bf16_vals(xr)[off[0]:off[1]]
    np.testing.assert_allclose(c3, ref3[[0, 11, M - 1]], rtol=1e-12, atol=1e-12 * np.abs(ref3).max())


def test_exp_f32_within_two_ulp_of_numpy():
    rng = np.random.default_rng(1)
    x = np.concatenate([rng.uniform(-87, 88, 400000), np.linspace(-20, 20, 20001)]).astype(np.float32)
    got = oracle.exp_f32_array(x).astype(np.float64)
    ref = np.exp(x.astype(np.float64))
    ulp = np.spacing(ref.astype(np.float32)).astype(np.float64)
    assert np.max(np.abs(got - ref) / ulp) <= 2.0
    assert oracle.exp_f32(0.0) == 1.0
    assert oracle.exp_f32(100.0) == np.inf and oracle.exp_f32(-200.0) == 0.0


def test_swiglu_matches_float64_formula():
    R, I = 64, 96
    h13 = synth.fp32_matrix(2, R, 2 * I, std=3.0)
    h = oracle.swiglu(h13)
    gate = h13[:, :I].astype(np.float64)
    up = h13[:, I:].astype(np.float64)
    ref = gate / (1.0 + np.exp(-gate)) * up
    got = synth.f32_from_bf16_bits(h).astype(np.float64)
    # bf16 rounding (2^-9 relative) plus a few f32 ulps
    np.testing.assert_allclose(got, ref, rtol=2.0 ** -8, atol=1e-30)
    # exact special values: silu(0) = 0, silu(-inf side) -> -0, silu(large) = z
    assert oracle.lib().orc_silu_f32(0.0) == 0.0
    assert oracle.lib().orc_silu_f32(100.0) == 100.0


def test_nvfp4_wgrad_matches_float64_matmul_per_group():
    """NVFP4 weight-gradient form on grouped columnwise copies with one outer
    scale per group and operand: C_g = gA_g gB_g A_g B_g^T over the group's
    padded columns (padding columns are zero codes)."""
    G, NA, NB, ld = 3, 32, 48, 128
    rng = np.random.default_rng(7)
    ac = rng.integers(0, 256, (NA, ld // 2)).astype(np.uint8)
    asc = rng.integers(0x20, 0x50, (NA, ld // 16)).astype(np.uint8)
    bc = rng.integers(0, 256, (NB, ld // 2)).astype(np.uint8)
    bsc = rng.integers(0x20, 0x50, (NB, ld // 16)).astype(np.uint8)
    off = np.array([0, 20, 20, 70], np.int64)          # padded starts 0, 32, 32, 96
    ag = np.array([0.5, 2.0, 0.125], np.float32)
    bg = np.array([3.0, 1.0, 0.25], np.float32)
    sel = np.array([[g, n] for g in range(G) for n in (0, 5, NA - 1)], np.int64)
    c, cabs = oracle.gemm_wgrad_nvfp4(ac, asc, ag, bc, bsc, bg, off, sel)
    A = nvfp4_exact(ac, asc, np.ones(NA, np.float32))
    B = nvfp4_exact(bc, bsc, np.ones(NB, np.float32))
    P = oracle.padded_offsets(off)
    for i, (g, n) in enumerate(sel):
        cols = slice(P[g], P[g + 1])
        ref = ag[g] * bg[g] * (B[:, cols] @ A[n, cols])
        np.testing.assert_allclose(c[i], ref, rtol=1e-12, atol=1e-12 * max(np.abs(ref).max(), 1e-300))
    assert not c[3:6].any()                            # the empty group
