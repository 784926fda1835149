"""Pins of the oracle's block quantizers, dequantizers and requant + SR.

Pins used (none re-types the oracle's own formula as the expectation):
  * the worked examples printed on the pages (tests/golden);
  * Philox4x32-10 known-answer vectors;
  * closed forms: exact round trips of representable tensors, exact SR
    probabilities, the transpose identity between rowwise and columnwise;
  * invariants: batch invariance of per-token scaling, block maximum = 6 in
    standard mode, SR unbiasedness within a binomial bound;
  * library routines: torch's float8 casts for decoding.
"""
import numpy as np
import pytest
import torch

import oracle
from block_scaled_precision_token_amd import synth
from tests.conftest import GOLDEN, read_golden

E2M1 = np.array([float(v) for v in read_golden("e2m1_value_set.txt")["values"].split()])


def bf16(values):
    return synth.bf16_bits_from_f32(np.asarray(values, np.float32))


def nib(codes, M, K):
    """Unpack NVFP4 codes [M, K/2] -> [M, K] (element 2j in the low nibble)."""
    c = codes.reshape(M, K // 2)
    out = np.empty((M, K), np.uint8)
    out[:, 0::2] = c & 15
    out[:, 1::2] = c >> 4
    return out


def e2m1_vals(n):
    return np.where(n & 8, -E2M1[n & 7], E2M1[n & 7])


def e4m3_vals(codes):
    return torch.from_numpy(np.ascontiguousarray(codes, np.uint8)).view(torch.float8_e4m3fn).double().numpy()


def e4m3_code(v):
    return int(torch.tensor([v], dtype=torch.float32).to(torch.float8_e4m3fn).view(torch.uint8)[0])


# --------------------------------------------------------------------------
# Worked examples of the pages
# --------------------------------------------------------------------------

def worked_rows():
    gold = read_golden("worked_encode.txt")
    big = float(gold["x_block0"])
    m54, v54 = (float(t) for t in gold["x_block1"].split())
    x = np.zeros((16, 32), np.float32)
    x[0, 0] = big
    x[0, 16] = m54
    x[0, 17] = v54
    x[1, 0] = big
    x[1, 17] = 12.0
    return bf16(x)


def test_worked_encode_minus54_is_minus6_times_9():
    gold = read_golden("worked_encode.txt")
    x = worked_rows()
    codes, scales, outer = oracle.quantize_nvfp4(x)
    assert outer[0] == 1.0
    q = nib(codes, 16, 32)
    assert e4m3_vals(scales[0:1, 1])[0] == float(gold["expect_block1_scale"])
    assert e2m1_vals(q[0, 16]) == float(gold["expect_element_minus54"])
    f, _ = oracle.dequantize_nvfp4(codes, scales, outer)
    assert f[0, 16] == -54.0
    assert f[0, 17] == float(gold["expect_dequant_5.4"])


def test_worked_requant_rtn_and_sr_probabilities():
    gold = read_golden("worked_requant.txt")
    col = int(gold["column"])
    codes, scales, outer = oracle.quantize_nvfp4(worked_rows())
    f, _ = oracle.dequantize_nvfp4(codes, scales, outer)
    assert f[1, col] == 12.0 and f[0, col] == 4.5
    cT, sT, G = oracle.requant_transpose_sr(codes, scales, outer, seed=7, use_sr=False)
    assert G[0] == 1.0
    assert e4m3_vals(sT[col:col + 1, 0])[0] == float(gold["expect_new_scale"])
    qT = nib(cT, 32, 16)
    assert e2m1_vals(qT[col, 0]) == float(gold["expect_rtn_element"])
    fT, _ = oracle.dequantize_nvfp4(cT, sT, np.full(32, G[0], np.float32))
    assert fT[col, 0] == float(gold["expect_rtn_dequant"])
    # stochastic rounding of 2.25: over all 2^16 random words the round-up
    # count is exactly 1/4 of them
    v = float(gold["expect_scaled_value"])
    ups = sum(oracle.e2m1_sr_mag(v, u) == 5 for u in range(65536))
    downs = sum(oracle.e2m1_sr_mag(v, u) == 4 for u in range(65536))
    assert E2M1[5] == float(gold["expect_sr_high_element"]) and E2M1[4] == float(gold["expect_sr_low_element"])
    assert ups / 65536 == float(gold["expect_sr_high_probability"])
    assert downs / 65536 == float(gold["expect_sr_low_probability"])
    # and the mean over many seeds of the requantized value returns 4.5
    vals = []
    for seed in range(4000):
        cT, sT, G = oracle.requant_transpose_sr(codes, scales, outer, seed=seed, use_sr=True)
        q = nib(cT, 32, 16)[col, 0]
        vals.append(e2m1_vals(q) * e4m3_vals(sT[col:col + 1, 0])[0] * G[0])
    vals = np.array(vals)
    assert set(np.unique(vals)) <= {4.0, 6.0}
    p = np.mean(vals == 6.0)
    assert abs(p - 0.25) < 4 * np.sqrt(0.25 * 0.75 / len(vals))
    assert abs(vals.mean() - float(gold["expect_sr_mean_dequant"])) < 4 * 2 * np.sqrt(0.25 * 0.75 / len(vals))


# --------------------------------------------------------------------------
# NVFP4 quantizer
# --------------------------------------------------------------------------

def test_nvfp4_round_trip_exact_on_representable_tensor():
    rng = np.random.default_rng(11)
    M, K = 24, 128
    x = np.zeros((M, K), np.float32)
    x[:, 0] = 2688.0                      # outer scale exactly 1 for every row
    for r in range(M):
        for b in range(1, K // 16):
            s = e4m3_vals(np.array([rng.integers(8, 0x7E)], np.uint8))[0]   # a normal E4M3 scale
            q = rng.integers(0, 16, 16)
            q[rng.integers(0, 16)] = 7 | (8 * rng.integers(0, 2))            # block max is 6
            x[r, b * 16:(b + 1) * 16] = e2m1_vals(q) * s
    xb = bf16(x)
    assert np.array_equal(synth.f32_from_bf16_bits(xb), x)                    # representable in bf16
    codes, scales, outer = oracle.quantize_nvfp4(xb)
    f, _ = oracle.dequantize_nvfp4(codes, scales, outer)
    np.testing.assert_array_equal(f, x)
    # the nibble order and scale layout are the canonical ones
    q = nib(codes, M, K)
    ref = e2m1_vals(q) * e4m3_vals(scales.reshape(-1)).reshape(M, K // 16).repeat(16, axis=1)
    np.testing.assert_array_equal(ref, x)


def test_nvfp4_batch_invariance_per_token():
    x = synth.activations(5, 64, 256)
    c0, s0, g0 = oracle.quantize_nvfp4(x, mode46=True)
    y = x.copy()
    y[1:] = synth.activations(6, 63, 256)                 # every other row changes
    y = np.concatenate([synth.activations(7, 5, 256), y])  # rows inserted before
    c1, s1, g1 = oracle.quantize_nvfp4(y, mode46=True)
    np.testing.assert_array_equal(c1[5], c0[0])
    np.testing.assert_array_equal(s1[5], s0[0])
    assert g1[5] == g0[0]
    # a per-tensor scope does depend on the other rows
    _, _, gt0 = oracle.quantize_nvfp4(x, rows_per_scale=64)
    _, _, gt1 = oracle.quantize_nvfp4(y[5:], rows_per_scale=64)
    assert gt0[0] != gt1[0]


def test_nvfp4_standard_block_max_is_six():
    x = synth.activations(8, 128, 512)
    codes, scales, outer = oracle.quantize_nvfp4(x)
    q = nib(codes, 128, 512).reshape(128, 32, 16)
    mag = (q & 7).max(axis=2)
    normal = (scales & 0x78) != 0
    assert normal.any()
    assert np.all(mag[normal] == 7)
    # each token's largest block has scale 448
    assert np.all(scales.max(axis=1) == 0x7E)


def test_nvfp4_scale_is_e4m3_of_block_ratio_library_cast():
    """Block scale equals torch's e4m3 cast of a / (6 g) (g read back from the oracle)."""
    x = synth.activations(9, 32, 256)
    codes, scales, outer = oracle.quantize_nvfp4(x)
    xf = synth.f32_from_bf16_bits(x).reshape(32, 16, 16)
    a = np.abs(xf).max(axis=2)
    ratio = (a / (np.float32(6.0) * outer[:, None]).astype(np.float32)).astype(np.float32)
    ref = torch.from_numpy(np.clip(ratio, 0, 448)).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    np.testing.assert_array_equal(scales, ref)


def test_nvfp4_per_group_scope_equals_tensor_max():
    E, N, K = 3, 32, 64
    w = synth.weights(10, E, N, K)
    codes, scales, outer = oracle.quantize_nvfp4(w, rows_per_scale=N)
    wf = np.abs(synth.f32_from_bf16_bits(w)).reshape(E, N * K).max(axis=1)
    assert outer.shape == (E,)
    # g = amax / 2688 within one rounding
    np.testing.assert_allclose(outer.astype(np.float64) * 2688.0, wf, rtol=2 ** -23)


def test_nvfp4_zero_and_tiny_and_signed_zero():
    x = np.zeros((3, 32), np.float32)
    x[1, :] = -0.0
    x[2, 0] = 1e-38            # tiny scope: eff underflows, block flushes
    xb = bf16(x)
    codes, scales, outer = oracle.quantize_nvfp4(xb)
    assert outer[0] == 0 and outer[1] == 0
    assert np.all(scales == 0)
    q = nib(codes, 3, 32)
    assert np.all(q[0] == 0) and np.all(q[1] == 8)
    f, _ = oracle.dequantize_nvfp4(codes, scales, outer)
    assert np.all(f == 0)


def _block_row(vals, g_one=True):
    x = np.zeros((1, 32), np.float32)
    x[0, 0] = 2688.0
    x[0, 16:16 + len(vals)] = vals
    return bf16(x)


def test_46_four_wins_strictly():
    # 52 = 4 * 13 exactly; with the "6" candidate 52/6 rounds to scale 9 and
    # the block reconstructs 54 (error 2 per element); the "4" candidate uses
    # scale 13 and is exact.
    xb = _block_row([52.0] * 16)
    _, s6, _ = oracle.quantize_nvfp4(xb, mode46=False)
    c, s46, g = oracle.quantize_nvfp4(xb, mode46=True)
    assert e4m3_vals(s6[0, 1:2])[0] == 9.0
    assert e4m3_vals(s46[0, 1:2])[0] == 13.0
    f, _ = oracle.dequantize_nvfp4(c, s46, g)
    assert np.all(f[0, 16:] == 52.0)
    # the "6" block of the row is untouched by the choice (ties keep 6)
    assert s46[0, 0] == s6[0, 0] == 0x7E


def test_46_tie_keeps_six():
    # 36 = 6 * 6 = 4 * 9: both candidates are exact (error 0): the tie keeps "6"
    xb = _block_row([36.0] * 16)
    _, s46, _ = oracle.quantize_nvfp4(xb, mode46=True)
    assert e4m3_vals(s46[0, 1:2])[0] == 6.0


def test_46_six_wins_strictly():
    # block of multiples of 9 with maximum 54: "6" (scale 9) is exact; the "4"
    # candidate needs scale 13.5 -> 14 and cannot reconstruct 54
    xb = _block_row([54.0, 27.0, 9.0, 4.5, -13.5, 18.0])
    _, s46, _ = oracle.quantize_nvfp4(xb, mode46=True)
    assert e4m3_vals(s46[0, 1:2])[0] == 9.0


def test_46_picks_lower_error_on_random_blocks():
    """Whenever the two candidates' float64 squared errors differ clearly, the
    oracle keeps the lower one (candidates rebuilt with torch's e4m3 cast)."""
    x = synth.activations(12, 64, 256)
    c46, s46, g = oracle.quantize_nvfp4(x, mode46=True)
    xf = synth.f32_from_bf16_bits(x).astype(np.float64).reshape(64, 16, 16)
    f46, _ = oracle.dequantize_nvfp4(c46, s46, g)
    err_chosen = ((f46.reshape(64, 16, 16) - xf) ** 2).sum(axis=2)
    decided = 0
    for D in (6.0, 4.0):
        a = np.abs(xf).max(axis=2).astype(np.float32)
        ratio = (a / (np.float32(D) * g[:, None]).astype(np.float32)).astype(np.float32)
        s = torch.from_numpy(np.clip(ratio, 0, 448)).to(torch.float8_e4m3fn).double().numpy()
        eff = (s.astype(np.float32) * g[:, None]).astype(np.float32).astype(np.float64)
        v = np.abs(xf) / eff[:, :, None]
        cand = E2M1[np.abs(v[..., None] - E2M1).argmin(axis=-1)]
        cand = np.where(v >= 6, 6.0, cand) * np.sign(xf)
        err = ((cand * eff[:, :, None] - xf) ** 2).sum(axis=2)
        if D == 6.0:
            err6 = err
        else:
            err4 = err
    clear = np.abs(err4 - err6) > 1e-3 * np.maximum(err4, err6)
    assert np.all(np.isclose(err_chosen[clear], np.minimum(err4, err6)[clear], rtol=1e-6, atol=0))
    decided = clear.sum()
    assert decided > 500
    # both candidates are actually used on this data
    four = np.isclose(err_chosen, err4, rtol=1e-9) & (err4 < err6) & clear
    assert four.any() and (clear & ~four).any()


# --------------------------------------------------------------------------
# MXFP8 quantizer
# --------------------------------------------------------------------------

def test_mxfp8_dequant_matches_library_decode_and_is_idempotent():
    x = synth.activations(13, 64, 256, row_log10_range=(-3, 2))
    codes, scales = oracle.quantize_mxfp8_rowwise(x)
    f, b = oracle.dequantize_mxfp8(codes, scales)
    ref = e4m3_vals(codes.reshape(-1)).reshape(64, 256) * np.exp2(scales.astype(np.float64) - 127).repeat(32, axis=1)
    np.testing.assert_array_equal(f.astype(np.float64), ref)
    # dequantized values are exact in bf16, and quantizing them again keeps
    # every value (codes may change: a block max that rounded down to 224 * 2^k
    # re-quantizes with exponent k - 1)
    np.testing.assert_array_equal(synth.f32_from_bf16_bits(b), f)
    c2, s2 = oracle.quantize_mxfp8_rowwise(b)
    f2, _ = oracle.dequantize_mxfp8(c2, s2)
    np.testing.assert_array_equal(f2, f)


def test_mxfp8_never_clips_and_is_nearest():
    x = synth.activations(14, 32, 256)
    codes, scales = oracle.quantize_mxfp8_rowwise(x)
    xf = synth.f32_from_bf16_bits(x).astype(np.float64)
    k = scales.astype(np.float64) - 127
    y = xf / np.exp2(k).repeat(32, axis=1)
    assert np.abs(y).max() <= 448
    # codes are torch's RNE e4m3 cast of the exactly scaled values
    ref = torch.from_numpy(y.astype(np.float32)).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    np.testing.assert_array_equal(codes, ref)
    # and the exponent is minimal: halving the scale would clip the block max
    amax = np.abs(y.reshape(32, 8, 32)).max(axis=2)
    assert np.all(amax > 224)


def test_mxfp8_columnwise_is_rowwise_of_transpose():
    x = synth.activations(15, 96, 64)
    cT, sT = oracle.quantize_mxfp8_colwise(x)
    cr, sr = oracle.quantize_mxfp8_rowwise(np.ascontiguousarray(x.T))
    np.testing.assert_array_equal(cT, cr)
    np.testing.assert_array_equal(sT, sr)


def test_mxfp8_columnwise_rejects_partial_blocks_without_groups():
    # an ungrouped copy has whole 32-row blocks only; one group pads instead
    x = synth.activations(17, 19, 64)
    with pytest.raises(ValueError):
        oracle.quantize_mxfp8_colwise(x)
    cT, sT = oracle.quantize_mxfp8_colwise(x, np.array([0, 19], np.int64))
    assert cT.shape == (64, 32) and sT.shape == (64, 1) and not cT[:, 19:].any()


def test_mxfp8_grouped_columnwise_pads_each_group():
    x = synth.activations(16, 100, 64)
    off = np.array([0, 5, 5, 40, 100], np.int64)      # includes an empty group
    P = oracle.padded_offsets(off)
    assert P.tolist() == [0, 32, 32, 96, 160]   # 5 -> 32, 0 -> 0, 35 -> 64, 60 -> 64
    cT, sT = oracle.quantize_mxfp8_colwise(x, off)
    for g in range(4):
        n = off[g + 1] - off[g]
        if n == 0:
            continue
        pad = np.zeros((P[g + 1] - P[g], 64), np.uint16)
        pad[:n] = x[off[g]:off[g + 1]]
        cr, sr = oracle.quantize_mxfp8_rowwise(np.ascontiguousarray(pad.T))
        np.testing.assert_array_equal(cT[:, P[g]:P[g + 1]], cr)
        np.testing.assert_array_equal(sT[:, P[g] // 32:P[g + 1] // 32], sr)


def test_mxfp8_edge_tensors():
    x = np.zeros((2, 64), np.float32)
    x[1, :32] = 3.3895313892515355e38       # bf16 max
    x[1, 32:] = -1e-40                      # bf16 subnormal-sized values
    xb = bf16(x)
    codes, scales = oracle.quantize_mxfp8_rowwise(xb)
    assert np.all(scales[0] == 0) and np.all(codes[0] == 0)
    f, b = oracle.dequantize_mxfp8(codes, scales)
    # bf16 max saturates at 448 * 2^119 rather than dequantizing to infinity
    assert scales[1, 0] == 119 + 127 and np.all(codes[1, :32] == 0x7E)
    assert np.all(f[1, :32] == np.float32(448.0 * 2.0 ** 119)) and np.all(np.isfinite(f))
    assert np.all(np.isfinite(synth.f32_from_bf16_bits(b)))
    assert np.all(np.signbit(f[1, 32:]))


# --------------------------------------------------------------------------
# Philox + stochastic rounding + requant
# --------------------------------------------------------------------------

def test_philox_known_answers():
    with open(f"{GOLDEN}/philox4x32_10_kat.txt") as fh:
        lines = [l for l in fh if l.strip() and not l.startswith("#")]
    assert len(lines) == 3
    for line in lines:
        lhs, rhs = line.split("->")
        w = [int(t, 16) for t in lhs.split()]
        expect = [int(t, 16) for t in rhs.split()]
        assert oracle.philox4x32_10(w[:4], w[4:6]).tolist() == expect


def test_sr_probability_is_ceiling_of_fraction():
    rng = np.random.default_rng(17)
    for v in np.concatenate([rng.uniform(0, 6, 40), [0.0, 0.5, 1.75, 2.9999, 5.999]]).astype(np.float32):
        v = float(v)
        lo = int(np.searchsorted(E2M1, v, side="right") - 1)
        frac = (v - E2M1[lo]) / (E2M1[lo + 1] - E2M1[lo])
        ups = sum(oracle.e2m1_sr_mag(v, u) == lo + 1 for u in range(0, 65536, 1))
        assert ups == int(np.ceil(frac * 65536)), v
    assert oracle.e2m1_sr_mag(6.0, 0) == 7 and oracle.e2m1_sr_mag(100.0, 65535) == 7


def test_sr_is_unbiased_over_seeds():
    x = synth.activations(18, 32, 32)
    codes, scales, outer = oracle.quantize_nvfp4(x)
    ref_c, ref_s, G = oracle.requant_transpose_sr(codes, scales, outer, use_sr=False)
    f_in, _ = oracle.dequantize_nvfp4(codes, scales, outer)
    acc = np.zeros((32, 32))
    n = 1500
    for seed in range(n):
        cT, sT, G = oracle.requant_transpose_sr(codes, scales, outer, seed=seed, use_sr=True)
        np.testing.assert_array_equal(sT, ref_s)   # scales do not depend on the random bits
        fT, _ = oracle.dequantize_nvfp4(cT, sT, np.full(32, G[0], np.float32))
        acc += fT
    mean = acc / n
    target = f_in.T.astype(np.float64)
    effs = e4m3_vals(sT.reshape(-1)).reshape(32, 2).repeat(16, axis=1) * G[0]
    # elements beyond 6 * eff (a block maximum whose scale rounded down) saturate
    # deterministically; every other element is rounded without bias
    sat = np.abs(target) > 6 * effs
    np.testing.assert_allclose(np.abs(mean[sat]), 6 * effs[sat], rtol=1e-6)
    inside = ~sat
    assert inside.sum() > 900
    # per element: |mean - target| within 5 sigma of the two-point distribution,
    # plus the 2^-16 resolution of the random bits
    gap = 2.0 * effs
    tol = 5 * gap * 0.5 / np.sqrt(n) + gap * 2 ** -16
    assert np.all(np.abs(mean - target)[inside] <= tol[inside] + 1e-12)
    # and the mean bias over the in-range elements is tiny
    assert abs((mean - target)[inside].mean()) < 0.005 * np.abs(target[inside]).mean()


def test_requant_rtn_equals_per_tensor_quantize_of_transpose():
    """With all per-row outer scales equal to 1/8 and the tensor maximum at
    6 * 448 * g, the requant's single outer scale equals the per-tensor scale,
    so RTN requant must equal per-tensor quantization of the transposed
    dequantized tensor (which is exact in bf16)."""
    rng = np.random.default_rng(19)
    M, K = 48, 64
    codes = rng.integers(0, 256, (M, K // 2)).astype(np.uint8)
    scales = rng.integers(0x20, 0x7F, (M, K // 16)).astype(np.uint8)
    scales[3, 1] = 0x7E
    codes[3, 10] = 0x07          # element (3, 20) = 6 in a block with scale 448
    outer = np.full(M, 0.125, np.float32)
    f, b = oracle.dequantize_nvfp4(codes, scales, outer)
    np.testing.assert_array_equal(synth.f32_from_bf16_bits(b), f)
    cT, sT, G = oracle.requant_transpose_sr(codes, scales, outer, use_sr=False)
    qc, qs, qg = oracle.quantize_nvfp4(np.ascontiguousarray(b.T), rows_per_scale=K)
    assert G[0] == qg[0] == 0.125
    np.testing.assert_array_equal(cT, qc)
    np.testing.assert_array_equal(sT, qs)


def test_sr_deterministic_in_seed_and_index():
    x = synth.activations(20, 32, 64)
    codes, scales, outer = oracle.quantize_nvfp4(x)
    a = oracle.requant_transpose_sr(codes, scales, outer, seed=123, use_sr=True)
    b = oracle.requant_transpose_sr(codes, scales, outer, seed=123, use_sr=True)
    c = oracle.requant_transpose_sr(codes, scales, outer, seed=124, use_sr=True)
    np.testing.assert_array_equal(a[0], b[0])
    assert not np.array_equal(a[0], c[0])
    # bits of element i come from Philox block i // 8 (low half for even i)
    w = oracle.philox4x32_10([5, 0, 0, 0], [123, 0])
    assert oracle.sr_bits(123, 40) == (w[0] & 0xFFFF)
    assert oracle.sr_bits(123, 43) == (w[1] >> 16)
    assert oracle.sr_bits(123, 47) == (w[3] >> 16)


def test_batched_requant_counter_stream_is_one_stacked_tensor():
    """Batched requant of E per-expert tensors with equal outer scales equals,
    bit for bit with stochastic rounding on, one requant of the tensors laid
    side by side along K (input [M, E*K] -> output [E*K, M]): output element
    (e, k, m) of the batch draws its bits at e*K*M + k*M + m."""
    E, M, K = 3, 32, 48
    w = synth.weights(31, E, M, K)
    codes, scales, g = oracle.quantize_nvfp4(w, rows_per_scale=E * M)      # one scale: G_e all equal
    outer_e = np.repeat(g, E)
    cT, sT, G = oracle.requant_transpose_sr_batched(codes, scales, outer_e, E, rows_per_scale=M, seed=77)
    side = lambda a: np.concatenate([a[e * M:(e + 1) * M] for e in range(E)], axis=1)
    cT1, sT1, G1 = oracle.requant_transpose_sr(side(codes), side(scales), np.repeat(g, M), seed=77)
    np.testing.assert_array_equal(cT, cT1)
    np.testing.assert_array_equal(sT, sT1)
    np.testing.assert_array_equal(G, np.repeat(G1, E))


def test_batched_requant_scales_each_expert_by_its_own_outer():
    """Per-expert weights (one outer scale per expert): each expert's output is
    its own requant (G_e = its outer scale), not one shared G."""
    E, M, K = 4, 32, 64
    w = synth.weights(32, E, M, K)
    wf = synth.f32_from_bf16_bits(w).reshape(E, M, K) * np.array([1, 10, 0.1, 3], np.float32)[:, None, None]
    w = synth.bf16_bits_from_f32(wf.reshape(E * M, K))
    codes, scales, g = oracle.quantize_nvfp4(w, rows_per_scale=M)
    assert len(set(g.tolist())) == E
    cT, sT, G = oracle.requant_transpose_sr_batched(codes, scales, g, E, rows_per_scale=M, use_sr=False)
    np.testing.assert_array_equal(G, g)
    for e in range(E):
        rows = slice(e * M, (e + 1) * M)
        c1, s1, G1 = oracle.requant_transpose_sr(codes[rows], scales[rows], np.full(M, g[e], np.float32),
                                                 use_sr=False)
        np.testing.assert_array_equal(cT[e * K:(e + 1) * K], c1)
        np.testing.assert_array_equal(sT[e * K:(e + 1) * K], s1)
        assert G1[0] == g[e]


def _stacked_padded(codes, scales, outer, src, off):
    """The grouped rows laid out as one rowwise tensor: group g's rows (read
    through src) then zero rows up to a multiple of 32."""
    K2, K16 = codes.shape[1], scales.shape[1]
    parts_c, parts_s, parts_o = [], [], []
    for g in range(off.size - 1):
        rows = src[off[g]:off[g + 1]]
        n = rows.size
        pad = (n + 31) // 32 * 32 - n
        parts_c += [codes[rows], np.zeros((pad, K2), np.uint8)]
        parts_s += [scales[rows], np.zeros((pad, K16), np.uint8)]
        parts_o += [outer[rows], np.zeros(pad, np.float32)]
    return np.concatenate(parts_c), np.concatenate(parts_s), np.concatenate(parts_o)


def test_grouped_requant_is_requant_of_the_padded_group_layout():
    """With every outer scale equal (so every G_g equals the single G), the
    grouped, gathered requant with stochastic rounding equals, bit for bit, one
    requant of the groups' rows laid out explicitly (gathered, each group
    zero-padded to 32 rows) -- the counter of output element (k, p) being
    k * ldT + p; columns past the padded total of a wider output stay
    untouched."""
    T, K = 40, 64
    off = np.array([0, 21, 21, 60, 93], np.int64)
    rng = np.random.default_rng(5)
    src = rng.integers(0, T, int(off[-1])).astype(np.int32)
    x = synth.activations(33, T, K)
    codes, scales, g = oracle.quantize_nvfp4(x, rows_per_scale=T)        # one outer scale for all rows
    outer = np.repeat(g, T)
    c2, s2, o2 = _stacked_padded(codes, scales, outer, src, off)
    P = c2.shape[0]
    cT, sT, G = oracle.requant_transpose_sr_grouped(codes, scales, outer, src, off, P, seed=11)
    cT1, sT1, G1 = oracle.requant_transpose_sr(c2, s2, np.where(o2 > 0, o2, g[0]), seed=11)
    np.testing.assert_array_equal(cT, cT1)
    np.testing.assert_array_equal(sT, sT1)
    np.testing.assert_array_equal(G, np.where(np.diff(off) > 0, g[0], 0.0).astype(np.float32))
    # a wider output: the counter follows the row length, so compare in RTN
    cTn, sTn, _ = oracle.requant_transpose_sr_grouped(codes, scales, outer, src, off, P, use_sr=False)
    cTw, sTw, _ = oracle.requant_transpose_sr_grouped(codes, scales, outer, src, off, P + 64, use_sr=False)
    np.testing.assert_array_equal(cTw[:, :P // 2], cTn)
    np.testing.assert_array_equal(sTw[:, :P // 16], sTn)
    assert not cTw[:, P // 2:].any() and not sTw[:, P // 16:].any()


def test_grouped_requant_scales_each_group_by_its_own_outer():
    """Per-token outer scales: each group is requantized with G_g = the max of
    its own rows' scales (RTN: equal to the single-tensor requant of that
    group's padded rows alone); a bad gather index reads as a zero row."""
    T, K = 50, 32
    off = np.array([0, 7, 40, 40, 71], np.int64)
    rng = np.random.default_rng(6)
    src = rng.integers(0, T, int(off[-1])).astype(np.int32)
    src[3] = -1
    x = synth.activations(34, T, K)
    codes, scales, outer = oracle.quantize_nvfp4(x)
    cT, sT, G = oracle.requant_transpose_sr_grouped(codes, scales, outer, src, off, 160, use_sr=False)
    Pg = np.concatenate([[0], np.cumsum((np.diff(off) + 31) // 32 * 32)])
    codes_x = np.concatenate([codes, np.zeros((1, K // 2), np.uint8)])   # row T: the zero row of a bad index
    scales_x = np.concatenate([scales, np.zeros((1, K // 16), np.uint8)])
    outer_x = np.concatenate([outer, np.zeros(1, np.float32)])
    src_x = np.where(src < 0, T, src)
    for gi in range(off.size - 1):
        rows = src_x[off[gi]:off[gi + 1]]
        if rows.size == 0:
            assert G[gi] == 0.0
            continue
        c1, s1, o1 = _stacked_padded(codes_x, scales_x, outer_x, rows, np.array([0, rows.size]))
        r1c, r1s, r1g = oracle.requant_transpose_sr(c1, s1, o1, use_sr=False)
        assert G[gi] == r1g[0] == outer_x[rows].max()
        np.testing.assert_array_equal(cT[:, Pg[gi] // 2:Pg[gi + 1] // 2], r1c)
        np.testing.assert_array_equal(sT[:, Pg[gi] // 16:Pg[gi + 1] // 16], r1s)


# --- numerics variants: 16x16 2-D scaling and the random Hadamard transform ---

def _nibble_transpose(codes, M, K):
    q = np.empty((M, K), np.uint8)
    q[:, 0::2] = codes & 15
    q[:, 1::2] = codes >> 4
    qt = np.ascontiguousarray(q.T)
    return (qt[:, 0::2] | (qt[:, 1::2] << 4)).astype(np.uint8)


def test_2d_scaling_is_transpose_invariant():
    """16x16 blocks keep their scales through a transpose [nopree.com, section
    第二个决定]: quantizing the transpose gives the transposed codes and scales."""
    M, K = 64, 96
    x = synth.activations(41, M, K)
    c, s, g = oracle.quantize_nvfp4_2d(x)
    ct, st, gt = oracle.quantize_nvfp4_2d(np.ascontiguousarray(x.T))
    assert g[0] == gt[0]
    np.testing.assert_array_equal(st, s.T)
    np.testing.assert_array_equal(ct, _nibble_transpose(c, M, K))


def test_2d_scaling_of_repeated_rows_equals_1x16_per_tensor():
    """When the 16 rows of every band are equal, a tile's amax is its row
    piece's amax, so 2-D scaling reduces to 1x16 blocks under one tensor scale."""
    M, K = 48, 64
    base = synth.activations(42, M // 16, K)
    x = np.repeat(base, 16, axis=0)
    c, s, g = oracle.quantize_nvfp4_2d(x)
    c1, s1, g1 = oracle.quantize_nvfp4(x, rows_per_scale=M)
    assert g[0] == g1[0]
    np.testing.assert_array_equal(c, c1)
    np.testing.assert_array_equal(np.repeat(s, 16, axis=0), s1)


def test_2d_scaling_one_outlier_flattens_its_tile():
    """The pages' warning about 16x16 blocks: one large value among 256 and the
    other 255 quantize to zero, where 1x16 blocks keep the other rows."""
    x = np.full((16, 16), 0.75, np.float32)
    x[::2] *= -1
    x[0, 0] = 2688.0                    # g = 1, tile scale E4M3(2688 / 6) = 448
    xb = synth.bf16_bits_from_f32(x)
    c, s, g = oracle.quantize_nvfp4_2d(xb)
    assert g[0] == 1.0 and s[0, 0] == oracle.e4m3_encode(448.0)
    mags = np.stack([c & 7, (c >> 4) & 7], axis=-1).reshape(16, 16)
    assert mags[0, 0] == 7 and np.count_nonzero(mags) == 1
    c1, s1, g1 = oracle.quantize_nvfp4(xb, rows_per_scale=16)
    mags1 = np.stack([c1 & 7, (c1 >> 4) & 7], axis=-1).reshape(16, 16)
    assert np.count_nonzero(mags1[1:]) == 15 * 16


def test_rht16_matches_the_hadamard_matrix():
    """The transform is (1/4) H16 D with H16 the Sylvester Hadamard matrix
    (scipy) and D the sign flips: exact on small integers, and inverted by
    D H16 / 4."""
    from scipy.linalg import hadamard
    Hm = hadamard(16).astype(np.float64)
    rng = np.random.default_rng(3)
    v = rng.integers(-64, 65, (50, 16)).astype(np.float32)
    for signs in (0, 0xA5C3, 0xFFFF):
        d = np.array([-1.0 if (signs >> i) & 1 else 1.0 for i in range(16)])
        got = oracle.rht16(v, signs).astype(np.float64)
        ref = (v.astype(np.float64) * d) @ Hm.T / 4
        np.testing.assert_array_equal(got, ref)
        back = (got @ Hm.T / 4) * d
        np.testing.assert_array_equal(back, v)


def test_rht_quantize_is_quantize_of_the_transformed_rows():
    """Rows built from signed Hadamard columns transform to scaled unit
    vectors, exact in bf16: RHT-then-quantize equals the plain per-token
    quantizer on the transformed rows."""
    from scipy.linalg import hadamard
    Hm = hadamard(16).astype(np.float64)
    signs = 0x3C5A
    d = np.array([-1.0 if (signs >> i) & 1 else 1.0 for i in range(16)])
    rng = np.random.default_rng(4)
    M, K = 8, 64
    y = np.zeros((M, K), np.float64)
    for r in range(M):
        for b in range(K // 16):
            y[r, 16 * b + rng.integers(0, 16)] = 4.0 * rng.choice([0.5, 1.0, 1.5, 3.0, -2.0, 6.0])
    x = np.empty_like(y)
    for b in range(K // 16):
        x[:, 16 * b:16 * b + 16] = (y[:, 16 * b:16 * b + 16] @ Hm / 4) * d   # the inverse transform
    xb = synth.bf16_bits_from_f32(x.astype(np.float32))
    assert np.array_equal(synth.f32_from_bf16_bits(xb).astype(np.float64), x)
    for m46 in (False, True):
        c, s, g = oracle.quantize_nvfp4_rht(xb, signs, mode46=m46)
        c1, s1, g1 = oracle.quantize_nvfp4(synth.bf16_bits_from_f32(y.astype(np.float32)), mode46=m46)
        np.testing.assert_array_equal(g, g1)
        np.testing.assert_array_equal(s, s1)
        np.testing.assert_array_equal(c, c1)
