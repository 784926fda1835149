"""CPU oracle for the block-scaled quantization path -- TEST INFRASTRUCTURE ONLY.

Thin numpy/ctypes wrapper around ``bsp_oracle.c`` (plain scalar C, IEEE f32
with no contraction, binary64 for the GEMM reference).  Only the tests, the
smoke check and the benchmark's CPU-baseline leg may import this package; the
HIP library and its Python binding never do.

Each wrapper states which passage of the pages it follows; the C source holds
the full readings.  Parity of the 4/6 choice and of the synthetic routing is
unpinned by the pages (no worked example); everything else is pinned by the
tests in ``tests/test_oracle_*.py``.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
import threading

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "bsp_oracle.c")
_LIB_DIR = os.path.join(_HERE, "_build")
_LIB = os.path.join(_LIB_DIR, "liboracle.so")
_CFLAGS = ["-O2", "-std=c11", "-fPIC", "-shared", "-fopenmp", "-ffp-contract=off", "-fno-fast-math",
           "-fvisibility=hidden", "-Wall", "-Wextra"]

_lock = threading.Lock()
_lib = None


def build(force: bool = False) -> str:
    """Compile the oracle with gcc (IEEE f32, no contraction, OpenMP over rows)."""
    os.makedirs(_LIB_DIR, exist_ok=True)
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        tmp = _LIB + f".tmp{os.getpid()}"
        subprocess.check_call(["gcc", *_CFLAGS, _SRC, "-o", tmp, "-lm"])
        os.replace(tmp, _LIB)
    return _LIB


def _load():
    global _lib
    with _lock:
        if _lib is None:
            lib = ctypes.CDLL(build())
            _declare(lib)
            _lib = lib
    return _lib


P = ctypes.c_void_p
I64 = ctypes.c_int64
U64 = ctypes.c_uint64


def _declare(lib):
    lib.orc_bf16_to_f32.argtypes = [ctypes.c_uint16]
    lib.orc_bf16_to_f32.restype = ctypes.c_float
    lib.orc_f32_to_bf16.argtypes = [ctypes.c_float]
    lib.orc_f32_to_bf16.restype = ctypes.c_uint16
    lib.orc_e2m1_value.argtypes = [ctypes.c_uint8]
    lib.orc_e2m1_value.restype = ctypes.c_float
    lib.orc_e2m1_encode.argtypes = [ctypes.c_float]
    lib.orc_e2m1_encode.restype = ctypes.c_uint8
    lib.orc_e4m3_value.argtypes = [ctypes.c_uint8]
    lib.orc_e4m3_value.restype = ctypes.c_float
    lib.orc_e4m3_encode_sat.argtypes = [ctypes.c_float]
    lib.orc_e4m3_encode_sat.restype = ctypes.c_uint8
    lib.orc_e8m0_value.argtypes = [ctypes.c_uint8]
    lib.orc_e8m0_value.restype = ctypes.c_float
    lib.orc_mxfp8_block_exponent.argtypes = [ctypes.c_float]
    lib.orc_mxfp8_block_exponent.restype = ctypes.c_int
    lib.orc_quantize_nvfp4.argtypes = [P, I64, I64, I64, ctypes.c_int, P, P, P]
    lib.orc_quantize_nvfp4_2d.argtypes = [P, I64, I64, P, P, P]
    lib.orc_rht16.argtypes = [P, ctypes.c_uint32]
    lib.orc_quantize_nvfp4_rht.argtypes = [P, I64, I64, ctypes.c_uint32, ctypes.c_int, P, P, P]
    lib.orc_dequantize_nvfp4.argtypes = [P, P, P, I64, I64, I64, P, P]
    lib.orc_quantize_mxfp8_rowwise.argtypes = [P, I64, I64, P, P]
    lib.orc_padded_offsets.argtypes = [P, I64, P]
    lib.orc_quantize_mxfp8_colwise.argtypes = [P, I64, I64, P, I64, I64, P, P]
    lib.orc_dequantize_mxfp8.argtypes = [P, P, I64, I64, P, P]
    lib.orc_philox4x32_10.argtypes = [P, P, P]
    lib.orc_sr_bits.argtypes = [U64, U64]
    lib.orc_sr_bits.restype = ctypes.c_uint16
    lib.orc_e2m1_sr_mag.argtypes = [ctypes.c_float, ctypes.c_uint16]
    lib.orc_e2m1_sr_mag.restype = ctypes.c_uint8
    lib.orc_requant_transpose_sr.argtypes = [P, P, P, I64, I64, U64, ctypes.c_int, P, P, P]
    lib.orc_requant_transpose_sr_batched.argtypes = [P, P, P, I64, I64, I64, I64, U64, ctypes.c_int, P, P, P]
    lib.orc_gemm_rowgroup.argtypes = [ctypes.c_int, P, P, P, P, P, I64, I64, I64, I64, P, P, P, P, I64, P, P]
    lib.orc_gemm_wgrad.argtypes = [P, P, P, P, P, I64, I64, I64, I64, P, I64, P, P]
    lib.orc_gemm_wgrad_fmt.argtypes = [ctypes.c_int, P, P, P, P, P, P, P, I64, I64, I64, I64, P, I64, P, P]
    lib.orc_requant_transpose_sr_grouped.argtypes = [P, P, P, I64, P, P, I64, I64, I64, U64, ctypes.c_int, P, P, P]
    lib.orc_gemm_bf16_rowgroup.argtypes = [ctypes.c_int, P, I64, I64, P, I64, P, P, I64, I64, I64, P, I64, P, P]
    lib.orc_gemm_bf16_wgrad.argtypes = [P, I64, P, I64, P, I64, P, I64, P, I64, P, P]
    lib.orc_exp_f32.argtypes = [ctypes.c_float]
    lib.orc_exp_f32.restype = ctypes.c_float
    lib.orc_silu_f32.argtypes = [ctypes.c_float]
    lib.orc_silu_f32.restype = ctypes.c_float
    lib.orc_silu_f64.argtypes = [ctypes.c_double]
    lib.orc_silu_f64.restype = ctypes.c_double
    lib.orc_swiglu.argtypes = [P, I64, I64, P]
    for name in ("orc_e2m1_encode_array", "orc_e4m3_encode_array", "orc_mxfp8_block_exponent_array",
                 "orc_f32_to_bf16_array", "orc_exp_f32_array"):
        getattr(lib, name).argtypes = [P, I64, P]
    lib.orc_num_threads.restype = ctypes.c_int
    lib.orc_set_num_threads.argtypes = [ctypes.c_int]


def _ptr(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _c(a, dtype):
    return np.ascontiguousarray(a, dtype=dtype)


def lib():
    return _load()


def num_threads() -> int:
    return _load().orc_num_threads()


def set_num_threads(n: int) -> None:
    _load().orc_set_num_threads(int(n))


# --- scalar codecs ----------------------------------------------------------

def e2m1_value(code: int) -> float:
    return _load().orc_e2m1_value(code)


def e2m1_encode(v: float) -> int:
    return _load().orc_e2m1_encode(v)


def e4m3_value(code: int) -> float:
    return _load().orc_e4m3_value(code)


def e4m3_encode(y: float) -> int:
    return _load().orc_e4m3_encode_sat(y)


def e8m0_value(code: int) -> float:
    return _load().orc_e8m0_value(code)


def mxfp8_block_exponent(amax: float) -> int:
    return _load().orc_mxfp8_block_exponent(amax)


def f32_to_bf16(x: float) -> int:
    return _load().orc_f32_to_bf16(x)


def exp_f32(x: float) -> float:
    return _load().orc_exp_f32(x)


def _array_call(name, v, in_dtype, out_dtype):
    v = _c(v, in_dtype)
    out = np.empty(v.shape, out_dtype)
    getattr(_load(), name)(_ptr(v), v.size, _ptr(out))
    return out


def e2m1_encode_array(v):
    return _array_call("orc_e2m1_encode_array", v, np.float32, np.uint8)


def e4m3_encode_array(v):
    return _array_call("orc_e4m3_encode_array", v, np.float32, np.uint8)


def mxfp8_block_exponent_array(a):
    return _array_call("orc_mxfp8_block_exponent_array", a, np.float32, np.int32)


def f32_to_bf16_array(v):
    return _array_call("orc_f32_to_bf16_array", v, np.float32, np.uint16)


def exp_f32_array(v):
    return _array_call("orc_exp_f32_array", v, np.float32, np.float32)


# --- NVFP4 ------------------------------------------------------------------

def quantize_nvfp4(x_bf16: np.ndarray, rows_per_scale: int = 1, mode46: bool = False):
    """x_bf16: uint16 [M, K].  Returns (codes u8 [M,K/2], scales u8 [M,K/16], outer f32 [M/rps])."""
    x = _c(x_bf16, np.uint16)
    M, K = x.shape
    codes = np.empty((M, K // 2), np.uint8)
    scales = np.empty((M, K // 16), np.uint8)
    outer = np.empty((M // rows_per_scale,), np.float32)
    _load().orc_quantize_nvfp4(_ptr(x), M, K, rows_per_scale, int(bool(mode46)), _ptr(codes), _ptr(scales),
                               _ptr(outer))
    return codes, scales, outer


def quantize_nvfp4_2d(x_bf16: np.ndarray):
    """NVFP4 with 16x16 2-D block scales and one per-tensor outer scale:
    (codes [M, K/2], scales [M/16, K/16], outer [1])."""
    x = _c(x_bf16, np.uint16)
    M, K = x.shape
    codes = np.empty((M, K // 2), np.uint8)
    scales = np.empty((M // 16, K // 16), np.uint8)
    outer = np.empty(1, np.float32)
    _load().orc_quantize_nvfp4_2d(_ptr(x), M, K, _ptr(codes), _ptr(scales), _ptr(outer))
    return codes, scales, outer


def rht16(v, signs: int):
    """The 16-point random Hadamard transform of each row of v (f32 [n, 16])."""
    v = np.array(v, dtype=np.float32, copy=True).reshape(-1, 16)
    for row in v:
        _load().orc_rht16(row.ctypes.data_as(ctypes.c_void_p), signs)
    return v


def quantize_nvfp4_rht(x_bf16: np.ndarray, signs: int, mode46: bool = False):
    """Per-token NVFP4 of the rows after a 16-point RHT of each block."""
    x = _c(x_bf16, np.uint16)
    M, K = x.shape
    codes = np.empty((M, K // 2), np.uint8)
    scales = np.empty((M, K // 16), np.uint8)
    outer = np.empty(M, np.float32)
    _load().orc_quantize_nvfp4_rht(_ptr(x), M, K, signs, int(mode46), _ptr(codes), _ptr(scales), _ptr(outer))
    return codes, scales, outer


def dequantize_nvfp4(codes, scales, outer, rows_per_scale: int = 1):
    """Returns (f32 [M,K], bf16 bits [M,K])."""
    codes = _c(codes, np.uint8)
    scales = _c(scales, np.uint8)
    outer = _c(outer, np.float32)
    M, K = codes.shape[0], codes.shape[1] * 2
    f = np.empty((M, K), np.float32)
    b = np.empty((M, K), np.uint16)
    _load().orc_dequantize_nvfp4(_ptr(codes), _ptr(scales), _ptr(outer), M, K, rows_per_scale, _ptr(f), _ptr(b))
    return f, b


# --- MXFP8 ------------------------------------------------------------------

def quantize_mxfp8_rowwise(x_bf16):
    x = _c(x_bf16, np.uint16)
    M, K = x.shape
    codes = np.empty((M, K), np.uint8)
    scales = np.empty((M, K // 32), np.uint8)
    _load().orc_quantize_mxfp8_rowwise(_ptr(x), M, K, _ptr(codes), _ptr(scales))
    return codes, scales


def padded_offsets(group_offsets):
    off = _c(group_offsets, np.int64)
    G = off.size - 1
    P_ = np.empty(G + 1, np.int64)
    _load().orc_padded_offsets(_ptr(off), G, _ptr(P_))
    return P_


def quantize_mxfp8_colwise(x_bf16, group_offsets=None, ldT=None):
    """Columnwise copy stored transposed: (codesT u8 [K, ldT], scalesT u8 [K, ldT/32]).

    Ungrouped: ldT = M.  Grouped: ldT defaults to the padded total; columns
    past the padded total are left zero.
    """
    x = _c(x_bf16, np.uint16)
    M, K = x.shape
    if group_offsets is None:
        if M % 32:
            raise ValueError("an ungrouped columnwise copy needs M % 32 == 0 (whole 32-row blocks); "
                             "pass group_offsets to pad a group to 32 rows")
        ldT = M if ldT is None else ldT
        if ldT < M or ldT % 32:
            raise ValueError("ldT must be a multiple of 32 and at least M")
        off = None
        G = 1
    else:
        off = _c(group_offsets, np.int64)
        G = off.size - 1
        if ldT is None:
            ldT = int(padded_offsets(off)[-1])
    codesT = np.zeros((K, ldT), np.uint8)
    scalesT = np.zeros((K, ldT // 32), np.uint8)
    _load().orc_quantize_mxfp8_colwise(_ptr(x), M, K, _ptr(off), G, ldT, _ptr(codesT), _ptr(scalesT))
    return codesT, scalesT


def dequantize_mxfp8(codes, scales):
    codes = _c(codes, np.uint8)
    scales = _c(scales, np.uint8)
    M, K = codes.shape
    f = np.empty((M, K), np.float32)
    b = np.empty((M, K), np.uint16)
    _load().orc_dequantize_mxfp8(_ptr(codes), _ptr(scales), M, K, _ptr(f), _ptr(b))
    return f, b


# --- stochastic rounding / requant --------------------------------------------

def philox4x32_10(ctr, key):
    c = _c(ctr, np.uint32)
    k = _c(key, np.uint32)
    out = np.empty(4, np.uint32)
    _load().orc_philox4x32_10(_ptr(c), _ptr(k), _ptr(out))
    return out


def sr_bits(seed: int, index: int) -> int:
    return _load().orc_sr_bits(seed, index)


def e2m1_sr_mag(v: float, u: int) -> int:
    return _load().orc_e2m1_sr_mag(v, u)


def requant_transpose_sr(codes, scales, outer, seed: int = 0, use_sr: bool = True):
    """Rowwise NVFP4 [M,K] -> columnwise NVFP4 of the transpose [K,M] (codes, scales, G)."""
    codes = _c(codes, np.uint8)
    scales = _c(scales, np.uint8)
    outer = _c(outer, np.float32)
    M, K = codes.shape[0], codes.shape[1] * 2
    codesT = np.empty((K, M // 2), np.uint8)
    scalesT = np.empty((K, M // 16), np.uint8)
    G = np.empty(1, np.float32)
    _load().orc_requant_transpose_sr(_ptr(codes), _ptr(scales), _ptr(outer), M, K, seed, int(bool(use_sr)),
                                     _ptr(codesT), _ptr(scalesT), _ptr(G))
    return codesT, scalesT, G


def requant_transpose_sr_batched(codes, scales, outer, E: int, rows_per_scale: int, seed: int = 0,
                                 use_sr: bool = True):
    """E stacked rowwise NVFP4 tensors [E*M, K] -> each transposed and requantized
    on its own: (codesT [E*K, M/2], scalesT [E*K, M/16], G [E]); random bits of
    output element (e, k, m) at index e*K*M + k*M + m [nopree.com, section
    第二个决定, applied per expert tensor]."""
    codes = _c(codes, np.uint8)
    scales = _c(scales, np.uint8)
    outer = _c(outer, np.float32)
    M = codes.shape[0] // E
    K = codes.shape[1] * 2
    codesT = np.empty((E * K, M // 2), np.uint8)
    scalesT = np.empty((E * K, M // 16), np.uint8)
    G = np.empty(E, np.float32)
    _load().orc_requant_transpose_sr_batched(_ptr(codes), _ptr(scales), _ptr(outer), rows_per_scale, E, M, K, seed,
                                             int(bool(use_sr)), _ptr(codesT), _ptr(scalesT), _ptr(G))
    return codesT, scalesT, G


def requant_transpose_sr_grouped(codes, scales, outer, gather, group_offsets, ldT: int, seed: int = 0,
                                 use_sr: bool = True):
    """Rowwise NVFP4 rows [src_rows, K], grouped (rows [off[g], off[g+1]) read
    through gather) -> per group dequantized, transposed and requantized into
    32-padded columns of [K, ldT] with G_g per group: (codesT [K, ldT/2],
    scalesT [K, ldT/16], G [G]) [nopree.com, section 第二个决定, for the weight
    gradient's token-blocked operands]."""
    codes = _c(codes, np.uint8)
    scales = _c(scales, np.uint8)
    outer = _c(outer, np.float32)
    off = _c(group_offsets, np.int64)
    gather = None if gather is None else _c(gather, np.int32)
    G = off.size - 1
    K = codes.shape[1] * 2
    codesT = np.zeros((K, ldT // 2), np.uint8)
    scalesT = np.zeros((K, ldT // 16), np.uint8)
    Gs = np.empty(G, np.float32)
    _load().orc_requant_transpose_sr_grouped(_ptr(codes), _ptr(scales), _ptr(outer), codes.shape[0], _ptr(gather),
                                             _ptr(off), G, K, ldT, seed, int(bool(use_sr)), _ptr(codesT),
                                             _ptr(scalesT), _ptr(Gs))
    return codesT, scalesT, Gs


# --- GEMM -------------------------------------------------------------------

FMT_NVFP4 = 0
FMT_MXFP8 = 1


def gemm_rowgroup(fmt, a_codes, a_scales, a_outer, a_gather, group_offsets, N, K, b_codes, b_scales,
                  b_outer, rows=None):
    """Forward/dgrad form in binary64.  Returns (C [len(rows), N], sum|AB| [len(rows), N])."""
    off = _c(group_offsets, np.int64)
    G = off.size - 1
    M = int(off[-1])
    a_codes = _c(a_codes, np.uint8)
    a_scales = _c(a_scales, np.uint8)
    b_codes = _c(b_codes, np.uint8)
    b_scales = _c(b_scales, np.uint8)
    a_outer = None if a_outer is None else _c(a_outer, np.float32)
    b_outer = None if b_outer is None else _c(b_outer, np.float32)
    gather = None if a_gather is None else _c(a_gather, np.int32)
    rows_arr = None if rows is None else _c(rows, np.int64)
    n = M if rows is None else rows_arr.size
    c = np.empty((n, N), np.float64)
    cabs = np.empty((n, N), np.float64)
    _load().orc_gemm_rowgroup(fmt, _ptr(a_codes), _ptr(a_scales), _ptr(a_outer), _ptr(gather), _ptr(off), G, M,
                              N, K, _ptr(b_codes), _ptr(b_scales), _ptr(b_outer), _ptr(rows_arr), n, _ptr(c),
                              _ptr(cabs))
    return c, cabs


def gemm_wgrad_nvfp4(a_codesT, a_scalesT, a_outer, b_codesT, b_scalesT, b_outer, group_offsets, sel):
    """Weight-gradient form on grouped NVFP4 columnwise copies (outer scale per
    group and operand) in binary64, for the (g, n) pairs in sel."""
    a_codesT = _c(a_codesT, np.uint8)
    a_scalesT = _c(a_scalesT, np.uint8)
    b_codesT = _c(b_codesT, np.uint8)
    b_scalesT = _c(b_scalesT, np.uint8)
    a_outer = _c(a_outer, np.float32)
    b_outer = _c(b_outer, np.float32)
    off = _c(group_offsets, np.int64)
    G = off.size - 1
    NA, ldk = a_codesT.shape[0], a_codesT.shape[1] * 2
    NB = b_codesT.shape[0]
    sel = _c(sel, np.int64).reshape(-1, 2)
    c = np.empty((sel.shape[0], NB), np.float64)
    cabs = np.empty((sel.shape[0], NB), np.float64)
    _load().orc_gemm_wgrad_fmt(FMT_NVFP4, _ptr(a_codesT), _ptr(a_scalesT), _ptr(a_outer), _ptr(b_codesT),
                               _ptr(b_scalesT), _ptr(b_outer), _ptr(off), G, NA, NB, ldk, _ptr(sel), sel.shape[0],
                               _ptr(c), _ptr(cabs))
    return c, cabs


def gemm_wgrad(a_codesT, a_scalesT, b_codesT, b_scalesT, group_offsets, sel):
    """Weight-gradient form (MXFP8) in binary64 for the (g, n) pairs in sel."""
    a_codesT = _c(a_codesT, np.uint8)
    a_scalesT = _c(a_scalesT, np.uint8)
    b_codesT = _c(b_codesT, np.uint8)
    b_scalesT = _c(b_scalesT, np.uint8)
    off = _c(group_offsets, np.int64)
    G = off.size - 1
    NA, ldk = a_codesT.shape
    NB = b_codesT.shape[0]
    sel = _c(sel, np.int64).reshape(-1, 2)
    c = np.empty((sel.shape[0], NB), np.float64)
    cabs = np.empty((sel.shape[0], NB), np.float64)
    _load().orc_gemm_wgrad(_ptr(a_codesT), _ptr(a_scalesT), _ptr(b_codesT), _ptr(b_scalesT), _ptr(off), G, NA,
                           NB, ldk, _ptr(sel), sel.shape[0], _ptr(c), _ptr(cabs))
    return c, cabs


GEMM_FPROP = 0
GEMM_DGRAD = 1


def gemm_bf16_rowgroup(mode, a, b, gather, group_offsets, N, K, rows=None):
    """BF16 forward (mode 0, B [G, N, K]) or data-gradient (mode 1, B [G, K, N])
    form in binary64 on bf16 bit arrays; the backward GEMMs of the NVFP4 MoE
    layer in either mode [remio.ai, section "Entrambe le ricette supportano";
    alphasignal.ai, Recipe 2].  Returns (C [len(rows), N], sum|AB|)."""
    a = _c(a, np.uint16)
    b = _c(b, np.uint16)
    off = _c(group_offsets, np.int64)
    G = off.size - 1
    M = int(off[-1])
    gather = None if gather is None else _c(gather, np.int32)
    rows_arr = None if rows is None else _c(rows, np.int64)
    n = M if rows is None else rows_arr.size
    c = np.empty((n, N), np.float64)
    cabs = np.empty((n, N), np.float64)
    _load().orc_gemm_bf16_rowgroup(int(mode), _ptr(a), a.shape[1], a.shape[0], _ptr(b), b.shape[-1],
                                   _ptr(gather), _ptr(off), G, N, K, _ptr(rows_arr), n, _ptr(c), _ptr(cabs))
    return c, cabs


def gemm_bf16_wgrad(a, b, gather, group_offsets, sel):
    """BF16 weight-gradient form in binary64: C_g[m, n] = sum over the rows r of
    group g of A[r, m] * B[gather[r], n], for the (g, m) pairs in sel."""
    a = _c(a, np.uint16)
    b = _c(b, np.uint16)
    off = _c(group_offsets, np.int64)
    gather = None if gather is None else _c(gather, np.int32)
    sel = _c(sel, np.int64).reshape(-1, 2)
    N = b.shape[1]
    c = np.empty((sel.shape[0], N), np.float64)
    cabs = np.empty((sel.shape[0], N), np.float64)
    _load().orc_gemm_bf16_wgrad(_ptr(a), a.shape[1], _ptr(b), b.shape[1], _ptr(gather), b.shape[0], _ptr(off), N,
                                _ptr(sel), sel.shape[0], _ptr(c), _ptr(cabs))
    return c, cabs


# --- SwiGLU -------------------------------------------------------------------

def bf16_ulp_distance(a_bits: np.ndarray, b_bits: np.ndarray) -> np.ndarray:
    """Units in the last place between two bf16 arrays (bit patterns mapped to
    an ordered integer line, so +0 and -0 are one unit apart)."""
    def ordered(x):
        x = np.asarray(x, np.uint16).astype(np.int32)
        return np.where(x & 0x8000, 0x7FFF - (x & 0x7FFF), x + 0x8000)
    return np.abs(ordered(a_bits) - ordered(b_bits))


def swiglu(h13: np.ndarray) -> np.ndarray:
    """h13 f32 [R, 2I] -> h bf16 bits [R, I]: bf16(f32(silu(gate) * up)) with
    silu evaluated in binary64 (the pages give no SwiGLU arithmetic; this is
    the plain definition, independent of any kernel's exp)."""
    h13 = _c(h13, np.float32)
    R, I2 = h13.shape
    h = np.empty((R, I2 // 2), np.uint16)
    _load().orc_swiglu(_ptr(h13), R, I2 // 2, _ptr(h))
    return h
