"""Python binding of the C ABI in ``include/bsp.h`` (argument marshalling only).

Every function allocates its outputs as torch tensors on the input's device,
passes raw device pointers and the current HIP stream to ``libbsp.so`` and
returns the outputs; all computation happens in the library's kernels.  The
library is loaded on first use and a missing library raises -- there is no
fallback path.
"""
from __future__ import annotations

import ctypes
import os
import threading

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "lib", "libbsp.so")

FMT_NVFP4 = 0
FMT_MXFP8 = 1
DTYPE_F32 = 0
DTYPE_BF16 = 1
GEMM_FPROP = 0
GEMM_DGRAD = 1
GEMM_WGRAD = 2
NVFP4_46 = 0x1
SR = 0x2

STATUS = {0: "BSP_OK", 1: "BSP_ERR_INVALID_ARG", 2: "BSP_ERR_SHAPE", 3: "BSP_ERR_ALIGNMENT",
          4: "BSP_ERR_UNSUPPORTED", 5: "BSP_ERR_WORKSPACE", 6: "BSP_ERR_HIP", 7: "BSP_ERR_SCRATCH_LIMIT"}
GEMM_SCRATCH_BYTES = 64 << 20   # static device scratch of the allocation-free GEMM (BSP_GEMM_SCRATCH_BYTES)

EXPORTED = [
    "bsp_version", "bsp_status_string", "bsp_quantize_nvfp4_per_token", "bsp_quantize_mxfp8", "bsp_dequantize",
    "bsp_requant_transpose_sr", "bsp_moe_grouped_gemm_blockscaled", "bsp_swiglu_quantize", "bsp_nvfp4_sizes",
    "bsp_mxfp8_sizes", "bsp_mxfp8_grouped_cols", "bsp_requant_workspace_size", "bsp_gemm_workspace_size",
    "bsp_moe_grouped_gemm_bf16", "bsp_gemm_bf16_workspace_size", "bsp_requant_transpose_sr_batched",
    "bsp_requant_batched_workspace_size", "bsp_requant_transpose_sr_grouped", "bsp_quantize_nvfp4_rht",
    "bsp_quantize_nvfp4_2d", "bsp_moe_grouped_gemm_blockscaled_tiled", "bsp_moe_grouped_gemm_bf16_tiled",
    "bsp_moe_grouped_gemm_blockscaled_noalloc",
]


class BspError(RuntimeError):
    def __init__(self, status: int, fn: str):
        self.status = status
        super().__init__(f"{fn} failed: {STATUS.get(status, status)} ({_lib_raw().bsp_status_string(status).decode()})")


_lock = threading.Lock()
_lib = None

P = ctypes.c_void_p
I64 = ctypes.c_int64
U32 = ctypes.c_uint32
U64 = ctypes.c_uint64
SZ = ctypes.c_size_t
INT = ctypes.c_int


def _declare(lib):
    lib.bsp_version.restype = INT
    lib.bsp_status_string.argtypes = [INT]
    lib.bsp_status_string.restype = ctypes.c_char_p
    lib.bsp_quantize_nvfp4_per_token.argtypes = [P, I64, I64, I64, I64, P, P, P, U32, P]
    lib.bsp_quantize_nvfp4_rht.argtypes = [P, I64, I64, I64, U32, P, P, P, U32, P]
    lib.bsp_quantize_nvfp4_2d.argtypes = [P, I64, I64, I64, P, P, P, P]
    lib.bsp_quantize_mxfp8.argtypes = [P, I64, I64, I64, P, I64, I64, P, P, P, P, I64, P, I64, U32, P]
    lib.bsp_dequantize.argtypes = [INT, P, P, P, I64, I64, I64, P, INT, P]
    lib.bsp_requant_transpose_sr.argtypes = [P, P, P, I64, I64, P, P, P, U64, U32, P, SZ, P]
    lib.bsp_requant_transpose_sr_batched.argtypes = [P, P, P, I64, I64, I64, I64, P, P, P, U64, U32, P, SZ, P]
    lib.bsp_requant_batched_workspace_size.argtypes = [I64, I64, I64]
    lib.bsp_requant_transpose_sr_grouped.argtypes = [P, P, P, I64, P, P, I64, I64, I64, P, P, I64, P, U64, U32, P]
    lib.bsp_requant_batched_workspace_size.restype = SZ
    lib.bsp_moe_grouped_gemm_blockscaled.argtypes = [INT, INT, P, P, P, P, I64, P, I64, I64, I64, I64, P, P, P, P,
                                                     INT, I64, P, SZ, P]
    lib.bsp_moe_grouped_gemm_bf16.argtypes = [INT, P, I64, P, I64, P, I64, P, I64, I64, I64, I64, P, INT, I64, P,
                                              SZ, P]
    lib.bsp_moe_grouped_gemm_blockscaled_tiled.argtypes = lib.bsp_moe_grouped_gemm_blockscaled.argtypes[:-1] + [INT, P]
    lib.bsp_moe_grouped_gemm_bf16_tiled.argtypes = lib.bsp_moe_grouped_gemm_bf16.argtypes[:-1] + [INT, P]
    lib.bsp_moe_grouped_gemm_blockscaled_noalloc.argtypes = lib.bsp_moe_grouped_gemm_blockscaled.argtypes[:18] + [P]
    lib.bsp_gemm_bf16_workspace_size.argtypes = [INT, I64, I64, I64, I64]
    lib.bsp_gemm_bf16_workspace_size.restype = SZ
    lib.bsp_swiglu_quantize.argtypes = [P, INT, I64, I64, P, INT, P, P, P, U32, P]
    lib.bsp_nvfp4_sizes.argtypes = [I64, I64, I64, ctypes.POINTER(SZ), ctypes.POINTER(SZ), ctypes.POINTER(SZ)]
    lib.bsp_mxfp8_sizes.argtypes = [I64, I64, ctypes.POINTER(SZ), ctypes.POINTER(SZ)]
    lib.bsp_mxfp8_grouped_cols.argtypes = [I64, I64]
    lib.bsp_mxfp8_grouped_cols.restype = I64
    lib.bsp_requant_workspace_size.argtypes = [I64]
    lib.bsp_requant_workspace_size.restype = SZ
    lib.bsp_gemm_workspace_size.argtypes = [INT, INT, I64, I64, I64, I64]
    lib.bsp_gemm_workspace_size.restype = SZ
    for name in ("bsp_quantize_nvfp4_per_token", "bsp_quantize_mxfp8", "bsp_dequantize", "bsp_requant_transpose_sr",
                 "bsp_moe_grouped_gemm_blockscaled", "bsp_swiglu_quantize", "bsp_nvfp4_sizes", "bsp_mxfp8_sizes",
                 "bsp_moe_grouped_gemm_bf16", "bsp_requant_transpose_sr_batched", "bsp_requant_transpose_sr_grouped",
                 "bsp_quantize_nvfp4_rht", "bsp_quantize_nvfp4_2d", "bsp_moe_grouped_gemm_blockscaled_tiled",
                 "bsp_moe_grouped_gemm_bf16_tiled", "bsp_moe_grouped_gemm_blockscaled_noalloc"):
        getattr(lib, name).restype = INT


def _lib_raw():
    """Load libbsp.so (raises if it has not been built)."""
    global _lib
    with _lock:
        if _lib is None:
            if not os.path.exists(LIB_PATH):
                raise RuntimeError(f"HIP library not built: {LIB_PATH} is missing "
                                   "(run `python -c 'import __graft_entry__ as g; g.build()'`)")
            lib = ctypes.CDLL(LIB_PATH)
            _declare(lib)
            _lib = lib
    return _lib


lib = _lib_raw


def _check(status: int, fn: str):
    if status != 0:
        raise BspError(status, fn)


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(device):
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


# Device type the tensor arguments must live on.  The CPU tests of the
# argument checks rebind it (with the library stubbed out) so that the checks
# can be exercised without a GPU; nothing is launched on that path.
DEVICE_TYPE = "cuda"

_DT = {"u8": torch.uint8, "bf16": torch.bfloat16, "f32": torch.float32, "i32": torch.int32, "i64": torch.int64}


def _need_cuda(t, name):
    if not isinstance(t, torch.Tensor) or t.device.type != DEVICE_TYPE:
        raise ValueError(f"{name} must be a device tensor")


def _rowmajor(t, name):
    if t.dim() != 2 or t.stride(1) != 1:
        raise ValueError(f"{name} must be a 2-D tensor with unit column stride")


def _arg(t, name, dev, dtype, numel=None, optional=False, contiguous=True):
    """Check one tensor argument before its pointer goes to the library: a
    device tensor on `dev` of the given dtype ("u8", "bf16", "f32", "i32",
    "i64" or a tuple of them), contiguous, with at least `numel` elements.
    Raises ValueError; returns t."""
    if t is None:
        if optional:
            return None
        raise ValueError(f"{name} is required")
    _need_cuda(t, name)
    if t.device != dev:
        raise ValueError(f"{name} is on {t.device}, expected {dev}")
    kinds = dtype if isinstance(dtype, tuple) else (dtype,)
    if t.dtype not in tuple(_DT[k] for k in kinds):
        raise ValueError(f"{name} must have dtype {' or '.join(kinds)}, not {t.dtype}")
    if contiguous and not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if numel is not None and t.numel() < numel:
        raise ValueError(f"{name} has {t.numel()} elements, needs at least {int(numel)}")
    return t


def _rows_arg(t, name, dev, dtype, cols):
    """A 2-D operand read row by row with its row stride: unit column stride,
    at least `cols` columns, 16-byte aligned rows."""
    _arg(t, name, dev, dtype, contiguous=False)
    _rowmajor(t, name)
    if t.shape[1] < cols:
        raise ValueError(f"{name} has {t.shape[1]} columns, needs {cols}")
    return t


def _offsets_arg(off, dev):
    _arg(off, "group_offsets", dev, "i64")
    if off.dim() != 1 or off.numel() < 2:
        raise ValueError("group_offsets must be a 1-D int64 tensor of G + 1 >= 2 entries")
    return off.numel() - 1


# ---------------------------------------------------------------------------
# ops
# ---------------------------------------------------------------------------

def _x_arg(x, name="x"):
    """The bf16 input of a quantizer: a 2-D device tensor with unit column stride."""
    _need_cuda(x, name)
    _rowmajor(x, name)
    if x.dtype != torch.bfloat16:
        raise ValueError(f"{name} must be bfloat16")
    return x


def quantize_nvfp4_per_token(x: torch.Tensor, rows_per_scale: int = 1, mode46: bool = False, out=None):
    """bf16 [M, K] -> (codes u8 [M, K/2], scales u8 [M, K/16], outer f32 [M / rows_per_scale])."""
    _x_arg(x)
    M, K = x.shape
    dev = x.device
    nscope = max(M // max(rows_per_scale, 1), 1)
    if out is None:
        codes = torch.empty((M, K // 2), dtype=torch.uint8, device=dev)
        scales = torch.empty((M, K // 16), dtype=torch.uint8, device=dev)
        outer = torch.empty((nscope,), dtype=torch.float32, device=dev)
    else:
        codes, scales, outer = out
        _arg(codes, "codes", dev, "u8", M * (K // 2))
        _arg(scales, "scales", dev, "u8", M * (K // 16))
        _arg(outer, "outer", dev, "f32", nscope)
    flags = NVFP4_46 if mode46 else 0
    st = _lib_raw().bsp_quantize_nvfp4_per_token(_ptr(x), M, K, x.stride(0), rows_per_scale, _ptr(codes),
                                                 _ptr(scales), _ptr(outer), flags, _stream(dev))
    _check(st, "bsp_quantize_nvfp4_per_token")
    return codes, scales, outer


def mxfp8_grouped_cols(M: int, G: int) -> int:
    return int(_lib_raw().bsp_mxfp8_grouped_cols(M, G))


def quantize_mxfp8(x: torch.Tensor, rowwise: bool = True, colwise: bool = False, group_offsets=None,
                   ld_colT: int | None = None, row_gather=None, out=None):
    """bf16 [x_rows, K] (or a stack [batch, x_rows, K]) -> dict with 'codes_row' [M,K],
    'scales_row' [M,K/32], 'codes_colT' [K,ld], 'scales_colT' [K,ld/32] (each with the
    leading batch dimension for a stack).

    M = x_rows, or the length of row_gather (row r is then x[row_gather[r]]).
    """
    _need_cuda(x, "x")
    if x.dtype != torch.bfloat16:
        raise ValueError("x must be bfloat16")
    batch = 1
    if x.dim() == 3:
        if not x.is_contiguous():
            raise ValueError("a stacked x must be contiguous")
        batch = x.shape[0]
        x2 = x[0]
    else:
        _rowmajor(x, "x")
        x2 = x
    x_rows, K = x2.shape
    dev = x.device
    if row_gather is not None:
        _arg(row_gather, "row_gather", dev, "i32")
    M = x_rows if row_gather is None else row_gather.numel()
    G = 0 if group_offsets is None else _offsets_arg(group_offsets, dev)
    lead = (batch,) if x.dim() == 3 else ()
    res = {"codes_row": None, "scales_row": None, "codes_colT": None, "scales_colT": None}
    if out is not None:
        res.update(out)
    else:
        if rowwise:
            res["codes_row"] = torch.empty(lead + (M, K), dtype=torch.uint8, device=dev)
            res["scales_row"] = torch.empty(lead + (M, K // 32), dtype=torch.uint8, device=dev)
        if colwise:
            if ld_colT is None:
                ld_colT = M if group_offsets is None else mxfp8_grouped_cols(M, G)
            res["codes_colT"] = torch.empty(lead + (K, ld_colT), dtype=torch.uint8, device=dev)
            res["scales_colT"] = torch.empty(lead + (K, ld_colT // 32), dtype=torch.uint8, device=dev)
    if res["codes_row"] is not None or res["scales_row"] is not None:
        _arg(res["codes_row"], "codes_row", dev, "u8", batch * M * K)
        _arg(res["scales_row"], "scales_row", dev, "u8", batch * M * (K // 32))
    if res["codes_colT"] is not None or res["scales_colT"] is not None:
        _arg(res["codes_colT"], "codes_colT", dev, "u8")
        ld_colT = res["codes_colT"].shape[-1]
        _arg(res["codes_colT"], "codes_colT", dev, "u8", batch * K * ld_colT)
        _arg(res["scales_colT"], "scales_colT", dev, "u8", batch * K * (ld_colT // 32))
    st = _lib_raw().bsp_quantize_mxfp8(_ptr(x), x_rows, K, x2.stride(0), _ptr(row_gather), M, batch,
                                       _ptr(res["codes_row"]),
                                       _ptr(res["scales_row"]), _ptr(res["codes_colT"]), _ptr(res["scales_colT"]),
                                       ld_colT or 0, _ptr(group_offsets), G, 0, _stream(dev))
    _check(st, "bsp_quantize_mxfp8")
    return res


def _nvfp4_out(out, M, K, nouter, dev):
    if out is None:
        return (torch.empty((M, K // 2), dtype=torch.uint8, device=dev),
                torch.empty((M, K // 16), dtype=torch.uint8, device=dev),
                torch.empty((nouter,), dtype=torch.float32, device=dev))
    codes, scales, outer = out
    _arg(codes, "codes", dev, "u8", M * (K // 2))
    _arg(scales, "scales", dev, "u8", M * (K // 16))
    _arg(outer, "outer", dev, "f32", nouter)
    return out


def quantize_nvfp4_rht(x: torch.Tensor, signs: int, mode46: bool = False, out=None):
    """bf16 [M, K] -> per-token NVFP4 of the 16-point-RHT'd rows (codes, scales, outer [M])."""
    _x_arg(x)
    M, K = x.shape
    dev = x.device
    codes, scales, outer = out = _nvfp4_out(out, M, K, M, dev)
    st = _lib_raw().bsp_quantize_nvfp4_rht(_ptr(x), M, K, x.stride(0), signs, _ptr(codes), _ptr(scales), _ptr(outer),
                                           NVFP4_46 if mode46 else 0, _stream(dev))
    _check(st, "bsp_quantize_nvfp4_rht")
    return codes, scales, outer


def quantize_nvfp4_2d(x: torch.Tensor, out=None):
    """bf16 [M, K] -> NVFP4 with 16x16 block scales (codes [M, K/2], scales [M/16, K/16], outer [1])."""
    _x_arg(x)
    M, K = x.shape
    dev = x.device
    if out is None:
        out = (torch.empty((M, K // 2), dtype=torch.uint8, device=dev),
               torch.empty((M // 16, K // 16), dtype=torch.uint8, device=dev),
               torch.empty((4,), dtype=torch.float32, device=dev))
    codes, scales, outer = out
    _arg(codes, "codes", dev, "u8", M * (K // 2))
    _arg(scales, "scales", dev, "u8", (M // 16) * (K // 16))
    _arg(outer, "outer", dev, "f32", 1)
    st = _lib_raw().bsp_quantize_nvfp4_2d(_ptr(x), M, K, x.stride(0), _ptr(codes), _ptr(scales), _ptr(outer),
                                          _stream(dev))
    _check(st, "bsp_quantize_nvfp4_2d")
    return codes, scales, outer


def dequantize(fmt: int, codes, scales, outer=None, rows_per_scale: int = 1, out_dtype=torch.float32, out=None):
    _arg(codes, "codes", codes.device if isinstance(codes, torch.Tensor) else None, "u8")
    if codes.dim() != 2:
        raise ValueError("codes must be 2-D [M, K/2] (NVFP4) or [M, K] (MXFP8)")
    dev = codes.device
    M = codes.shape[0]
    K = codes.shape[1] * (2 if fmt == FMT_NVFP4 else 1)
    _arg(scales, "scales", dev, "u8", M * (K // (16 if fmt == FMT_NVFP4 else 32)))
    if fmt == FMT_NVFP4:
        _arg(outer, "outer", dev, "f32", M // max(rows_per_scale, 1))
    if out is None:
        out = torch.empty((M, K), dtype=out_dtype, device=dev)
    _arg(out, "out", dev, ("f32", "bf16"), M * K)
    dt = DTYPE_BF16 if out.dtype == torch.bfloat16 else DTYPE_F32
    st = _lib_raw().bsp_dequantize(fmt, _ptr(codes), _ptr(scales), _ptr(outer), M, K, rows_per_scale, _ptr(out), dt,
                                   _stream(dev))
    _check(st, "bsp_dequantize")
    return out


def requant_workspace_size(M: int) -> int:
    return int(_lib_raw().bsp_requant_workspace_size(M))


def requant_batched_workspace_size(E: int, M: int, rows_per_scale: int) -> int:
    return int(_lib_raw().bsp_requant_batched_workspace_size(E, M, rows_per_scale))


def _nvfp4_in(codes, scales, outer, nouter):
    """Rowwise NVFP4 operand [rows, K/2] + [rows, K/16] + f32 [nouter]."""
    _arg(codes, "codes", codes.device if isinstance(codes, torch.Tensor) else None, "u8")
    if codes.dim() != 2:
        raise ValueError("codes must be 2-D [rows, K/2]")
    dev = codes.device
    rows, K = codes.shape[0], codes.shape[1] * 2
    _arg(scales, "scales", dev, "u8", rows * (K // 16))
    _arg(outer, "outer", dev, "f32", nouter(rows))
    return dev, rows, K


def requant_transpose_sr_batched(codes, scales, outer, E: int, rows_per_scale: int, seed: int = 0, sr: bool = True,
                                 workspace=None, out=None):
    """E stacked rowwise NVFP4 tensors [E*M, K] -> (codesT [E*K, M/2], scalesT [E*K, M/16], outerT [E])."""
    dev, EM, K = _nvfp4_in(codes, scales, outer, lambda r: r // max(rows_per_scale, 1))
    M = EM // E
    if out is None:
        out = (torch.empty((E * K, M // 2), dtype=torch.uint8, device=dev),
               torch.empty((E * K, M // 16), dtype=torch.uint8, device=dev),
               torch.empty((max(E, 4),), dtype=torch.float32, device=dev))
    codesT, scalesT, outerT = out
    _arg(codesT, "codesT", dev, "u8", E * K * (M // 2))
    _arg(scalesT, "scalesT", dev, "u8", E * K * (M // 16))
    _arg(outerT, "outerT", dev, "f32", E)
    need = requant_batched_workspace_size(E, M, rows_per_scale)
    if workspace is None:
        workspace = torch.empty((max(need, 16),), dtype=torch.uint8, device=dev)
    _arg(workspace, "workspace", dev, "u8", need)
    st = _lib_raw().bsp_requant_transpose_sr_batched(_ptr(codes), _ptr(scales), _ptr(outer), rows_per_scale, E, M, K,
                                                     _ptr(codesT), _ptr(scalesT), _ptr(outerT), seed, SR if sr else 0,
                                                     _ptr(workspace), workspace.numel(), _stream(dev))
    _check(st, "bsp_requant_transpose_sr_batched")
    return codesT, scalesT, outerT


def requant_transpose_sr_grouped(codes, scales, outer, group_offsets, R: int, ldT: int | None = None, gather=None,
                                 seed: int = 0, sr: bool = True, out=None):
    """Rowwise NVFP4 [src_rows, K] grouped through `gather` -> (codesT [K, ldT/2],
    scalesT [K, ldT/16], outerT [G]); columns past the padded total untouched
    (zero when allocated here)."""
    dev, src_rows, K = _nvfp4_in(codes, scales, outer, lambda r: r)
    G = _offsets_arg(group_offsets, dev)
    _arg(gather, "gather", dev, "i32", R, optional=True)
    if ldT is None:
        ldT = mxfp8_grouped_cols(R, G)
    if out is None:
        out = (torch.zeros((K, ldT // 2), dtype=torch.uint8, device=dev),
               torch.zeros((K, ldT // 16), dtype=torch.uint8, device=dev),
               torch.empty((max(G, 4),), dtype=torch.float32, device=dev))
    codesT, scalesT, outerT = out
    _arg(codesT, "codesT", dev, "u8", K * (ldT // 2))
    _arg(scalesT, "scalesT", dev, "u8", K * (ldT // 16))
    _arg(outerT, "outerT", dev, "f32", G)
    st = _lib_raw().bsp_requant_transpose_sr_grouped(_ptr(codes), _ptr(scales), _ptr(outer), src_rows, _ptr(gather),
                                                     _ptr(group_offsets), G, R, K, _ptr(codesT), _ptr(scalesT), ldT,
                                                     _ptr(outerT), seed, SR if sr else 0, _stream(dev))
    _check(st, "bsp_requant_transpose_sr_grouped")
    return codesT, scalesT, outerT


def requant_transpose_sr(codes, scales, outer, seed: int = 0, sr: bool = True, workspace=None, out=None):
    """Rowwise NVFP4 [M, K] -> (codesT [K, M/2], scalesT [K, M/16], outerT [1])."""
    dev, M, K = _nvfp4_in(codes, scales, outer, lambda r: r)
    if out is None:
        codesT = torch.empty((K, M // 2), dtype=torch.uint8, device=dev)
        scalesT = torch.empty((K, M // 16), dtype=torch.uint8, device=dev)
        outerT = torch.empty((4,), dtype=torch.float32, device=dev)
    else:
        codesT, scalesT, outerT = out
    _arg(codesT, "codesT", dev, "u8", K * (M // 2))
    _arg(scalesT, "scalesT", dev, "u8", K * (M // 16))
    _arg(outerT, "outerT", dev, "f32", 1)
    need = requant_workspace_size(M)
    if workspace is None:
        workspace = torch.empty((max(need, 16),), dtype=torch.uint8, device=dev)
    _arg(workspace, "workspace", dev, "u8", need)
    st = _lib_raw().bsp_requant_transpose_sr(_ptr(codes), _ptr(scales), _ptr(outer), M, K, _ptr(codesT),
                                             _ptr(scalesT), _ptr(outerT), seed & (2 ** 64 - 1), SR if sr else 0,
                                             _ptr(workspace), workspace.numel(), _stream(dev))
    _check(st, "bsp_requant_transpose_sr")
    return codesT, scalesT, outerT[:1]


def gemm_workspace_size(fmt: int, mode: int, M: int, N: int, K: int, G: int) -> int:
    """Bytes of device workspace for one grouped GEMM call of these sizes."""
    return int(_lib_raw().bsp_gemm_workspace_size(fmt, mode, M, N, K, G))


def _gemm_blockscaled_args(fmt, mode, a_codes, a_scales, b_codes, b_scales, group_offsets, N, K, M, a_outer,
                           b_outer, a_gather, out_dtype, out):
    """Checks and output allocation shared by the grouped GEMM wrappers; returns
    (device, G, M, a_rows, out, ldc, c_dtype)."""
    _arg(a_codes, "a_codes", a_codes.device if isinstance(a_codes, torch.Tensor) else None, "u8")
    dev = a_codes.device
    G = _offsets_arg(group_offsets, dev)
    if a_codes.dim() != 2:
        raise ValueError("a_codes must be 2-D")
    a_rows = a_codes.shape[0]
    wg = mode == GEMM_WGRAD
    nv = fmt == FMT_NVFP4
    rowb = K // 2 if nv else K                      # code bytes per operand row
    sblk = 16 if nv else 32
    if a_codes.shape[1] * (2 if nv else 1) != K:
        raise ValueError(f"a_codes has {a_codes.shape[1]} bytes per row, K = {K} needs {rowb}")
    _arg(a_gather, "a_gather", dev, "i32", optional=True)
    if M is None:
        M = a_gather.numel() if a_gather is not None else a_rows
    if a_gather is not None and a_gather.numel() < M:
        raise ValueError(f"a_gather has {a_gather.numel()} entries, needs {M}")
    _arg(a_scales, "a_scales", dev, "u8", a_rows * (K // sblk))
    nb_rows = N if wg else G * N                    # rows of B
    _arg(b_codes, "b_codes", dev, "u8", nb_rows * rowb)
    _arg(b_scales, "b_scales", dev, "u8", nb_rows * (K // sblk))
    if nv:
        _arg(a_outer, "a_outer", dev, "f32", G if wg else a_rows)
        _arg(b_outer, "b_outer", dev, "f32", G)
    elif a_outer is not None or b_outer is not None:
        raise ValueError("MXFP8 takes no outer scales")
    if out is None:
        out = torch.empty((G, M, N) if wg else (M, N), dtype=out_dtype, device=dev)
    _arg(out, "out", dev, ("f32", "bf16"))
    ldc = out.shape[-1] if out.dim() >= 2 else N
    if ldc < N:
        raise ValueError(f"out has rows of {ldc} elements, fewer than the {N} columns of C")
    _arg(out, "out", dev, ("f32", "bf16"), (G * M if wg else M) * ldc)
    dt = DTYPE_BF16 if out.dtype == torch.bfloat16 else DTYPE_F32
    return dev, G, M, a_rows, out, ldc, dt


def moe_grouped_gemm_blockscaled(fmt: int, mode: int, a_codes, a_scales, b_codes, b_scales, group_offsets, N: int,
                                 K: int, M: int | None = None, a_outer=None, b_outer=None, a_gather=None,
                                 out_dtype=torch.float32, out=None, workspace=None, tile: int = 0):
    """Grouped block-scaled GEMM; see bsp_moe_grouped_gemm_blockscaled in include/bsp.h.

    FPROP/DGRAD: C [M, N] with M = rows of C (grouped rows).  WGRAD: C [G, M, N]
    with M = rows of A (the columnwise copies' K dimension is their ld).
    tile: 0 (the library's choice), 128 or 256.
    """
    dev, G, M, a_rows, out, ldc, dt = _gemm_blockscaled_args(fmt, mode, a_codes, a_scales, b_codes, b_scales,
                                                             group_offsets, N, K, M, a_outer, b_outer, a_gather,
                                                             out_dtype, out)
    need = gemm_workspace_size(fmt, mode, M, N, K, G)
    if workspace is None:
        workspace = torch.empty((max(need, 16),), dtype=torch.uint8, device=dev)
    _arg(workspace, "workspace", dev, "u8", need)
    args = (fmt, mode, _ptr(a_codes), _ptr(a_scales), _ptr(a_outer), _ptr(a_gather), a_rows, _ptr(group_offsets), G,
            M, N, K, _ptr(b_codes), _ptr(b_scales), _ptr(b_outer), _ptr(out), dt, ldc, _ptr(workspace),
            workspace.numel())
    if tile:
        st = _lib_raw().bsp_moe_grouped_gemm_blockscaled_tiled(*args, tile, _stream(dev))
    else:
        st = _lib_raw().bsp_moe_grouped_gemm_blockscaled(*args, _stream(dev))
    _check(st, "bsp_moe_grouped_gemm_blockscaled")
    return out


def moe_grouped_gemm_blockscaled_noalloc(fmt: int, mode: int, a_codes, a_scales, b_codes, b_scales, group_offsets,
                                         N: int, K: int, M: int | None = None, a_outer=None, b_outer=None,
                                         a_gather=None, out=None):
    """The allocation-free grouped GEMM (bsp_moe_grouped_gemm_blockscaled_noalloc):
    no workspace, and `out` must be given -- nothing is allocated on this path.
    Problems whose workspace exceeds GEMM_SCRATCH_BYTES raise BspError
    (BSP_ERR_SCRATCH_LIMIT).  Calls that overlap on one GPU race."""
    if out is None:
        raise ValueError("out is required: the allocation-free call allocates nothing")
    dev, G, M, a_rows, out, ldc, dt = _gemm_blockscaled_args(fmt, mode, a_codes, a_scales, b_codes, b_scales,
                                                             group_offsets, N, K, M, a_outer, b_outer, a_gather,
                                                             None, out)
    st = _lib_raw().bsp_moe_grouped_gemm_blockscaled_noalloc(
        fmt, mode, _ptr(a_codes), _ptr(a_scales), _ptr(a_outer), _ptr(a_gather), a_rows, _ptr(group_offsets), G, M,
        N, K, _ptr(b_codes), _ptr(b_scales), _ptr(b_outer), _ptr(out), dt, ldc, _stream(dev))
    _check(st, "bsp_moe_grouped_gemm_blockscaled_noalloc")
    return out


def gemm_bf16_workspace_size(mode: int, M: int, N: int, K: int, G: int) -> int:
    return _lib_raw().bsp_gemm_bf16_workspace_size(mode, M, N, K, G)


def moe_grouped_gemm_bf16(mode: int, a: torch.Tensor, b: torch.Tensor, group_offsets, N: int, K: int,
                          M: int | None = None, gather=None, out_dtype=torch.float32, out=None, workspace=None,
                          tile: int = 0):
    """BF16 grouped GEMM; see bsp_moe_grouped_gemm_bf16 in include/bsp.h.

    FPROP: a [src_rows, K], b [G*N, K] (or [G, N, K]); DGRAD: b [G*K, N] (or
    [G, K, N]); C [M, N] with M = rows of C (gather length, else a's rows).
    WGRAD: a [K, M] (K = grouped rows), b [src_rows, N]; C [G, M, N].
    tile: 0 (the library's choice), 128 or 256.
    """
    _arg(a, "a", a.device if isinstance(a, torch.Tensor) else None, "bf16", contiguous=False)
    _rowmajor(a, "a")
    dev = a.device
    G = _offsets_arg(group_offsets, dev)
    _arg(b, "b", dev, "bf16")
    lda, ldb = a.stride(0), b.shape[-1]
    _arg(gather, "gather", dev, "i32", optional=True)
    if mode == GEMM_WGRAD:
        M = a.shape[1] if M is None else M
        src_rows = b.shape[0] if b.dim() == 2 else b.numel() // ldb
        if a.shape[0] < K:
            raise ValueError(f"a has {a.shape[0]} rows, needs K = {K}")
        if gather is not None and gather.numel() < K:
            raise ValueError(f"gather has {gather.numel()} entries, needs {K}")
        b_need = src_rows * ldb
    else:
        src_rows = a.shape[0]
        if M is None:
            M = gather.numel() if gather is not None else src_rows
        if gather is not None and gather.numel() < M:
            raise ValueError(f"gather has {gather.numel()} entries, needs {M}")
        b_need = G * (N if mode == GEMM_FPROP else K) * ldb
    _arg(b, "b", dev, "bf16", b_need)
    if out is None:
        shape = (G, M, N) if mode == GEMM_WGRAD else (M, N)
        out = torch.empty(shape, dtype=out_dtype, device=dev)
    _arg(out, "out", dev, ("f32", "bf16"))
    ldc = out.shape[-1]
    if ldc < N:
        raise ValueError(f"out has rows of {ldc} elements, fewer than the {N} columns of C")
    _arg(out, "out", dev, ("f32", "bf16"), (G * M if mode == GEMM_WGRAD else M) * ldc)
    dt = DTYPE_BF16 if out.dtype == torch.bfloat16 else DTYPE_F32
    need = gemm_bf16_workspace_size(mode, M, N, K, G)
    if workspace is None:
        workspace = torch.empty((max(need, 16),), dtype=torch.uint8, device=dev)
    _arg(workspace, "workspace", dev, "u8", need)
    args = (mode, _ptr(a), lda, _ptr(b), ldb, _ptr(gather), src_rows, _ptr(group_offsets), G, M, N, K, _ptr(out), dt,
            ldc, _ptr(workspace), workspace.numel())
    if tile:
        st = _lib_raw().bsp_moe_grouped_gemm_bf16_tiled(*args, tile, _stream(dev))
    else:
        st = _lib_raw().bsp_moe_grouped_gemm_bf16(*args, _stream(dev))
    _check(st, "bsp_moe_grouped_gemm_bf16")
    return out


def swiglu_quantize(h13: torch.Tensor, fmt: int = -1, mode46: bool = False, return_h: bool = True, out=None):
    """h13 [R, 2I] (f32 or bf16) -> (h bf16 [R, I] or None, codes, scales, outer)."""
    _arg(h13, "h13", h13.device if isinstance(h13, torch.Tensor) else None, ("f32", "bf16"))
    if h13.dim() != 2:
        raise ValueError("h13 must be 2-D [R, 2I]")
    R, I2 = h13.shape
    I = I2 // 2
    dev = h13.device
    h = codes = scales = outer = None
    if out is not None:
        h, codes, scales, outer = out
    else:
        if return_h or fmt < 0:
            h = torch.empty((R, I), dtype=torch.bfloat16, device=dev)
        if fmt == FMT_NVFP4:
            codes = torch.empty((R, I // 2), dtype=torch.uint8, device=dev)
            scales = torch.empty((R, I // 16), dtype=torch.uint8, device=dev)
            outer = torch.empty((R,), dtype=torch.float32, device=dev)
        elif fmt == FMT_MXFP8:
            codes = torch.empty((R, I), dtype=torch.uint8, device=dev)
            scales = torch.empty((R, I // 32), dtype=torch.uint8, device=dev)
    _arg(h, "h", dev, "bf16", R * I, optional=fmt >= 0)
    if fmt >= 0:
        nv = fmt == FMT_NVFP4
        _arg(codes, "codes", dev, "u8", R * (I // 2 if nv else I))
        _arg(scales, "scales", dev, "u8", R * (I // (16 if nv else 32)))
        _arg(outer, "outer", dev, "f32", R, optional=not nv)
    dt = DTYPE_BF16 if h13.dtype == torch.bfloat16 else DTYPE_F32
    st = _lib_raw().bsp_swiglu_quantize(_ptr(h13), dt, R, I, _ptr(h), fmt, _ptr(codes), _ptr(scales), _ptr(outer),
                                        NVFP4_46 if mode46 else 0, _stream(dev))
    _check(st, "bsp_swiglu_quantize")
    return h, codes, scales, outer
