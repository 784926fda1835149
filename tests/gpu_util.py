"""Helpers shared by the GPU parity tests (host <-> device marshalling and the
GEMM tolerance)."""
import numpy as np
import torch

DEV = torch.device("cuda:0")


def to_dev_bf16(bits: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).to(DEV)


def to_dev(a: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a)).to(DEV)


def host(t: torch.Tensor) -> np.ndarray:
    torch.cuda.synchronize()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).cpu().numpy().view(np.uint16)
    return t.cpu().numpy()


def assert_bytes_equal(got, ref, what=""):
    got = np.asarray(got)
    ref = np.asarray(ref)
    assert got.shape == ref.shape, (what, got.shape, ref.shape)
    if got.dtype == np.float32:
        got = got.view(np.uint32)
        ref = ref.view(np.uint32)
    bad = np.argwhere(got != ref)
    assert bad.size == 0, f"{what}: {len(bad)} mismatches, first at {bad[:5].tolist()}: " \
                          f"got {got[tuple(bad[0])]} ref {ref[tuple(bad[0])]}"


def gemm_errors(c: np.ndarray, ref: np.ndarray, refabs: np.ndarray):
    """(max |C-R| / sum|a b|, max |C-R| / max |R|) -- the parity bound of the GEMM."""
    d = np.abs(c.astype(np.float64) - ref)
    norm = d / np.maximum(refabs, 1e-300)
    norm[refabs == 0] = d[refabs == 0]
    return float(norm.max()), float(d.max() / max(np.abs(ref).max(), 1e-300))


def assert_gemm_close(c, ref, refabs, bf16=False, tol=1e-3):
    c = np.asarray(c, dtype=np.float64)
    if bf16:
        # bf16 output adds its own relative rounding of 2^-9
        d = np.abs(c - ref)
        allowed = tol * refabs + 2.0 ** -8 * np.abs(ref) + 1e-300
        assert np.all(d <= allowed), float((d / allowed).max())
        return
    e_norm, e_wise = gemm_errors(c, ref, refabs)
    assert e_norm <= tol, e_norm
    assert e_wise <= tol, e_wise


def assert_swiglu_close(h_dev_bits, h13_f32):
    """Stage one of the SwiGLU contract: the device's bf16 h within one bf16 unit
    of the oracle's binary64 SwiGLU.  Both round a value that f32 arithmetic
    gets to a few f32 units, so they can straddle one bf16 rounding boundary
    but not two.  The one exception is f32's range: exp(-z) overflows f32 for
    z < -88.72, where an f32 evaluation of z / (1 + exp(-z)) gives -0 against
    a true magnitude below 89 e^-88.72 |up| < 3e-37 |up|; such elements may
    differ by that much instead."""
    import oracle
    h_ref = oracle.swiglu(h13_f32)
    dist = oracle.bf16_ulp_distance(h_dev_bits, h_ref)
    I = h_ref.shape[1]
    up = np.abs(h13_f32[:, I:].astype(np.float64))
    f = lambda b: (np.asarray(b, np.uint32) << 16).view(np.float32).astype(np.float64)
    absdiff = np.abs(f(h_dev_bits) - f(h_ref))
    ok = (dist <= 1) | (absdiff <= 3e-37 * up)
    bad = np.argwhere(~ok)
    assert bad.size == 0, f"h: {len(bad)} elements beyond one bf16 unit, first at {bad[:5].tolist()}"
