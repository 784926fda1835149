"""The library's calls captured in a HIP graph give the eager results on every
replay.

bench.py times the short-step workloads (requant with stochastic rounding,
MXFP8 quantization) by graph replay, so each call it captures is checked
here: captured once, replayed several times with eager work, output clobbering
and synchronizations between the replays, and every replay compared byte for
byte with the eager call.
"""
import numpy as np
import pytest
import torch

from block_scaled_precision_token_amd import ops, synth
from tests.gpu_util import DEV, assert_bytes_equal, host, to_dev_bf16

pytestmark = pytest.mark.gpu

REPLAYS = 3


def _clobber(tensors):
    for t in tensors:
        t.fill_(0xAB if t.dtype == torch.uint8 else 1.0)


def test_graph_replays_match_eager():
    M, K = 512, 2048
    x = to_dev_bf16(synth.activations(20261211, M, K))
    x_other = to_dev_bf16(synth.activations(20261212, M, K))
    xn = ops.quantize_nvfp4_per_token(x)
    u8, f32 = torch.uint8, torch.float32
    emp = lambda *s, dt=u8: torch.empty(s, dtype=dt, device=DEV)

    # eager references
    mx_ref = ops.quantize_mxfp8(x, True, True)
    rq_ref = ops.requant_transpose_sr(*xn, seed=0x5EED, sr=True)
    torch.cuda.synchronize()
    mx_ref = {k: host(v) for k, v in mx_ref.items() if v is not None}
    rq_ref = [host(t) for t in rq_ref]

    mx_out = {"codes_row": emp(M, K), "scales_row": emp(M, K // 32), "codes_colT": emp(K, M),
              "scales_colT": emp(K, M // 32)}
    rq_out = (emp(K, M // 2), emp(K, M // 16), emp(4, dt=f32))
    ws = emp(ops.requant_workspace_size(M))
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        ops.quantize_mxfp8(x, True, True, out=mx_out)
        ops.requant_transpose_sr(*xn, seed=0x5EED, sr=True, workspace=ws, out=rq_out)
    torch.cuda.synchronize()

    for rep in range(REPLAYS):
        _clobber(list(mx_out.values()) + list(rq_out) + [ws])
        ops.quantize_mxfp8(x_other, True, True)        # unrelated eager work between replays
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for k, ref in mx_ref.items():
            assert_bytes_equal(host(mx_out[k]), ref, f"replay {rep} mxfp8 {k}")
        assert_bytes_equal(host(rq_out[0]), rq_ref[0], f"replay {rep} requant codes")
        assert_bytes_equal(host(rq_out[1]), rq_ref[1], f"replay {rep} requant scales")
        assert_bytes_equal(host(rq_out[2])[:1], rq_ref[2], f"replay {rep} requant outer")


def test_graph_replays_match_eager_gemm():
    """The grouped GEMM builds its tile list and scale planes in the workspace on
    every call; replays must rebuild them the same way."""
    R, K, N, G = 384, 512, 256, 3
    x = to_dev_bf16(synth.activations(20261213, R, K))
    w = to_dev_bf16(synth.weights(20261214, G, N, K).reshape(G * N, K))
    off = torch.tensor([0, 100, 100, R], dtype=torch.int64, device=DEV)
    xq = ops.quantize_mxfp8(x)
    wq = ops.quantize_mxfp8(w)
    ref = ops.moe_grouped_gemm_blockscaled(ops.FMT_MXFP8, ops.GEMM_FPROP, xq["codes_row"], xq["scales_row"],
                                           wq["codes_row"], wq["scales_row"], off, N, K)
    torch.cuda.synchronize()
    ref = host(ref)
    out = torch.empty((R, N), dtype=torch.float32, device=DEV)
    ws = torch.empty((ops.gemm_workspace_size(ops.FMT_MXFP8, ops.GEMM_FPROP, R, N, K, G),), dtype=torch.uint8,
                     device=DEV)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        ops.moe_grouped_gemm_blockscaled(ops.FMT_MXFP8, ops.GEMM_FPROP, xq["codes_row"], xq["scales_row"],
                                         wq["codes_row"], wq["scales_row"], off, N, K, out=out, workspace=ws)
    torch.cuda.synchronize()
    for rep in range(REPLAYS):
        _clobber([out, ws])
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        np.testing.assert_array_equal(host(out), ref, err_msg=f"replay {rep}")
