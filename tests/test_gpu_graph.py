"""The rollout step captured into a HIP graph: activation quantization and
FProp (block-scaled and MXFP8, on the row-major and on the packed decode
weight) recorded once, replayed on fresh
inputs with eager work and synchronizations between the replays, and every
replay compared bit for bit with the same calls made eagerly.  The entry
points launch kernels only (no allocation, no memset), so they can be
captured; the outputs are allocated before the capture."""
import pytest
import torch

import block_scaled_fp8_02_amd as fb
from block_scaled_fp8_02_amd import workloads as wl
from gpu_util import banner, dev

pytestmark = pytest.mark.gpu


def fresh_x(step: int, rows: int = 64, cols: int = 4096) -> torch.Tensor:
    rng = wl.rng_for(300 + step)
    x = wl.normal(rng, (rows, cols), 1.0)
    wl.add_outlier_channels(rng, x)
    return dev(wl.f32_to_bf16_bits(x))


@pytest.mark.parametrize("packed", [False, True])
@pytest.mark.parametrize("mx", [False, True])
def test_rollout_step_in_a_graph_matches_eager(mx, packed):
    w = wl.decode(0)
    M, C, D = 64, 4096, 24576
    banner(f"graph: {'MX' if mx else 'block-scaled'} quantize + FProp {M}x{D}x{C}"
           f"{' (packed weight)' if packed else ''}, 4 replays")
    wd = dev(w["W"])
    if mx:
        wq, ws, _, _ = fb.fp8_mx_quantize_1x32(wd, colwise=False)
        wp, wep = fb.fp8_pack_decode_weight(wq, D, C, we=ws) if packed else (None, None)
    else:
        wq, ws, _ = fb.fp8_quantize_weight_128x128(wd, transpose=False)
        wp, _ = fb.fp8_pack_decode_weight(wq, D, C) if packed else (None, None)
    x_static = fresh_x(0).clone()

    def step(x, q=None, s=None, y=None):
        if mx:
            q, s, _, _ = fb.fp8_mx_quantize_1x32(x, colwise=False, q=q, e=s)
            if packed:
                return q, s, fb.fp8_mx_gemm_fprop_decode(q, s, wp, wep, M, D, C, y=y)
            return q, s, fb.fp8_mx_gemm_fprop(q, s, wq, ws, M, D, C, y=y)
        q, s = fb.fp8_quantize_act_1x128(x, q=q, s=s)
        if packed:
            return q, s, fb.fp8_gemm_fprop_decode(q, s, wp, ws, M, D, C, y=y)
        return q, s, fb.fp8_gemm_fprop(q, s, wq, ws, M, D, C, y=y)

    # outputs allocated, and every kernel run once, before the capture
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        q, s, y = step(x_static)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()

    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step(x_static, q, s, y)
    torch.cuda.synchronize()
    for i in range(1, 5):
        x_new = fresh_x(i)
        x_static.copy_(x_new)                                          # eager work between replays
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        q_ref, s_ref, y_ref = step(x_new)
        torch.cuda.synchronize()
        assert torch.equal(q, q_ref), ("codes", i)
        assert torch.equal(s.view(torch.uint8), s_ref.view(torch.uint8)), ("scales", i)
        assert torch.equal(y, y_ref), ("output", i)
