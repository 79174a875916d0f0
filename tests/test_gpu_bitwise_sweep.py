"""GPU sweep: every tile width and the persistent loop give the same bits,
call after call, over a spread of shapes in both precisions.

The per-product launches at each forced width (64, 128, 256 where the padded
sides allow it) and the persistent loop accumulate every 32 x 32 output block
with the same MFMA sequence and finish it with the same epilogue arithmetic,
so their results are bitwise equal; repeating each call also catches a
result that depends on timing.  ACCURATE keeps the lo planes of B' and X,
which expose fp32-level differences that bf16 rounding would hide.  Shapes:
the metric batch, the attn view, the 124M mlp wave (22 blocks, not a
multiple of the 8 queues), 96 x 768^2, the GPT-2-medium blocks, large square
and tall blocks, ragged sides padded to 128, and single 4096^2 blocks.
"""
import numpy as np
import pytest

import workloads
from parity import torch_bf16_to_bits

pytestmark = pytest.mark.gpu

SHAPES = [(32, 768, 3072, 1), (8, 768, 3072, 4), (22, 768, 3072, 1), (96, 768, 768, 1), (16, 1024, 4096, 1),
          (4, 2048, 2048, 1), (12, 512, 1536, 1), (8, 1280, 1280, 1), (3, 2048, 768, 1), (64, 256, 1024, 1),
          (5, 300, 700, 1), (4, 1000, 260, 1), (6, 384, 1280, 1), (2, 1536, 4608, 1), (10, 640, 1920, 1),
          (3, 4096, 1024, 1), (1, 4096, 4096, 1)]


@pytest.fixture(scope="module")
def nsm():
    import torch
    if not torch.cuda.is_available():
        pytest.fail("no GPU visible: the gpu-marked tests must run on an MI355X")
    import newton_schulz_muon_amd as m
    m.load_library()
    yield m
    m.muon_set_gemm_tiling(0)
    m.muon_set_ns_schedule("auto")


@pytest.mark.parametrize("precision", ["fast", "accurate"])
@pytest.mark.parametrize("shape", SHAPES, ids=lambda s: "x".join(map(str, s)))
def test_widths_and_loop_bitwise(nsm, shape, precision):
    b, m, n, v = shape
    if precision == "accurate" and b * m * n > 40e6:
        pytest.skip("ACCURATE covered on the smaller batches")
    print(f"[sweep] {shape} {precision}", flush=True)
    x = workloads.to_device_bf16(workloads.gaussian_bits((b, m, n), seed=b * 7 + m + n + v))
    mm, nn = min(m, n // v), max(m, n // v)
    mp, np_ = -(-mm // 128) * 128, -(-nn // 128) * 128
    runs = {}
    try:
        nsm.muon_set_ns_schedule("per_product")
        for w in (64, 128, 256):
            if w == 256 and (mp % 256 or np_ % 256):
                continue
            nsm.muon_set_gemm_tiling(w)
            runs[f"{w}-wide"] = [torch_bf16_to_bits(nsm.ns_orthogonalize_batched(x, view_blocks=v,
                                                                                precision=precision))
                                 for _ in range(2)]
        nsm.muon_set_gemm_tiling(0)
        nsm.muon_set_ns_schedule("persistent")
        runs["loop"] = [torch_bf16_to_bits(nsm.ns_orthogonalize_batched(x, view_blocks=v, precision=precision))
                        for _ in range(3)]
    finally:
        nsm.muon_set_gemm_tiling(0)
        nsm.muon_set_ns_schedule("auto")
    ref = runs["64-wide"][0]
    for name, outs in runs.items():
        for i, o in enumerate(outs):
            np.testing.assert_array_equal(o, ref, err_msg=f"{name} call {i} vs 64-wide call 0")
