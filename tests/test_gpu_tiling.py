"""GPU checks of the per-product tile widths (64, 128 and 256 wide).

Every width accumulates each 32 x 32 output block with the same MFMA sequence
in k order and finishes it with the same epilogue arithmetic, so the NS result
is bitwise the same whichever width the Gram, polynomial and B X launches use
(muon_set_gemm_tiling forces one).  Parity of the 128-wide path with the fp64
oracle is established by the other GPU tests; the 64-wide path is also checked
against the oracle directly.  Cases: the per-GPU shares of the 124M set (8
blocks of 768 x 768, 2 of 768 x 3072), ragged sides padded to 128 only, tall
blocks, a block of one 128-wide tile (2 x 2 of 64), ACCURATE precision (split
polynomial and three-segment B X), a full Muon step, several shape groups in
one launch (muon_step_multi) and the executed-flops accounting of each width.
"""
import numpy as np
import pytest

import oracle
import workloads
from parity import assert_ns_close, bits_to_f64, torch_bf16_to_bits

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def nsm():
    import torch
    if not torch.cuda.is_available():
        pytest.fail("no GPU visible: the gpu-marked tests must run on an MI355X")
    import newton_schulz_muon_amd as m
    m.load_library()
    m.muon_set_ns_schedule("per_product")
    yield m
    m.muon_set_gemm_tiling(0)
    m.muon_set_ns_schedule("auto")


def _widths(nsm, fn, widths):
    """{width: fn()} with the tile width forced, and {width: executed Gram flops}."""
    import torch
    out, flops = {}, {}
    for w in widths:
        nsm.muon_set_gemm_tiling(w)
        nsm.muon_timing_collect()
        nsm.muon_timing_enable(["gram"])
        try:
            out[w] = fn()
            torch.cuda.synchronize()
        finally:
            nsm.muon_timing_enable([])
            nsm.muon_set_gemm_tiling(0)
        k = nsm.muon_timing_collect(with_flops=True)
        flops[w] = k["gram"][3] if "gram" in k else 0.0
    return out, flops


def _padded(n):
    return (n + 127) // 128 * 128


def _gram_tiles(mp, bt):
    # upper-triangle tiles; a diagonal 256-wide tile computes 10 of its 16 64 x 64 blocks
    t = mp // bt
    return t * (t + 1) // 2 - (0.375 * t if bt == 256 else 0.0)


# (batch, rows, cols, view_blocks, ns_steps, precision)
CASES = [
    (8, 768, 768, 1, 5, "fast"),        # attn share of one GPU: 8 blocks of 768 x 768
    (2, 768, 3072, 1, 5, "fast"),       # mlp share: 2 blocks of 768 x 3072
    (2, 768, 3072, 4, 5, "fast"),       # the attn view of a 768 x 3072 matrix
    (3, 300, 700, 1, 5, "fast"),        # ragged, padded to 384 x 768 (not 256 multiples)
    (2, 1000, 260, 1, 3, "fast"),       # tall ragged, odd step count
    (5, 96, 200, 1, 5, "fast"),         # one 128-wide tile per side of A
    (3, 300, 700, 1, 5, "accurate"),
    (2, 512, 1024, 1, 2, "accurate"),
    (2, 1024, 512, 1, 5, "accurate"),   # tall
    (8, 1280, 1280, 1, 1, "accurate"),  # many mirrored 128-wide polynomial tiles per block
]


@pytest.mark.parametrize("case", CASES)
def test_tilings_bitwise_equal(nsm, case):
    b, r, c, v, steps, prec = case
    print(f"[tiling] batch={b} shape={(r, c)} view={v} steps={steps} {prec}", flush=True)
    bits = workloads.gaussian_bits((b, r, c), seed=r * 13 + c * 7 + steps)
    x = workloads.to_device_bf16(bits)

    def run():
        return torch_bf16_to_bits(nsm.ns_orthogonalize_batched(x, view_blocks=v, ns_steps=steps, precision=prec))

    m, n = min(r, c), max(r, c)
    if v > 1:
        m, n = (m, n // v) if c > r else (m // v, n)
        m, n = min(m, n), max(m, n)
    mp, np_ = _padded(m), _padded(n)
    widths = [64, 128] + ([256] if mp % 256 == 0 and np_ % 256 == 0 else [])
    outs, flops = _widths(nsm, run, widths)
    for w in widths[1:]:
        np.testing.assert_array_equal(outs[64], outs[w], err_msg=f"64-wide vs {w}-wide")
    # every Gram launch of the forced width executes its upper-triangle tiles
    nblk = b * v
    for w in widths:
        want = steps * nblk * _gram_tiles(mp, w) * 2.0 * w * w * np_
        assert flops[w] == pytest.approx(want, rel=1e-9), (w, flops[w], want)
    if steps == 5:
        ref = oracle.ns_batched(bits_to_f64(bits), view_blocks=v)
        tol = 1e-2 if prec == "accurate" else 2e-2
        for i in range(b):
            assert_ns_close(bits_to_f64(outs[64][i]), ref[i], view_blocks=v, tol=tol, label=f"64-wide [{i}]")


def test_tilings_muon_step_bitwise(nsm):
    # the full Muon step (momentum, normalisation folded into the first
    # products, the scaled update) is bitwise the same at every width
    import torch
    print("[tiling] muon_step_batched 4 x 640 x 1280", flush=True)
    gen = torch.Generator(device="cuda")
    gen.manual_seed(31)
    P0 = torch.randn((4, 640, 1280), generator=gen, device="cuda") / 1280 ** 0.5
    G = (torch.randn((4, 640, 1280), generator=gen, device="cuda") * 1e-2).to(torch.bfloat16)
    M0 = torch.randn((4, 640, 1280), generator=gen, device="cuda") * 1e-3

    def run():
        P, M = P0.clone(), M0.clone()
        O = torch.empty_like(G)
        nsm.muon_step_batched(P, G, M, lr=0.02, weight_decay=0.01, momentum=0.95, update_out=O)
        torch.cuda.synchronize()
        return P.cpu().numpy().view(np.int32), M.cpu().numpy().view(np.int32), O.view(torch.int16).cpu().numpy()

    outs, _ = _widths(nsm, run, [64, 128])
    for a, b in zip(outs[64], outs[128]):
        np.testing.assert_array_equal(a, b)


def test_tilings_multi_bitwise(nsm):
    # several shape groups share each launch (one problem per group)
    import torch
    print("[tiling] muon_step_multi 768x768, 768x3072 (view 4), 512x1536, 1536x512", flush=True)
    gen = torch.Generator(device="cuda")
    gen.manual_seed(5)
    shapes = [((768, 768), 1), ((768, 3072), 4), ((512, 1536), 1), ((1536, 512), 1)]
    init = []
    for (r, c), v in shapes:
        P = torch.randn((r, c), generator=gen, device="cuda") / c ** 0.5
        G = (torch.randn((r, c), generator=gen, device="cuda") * 1e-2).to(torch.bfloat16)
        init.append((P, G, v))

    def run():
        mats, outs = [], []
        for P, G, v in init:
            O = torch.empty_like(G)
            mats.append(dict(params=P.clone(), grads=G, momentum_buf=torch.zeros_like(P), update_out=O,
                             view_blocks=v))
            outs.append(O)
        nsm.muon_step_multi(mats, lr=0.02, weight_decay=0.01, momentum=0.95)
        torch.cuda.synchronize()
        return [o.view(torch.int16).cpu().numpy() for o in outs]

    outs, _ = _widths(nsm, run, [64, 128, 256])
    for w in (128, 256):
        for a, b in zip(outs[64], outs[w]):
            np.testing.assert_array_equal(a, b, err_msg=f"64-wide vs {w}-wide")



@pytest.mark.parametrize("shape", [(8, 1280, 1280), (2, 2048, 2048)])
def test_tilings_accurate_repeatable(nsm, shape):
    # ACCURATE keeps the lo planes of B' and X, which expose fp32-level
    # differences that bf16 rounding hides: every width gives the same bits on
    # every call (a store of the mirror tile racing with its offset register
    # once made the 128-wide split polynomial differ between calls by one ulp
    # in a few elements of the lo plane)
    b, r, c = shape
    print(f"[tiling] ACCURATE repeatability batch={b} shape={(r, c)}", flush=True)
    x = workloads.to_device_bf16(workloads.gaussian_bits(shape, seed=b * 7 + r + c))

    def run():
        return [torch_bf16_to_bits(nsm.ns_orthogonalize_batched(x, ns_steps=1, precision="accurate"))
                for _ in range(4)]

    outs, _ = _widths(nsm, run, [64, 128, 256])
    for w, runs in outs.items():
        for i, o in enumerate(runs):
            np.testing.assert_array_equal(o, outs[64][0], err_msg=f"{w}-wide call {i} vs 64-wide call 0")
