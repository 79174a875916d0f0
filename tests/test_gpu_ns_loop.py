"""GPU checks of the persistent NS loop (one launch for every iteration of the
Gram, polynomial and B X products, tiles taken from a precomputed queue).

Its results must be bitwise those of the per-product launches: every 32 x 32
output block accumulates the same MFMA sequence over k whatever the tiling and
the order in which tiles run.  The per-product path's parity with the fp64
oracle is established by the other GPU tests; here the loop's own output is
also checked against the oracle on sampled blocks.  Cases: one and several
256-wide tiles per side, tall blocks, the attn view, 1 to 5 iterations (the
result lands in either iterate), several shape groups in one launch
(muon_step_multi), a batch that fills more than one round of workgroups, and
repeated calls that reuse the cached queue and the workspace counters.
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
    yield m
    m.muon_set_ns_schedule("auto")


def _both(nsm, fn):
    """fn() under each schedule; returns (persistent, per_product) results and
    the launch counts of the persistent run."""
    import torch
    out = []
    counts = None
    for sched in ("persistent", "per_product"):
        nsm.muon_set_ns_schedule(sched)
        nsm.muon_timing_collect()
        nsm.muon_timing_enable(["ns_loop", "gram", "bx"])
        try:
            out.append(fn())
            torch.cuda.synchronize()
        finally:
            nsm.muon_timing_enable([])
            nsm.muon_set_ns_schedule("auto")
        k = nsm.muon_timing_collect()
        if sched == "persistent":
            counts = k
    return out[0], out[1], counts


# (batch, rows, cols, view_blocks, ns_steps)
NS_CASES = [
    (3, 256, 512, 1, 5),      # one tile per side of A, two B X tiles
    (2, 512, 256, 1, 5),      # tall: oriented 256 x 512
    (5, 768, 768, 1, 5),
    (4, 768, 3072, 1, 5),
    (2, 768, 3072, 4, 5),     # attn view: 8 blocks of 768 x 768
    (2, 1024, 1024, 1, 3),    # odd step count: result in the second iterate
    (3, 512, 1536, 1, 1),
    (2, 256, 256, 1, 2),
]


@pytest.mark.parametrize("case", NS_CASES)
def test_loop_bitwise_equals_per_product(nsm, case):
    b, r, c, v, steps = case
    print(f"[ns loop] batch={b} shape={(r, c)} view={v} steps={steps}", flush=True)
    bits = workloads.gaussian_bits((b, r, c), seed=r * 31 + c + steps)
    x = workloads.to_device_bf16(bits)

    def run():
        return torch_bf16_to_bits(nsm.ns_orthogonalize_batched(x, view_blocks=v, ns_steps=steps))

    got, ref, counts = _both(nsm, run)
    assert counts.get("ns_loop", (0, 0.0))[0] == 1 and "gram" not in counts, counts
    np.testing.assert_array_equal(got, ref)


# ACCURATE precision: B' and X as hi + lo planes, B' X over the three segments
# Bh Xh, Bh Xl, Bl Xh (batch, rows, cols, view_blocks, ns_steps)
ACC_CASES = [
    (3, 512, 1024, 1, 5),
    (2, 1024, 512, 1, 5),     # tall
    (4, 768, 768, 1, 2),
    (2, 256, 256, 1, 3),
]


@pytest.mark.parametrize("case", ACC_CASES)
def test_loop_accurate_bitwise_equals_per_product(nsm, case):
    b, r, c, v, steps = case
    print(f"[ns loop] accurate batch={b} shape={(r, c)} steps={steps}", flush=True)
    bits = workloads.gaussian_bits((b, r, c), seed=r * 17 + c + steps)
    x = workloads.to_device_bf16(bits)

    def run():
        return torch_bf16_to_bits(nsm.ns_orthogonalize_batched(x, view_blocks=v, ns_steps=steps,
                                                                precision="accurate"))

    got, ref, counts = _both(nsm, run)
    assert counts.get("ns_loop", (0, 0.0))[0] == 1 and "gram" not in counts, counts
    np.testing.assert_array_equal(got, ref)
    if steps == 5:
        want = oracle.ns_batched(bits_to_f64(bits), view_blocks=v)
        for i in range(b):
            assert_ns_close(bits_to_f64(got[i]), want[i], tol=1e-2, label=f"accurate loop[{i}]")


def test_loop_accurate_step_bitwise(nsm):
    # a full ACCURATE Muon step in the loop equals the per-product step bit for bit
    import torch
    print("[ns loop] accurate muon_step_batched 4 x 512 x 1536", flush=True)
    gen = torch.Generator(device="cuda")
    gen.manual_seed(12)
    P0 = torch.randn((4, 512, 1536), generator=gen, device="cuda") / 1536 ** 0.5
    G = (torch.randn((4, 512, 1536), generator=gen, device="cuda") * 1e-2).to(torch.bfloat16)
    M0 = torch.randn((4, 512, 1536), generator=gen, device="cuda") * 1e-3

    def run():
        P, M = P0.clone(), M0.clone()
        O = torch.empty_like(G)
        nsm.muon_step_batched(P, G, M, lr=0.02, weight_decay=0.01, momentum=0.95, update_out=O,
                              precision="accurate")
        torch.cuda.synchronize()
        return P.cpu().numpy().view(np.int32), M.cpu().numpy().view(np.int32), O.view(torch.int16).cpu().numpy()

    got, ref, counts = _both(nsm, run)
    assert counts.get("ns_loop", (0, 0.0))[0] == 1, counts
    for a, b in zip(got, ref):
        np.testing.assert_array_equal(a, b)


def test_loop_parity_with_oracle(nsm):
    print("[ns loop] oracle parity 3 x 512 x 1024", flush=True)
    bits = workloads.gaussian_bits((3, 512, 1024), seed=4242)
    x = workloads.to_device_bf16(bits)
    nsm.muon_set_ns_schedule("persistent")
    got = bits_to_f64(torch_bf16_to_bits(nsm.ns_orthogonalize_batched(x)))
    ref = oracle.ns_batched(bits_to_f64(bits), view_blocks=1, steps=5, coeffs=oracle.NS_COEFFS)
    for i in range(3):
        assert_ns_close(got[i], ref[i], label=f"loop[{i}]")


def test_loop_many_blocks_repeated(nsm):
    # 40 blocks of 768 x 3072: 240 symmetric and 1440 B X tiles per
    # iteration, several rounds of the 256 workgroups; three calls in a row
    # reuse the cached queue and re-zero the counters each time.
    import torch
    print("[ns loop] 40 x 768 x 3072, three calls", flush=True)
    gen = torch.Generator(device="cuda")
    gen.manual_seed(7)
    x = (torch.randn((40, 768, 3072), generator=gen, device="cuda") * 1e-2).to(torch.bfloat16)

    def run():
        outs = [nsm.ns_orthogonalize_batched(x) for _ in range(3)]
        torch.cuda.synchronize()
        return [o.view(torch.int16).cpu().numpy() for o in outs]

    got, ref, counts = _both(nsm, run)
    assert counts.get("ns_loop", (0, 0.0))[0] == 3, counts
    for g in got:
        np.testing.assert_array_equal(g, ref[0])
    np.testing.assert_array_equal(ref[1], ref[0])


def test_loop_step_batched_bitwise(nsm):
    import torch
    print("[ns loop] muon_step_batched 6 x 768 x 1536", flush=True)
    gen = torch.Generator(device="cuda")
    gen.manual_seed(11)
    P0 = torch.randn((6, 768, 1536), generator=gen, device="cuda") / 1536 ** 0.5
    G = (torch.randn((6, 768, 1536), generator=gen, device="cuda") * 1e-2).to(torch.bfloat16)
    M0 = torch.randn((6, 768, 1536), generator=gen, device="cuda") * 1e-3

    def run():
        P, M = P0.clone(), M0.clone()
        O = torch.empty_like(G)
        nsm.muon_step_batched(P, G, M, lr=0.02, weight_decay=0.01, momentum=0.95, update_out=O)
        torch.cuda.synchronize()
        return P.cpu().numpy().view(np.int32), M.cpu().numpy().view(np.int32), O.view(torch.int16).cpu().numpy()

    got, ref, counts = _both(nsm, run)
    assert counts.get("ns_loop", (0, 0.0))[0] == 1, counts
    for g, r in zip(got, ref):
        np.testing.assert_array_equal(g, r)


def test_loop_multi_mixed_groups_bitwise(nsm):
    # One wave of several shape groups sharing the launch: 768 x 768 (attn
    # view of 768 x 3072), 768 x 3072, tall 1536 x 768, plus gates on the
    # small-block path.
    import torch
    print("[ns loop] muon_step_multi mixed groups", flush=True)
    shapes = ([(1, 12, 1)] * 3 + [(768, 3072, 4)] * 2 + [(768, 3072, 1)] * 3 + [(1536, 768, 1)] * 2)
    gen = torch.Generator(device="cuda")
    gen.manual_seed(5)
    base = []
    for r, c, v in shapes:
        base.append(dict(params=torch.randn((r, c), generator=gen, device="cuda") / c ** 0.5,
                         grads=(torch.randn((r, c), generator=gen, device="cuda") * 1e-2).to(torch.bfloat16),
                         momentum_buf=torch.randn((r, c), generator=gen, device="cuda") * 1e-3,
                         view_blocks=v))

    def run():
        mats = [dict(m, params=m["params"].clone(), momentum_buf=m["momentum_buf"].clone(),
                     update_out=torch.empty_like(m["grads"])) for m in base]
        for _ in range(2):
            nsm.muon_step_multi(mats, lr=0.02, weight_decay=0.01, momentum=0.95)
        torch.cuda.synchronize()
        return [(m["params"].cpu().numpy().view(np.int32), m["momentum_buf"].cpu().numpy().view(np.int32),
                 m["update_out"].view(torch.int16).cpu().numpy()) for m in mats]

    got, ref, counts = _both(nsm, run)
    assert counts.get("ns_loop", (0, 0.0))[0] >= 2, counts
    for i, (g, r) in enumerate(zip(got, ref)):
        for k in range(3):
            np.testing.assert_array_equal(g[k], r[k], err_msg=f"matrix {i} field {k}")


def test_auto_schedule_choice(nsm):
    # A set of shapes no other test uses: the first ten calls alternate the
    # per-product launches and the persistent loop (timed), later calls keep
    # one of them; every call gives the same bits.
    import torch
    print("[ns loop] automatic choice 6 x 512 x 1024", flush=True)
    bits = workloads.gaussian_bits((6, 512, 1024), seed=777)
    x = workloads.to_device_bf16(bits)
    nsm.muon_set_ns_schedule("auto")
    outs, fams = [], []
    for _ in range(14):
        nsm.muon_timing_collect()
        nsm.muon_timing_enable(["ns_loop", "gram"])
        try:
            outs.append(torch_bf16_to_bits(nsm.ns_orthogonalize_batched(x)))
            torch.cuda.synchronize()
        finally:
            nsm.muon_timing_enable([])
        fams.append(nsm.muon_timing_collect())
    for o in outs[1:]:
        np.testing.assert_array_equal(o, outs[0])
    persistent = ["ns_loop" in f for f in fams]
    assert persistent[:10] == [False, True] * 5, fams
    assert len(set(persistent[10:])) == 1, fams


@pytest.mark.parametrize("shape", [(18, 512, 256), (9, 512, 512), (24, 256, 768)])
def test_loop_small_blocks_repeated(nsm, shape):
    # Many small blocks (one or two tiles per product): operands small enough
    # to stay in a CU's L1 between iterations, so a stale line would be read
    # if the loop's acquire did not drop it.  Ten calls per schedule, each
    # bitwise equal to the per-product result.
    import torch
    print(f"[ns loop] small blocks {shape}, ten calls", flush=True)
    gen = torch.Generator(device="cuda")
    gen.manual_seed(shape[0] * 1000 + shape[2])
    x = (torch.randn(shape, generator=gen, device="cuda") * 1e-2).to(torch.bfloat16)

    def run():
        outs = [nsm.ns_orthogonalize_batched(x) for _ in range(10)]
        torch.cuda.synchronize()
        return [o.view(torch.int16).cpu().numpy() for o in outs]

    got, ref, _ = _both(nsm, run)
    for k, g in enumerate(got):
        np.testing.assert_array_equal(g, ref[0], err_msg=f"persistent call {k}")


@pytest.mark.parametrize("case", [
    (2, 300, 700, "fast"),        # padded sides 384 x 768: not multiples of 256
    (2, 300, 700, "accurate"),
])
def test_forced_loop_falls_back(nsm, case):
    # With the persistent schedule forced, calls it does not apply to run the
    # per-product launches, and give the same bits as under that schedule.
    import torch
    b, r, c, precision = case
    print(f"[ns loop] fallback {case}", flush=True)
    bits = workloads.gaussian_bits((b, r, c), seed=r + c)
    x = workloads.to_device_bf16(bits)

    def run():
        return torch_bf16_to_bits(nsm.ns_orthogonalize_batched(x, precision=precision))

    got, ref, counts = _both(nsm, run)
    assert "ns_loop" not in counts and counts.get("gram", (0, 0.0))[0] == 5, counts
    np.testing.assert_array_equal(got, ref)


@pytest.mark.parametrize("sched", ["persistent", "per_product"])
@pytest.mark.parametrize("shape", [(3, 512, 1024, 1), (2, 768, 3072, 4), (2, 300, 700, 1)])
def test_timing_reports_nominal_flops(nsm, sched, shape):
    # The nominal flops muon_timing_collect reports per kernel family add up,
    # over the families, to 5 (4 m^2 n + 2 m^3) per NS block (m <= n, the
    # unpadded block), whichever kernels ran: the persistent loop reports them
    # all, the per-product launches 2 m^2 n (X X^T, B X) and 2 m^3 (A A) each
    # per iteration.  300 x 700 blocks (padded sides not multiples of 256)
    # always run per product.
    import torch
    b, r, c, v = shape
    print(f"[timing flops] {sched} {shape}", flush=True)
    x = workloads.to_device_bf16(workloads.gaussian_bits((b, r, c), seed=r + c + v))
    nsm.muon_set_ns_schedule(sched)
    nsm.muon_timing_collect()
    nsm.muon_timing_enable(["ns_loop", "gram", "poly", "bx"])
    try:
        nsm.ns_orthogonalize_batched(x, view_blocks=v)
        torch.cuda.synchronize()
    finally:
        nsm.muon_timing_enable([])
        nsm.muon_set_ns_schedule("auto")
    k = nsm.muon_timing_collect(with_flops=True)
    m, n = min(r, c // v), max(r, c // v)
    expect = b * v * 5 * (4.0 * m * m * n + 2.0 * m ** 3)
    assert sum(f for _, _, f, _ in k.values()) == pytest.approx(expect, rel=1e-12), k
    loop = sched == "persistent" and r % 256 == 0 and (c // v) % 256 == 0
    assert set(k) == ({"ns_loop"} if loop else {"gram", "poly", "bx"}), k
    if not loop:
        assert k["gram"][2] == pytest.approx(b * v * 5 * 2.0 * m * m * n, rel=1e-12)
        assert k["poly"][2] == pytest.approx(b * v * 5 * 2.0 * m ** 3, rel=1e-12)
    # executed flops: the tiles that ran, on the padded block; never below the
    # symmetric work 5 (3 m^2 n + m^3) nor above the padded dense work
    mp, np_ = -(-m // 128) * 128, -(-n // 128) * 128
    executed = sum(e for _, _, _, e in k.values())
    assert b * v * 5 * (3.0 * m * m * n + m ** 3) <= executed <= b * v * 5 * (4.0 * mp * mp * np_ + 2.0 * mp ** 3)
    if loop:
        # diagonal tiles of the symmetric products compute 10 of their 16 64 x 64 blocks
        t, tn = mp // 256, np_ // 256
        sym = t * (t + 1) // 2 - 0.375 * t
        assert executed == pytest.approx(b * v * 5 * 2.0 * 256 * 256 * (sym * np_ + sym * mp + t * tn * mp),
                                         rel=1e-12)


@pytest.mark.parametrize("sched,shape", [("per_product", (2, 256, 640)), ("persistent", (2, 256, 512)),
                                         ("per_product", (2, 512, 1024))])
def test_accurate_workspace_at_high_addresses(nsm, sched, shape):
    # The split B X kernels rebuild their buffer descriptors from 64-bit plane
    # addresses in scalar registers.  A workspace whose planes sit at
    # addresses with bit 31 set (the low word >= 2^31) must give the same
    # bits as one elsewhere (a sign-extended low word once corrupted the
    # descriptor's high address bits there).
    import ctypes
    import torch
    b, r, c = shape
    print(f"[ns loop] accurate, workspace at high address bits, {sched} {shape}", flush=True)
    lib = nsm.load_library()
    cfg = nsm.make_config(precision="accurate")
    need = nsm.muon_workspace_bytes(b, r, c, 1, cfg)
    assert need < (1 << 30)
    big = torch.empty(need + (1 << 32), dtype=torch.uint8, device="cuda")
    base = big.data_ptr()
    d = ((0x80000000 - (base & 0xFFFFFFFF)) % (1 << 32) + 255) // 256 * 256
    ws_hi = base + d
    assert (ws_hi & 0xFFFFFFFF) >= 0x80000000 and ((ws_hi + need) & 0xFFFFFFFF) >= 0x80000000
    assert d + need <= big.numel()
    x = workloads.to_device_bf16(workloads.gaussian_bits(shape, seed=r + c + 99))
    ref_ws = torch.empty(need, dtype=torch.uint8, device="cuda")
    outs = []
    nsm.muon_set_ns_schedule(sched)
    try:
        for ws in (ref_ws.data_ptr(), ws_hi):
            out = torch.empty_like(x)
            st = lib.ns_orthogonalize_batched(x.data_ptr(), out.data_ptr(), b, r, c, 1, ctypes.byref(cfg),
                                              ctypes.c_void_p(ws), need, torch.cuda.current_stream().cuda_stream)
            assert st == 0, nsm.muon_last_error()
            torch.cuda.synchronize()
            outs.append(torch_bf16_to_bits(out))
    finally:
        nsm.muon_set_ns_schedule("auto")
    np.testing.assert_array_equal(outs[0], outs[1])
    del big
