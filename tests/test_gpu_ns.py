"""GPU parity of ns_orthogonalize_batched against the fp64 oracle, plus the
invariants the HIP path must keep (bitwise: transpose, batch position, attn view,
determinism, aliasing, zero input, power-of-two scaling; to rounding: oddness)."""
import numpy as np
import pytest

import oracle
import workloads
from parity import assert_ns_close, bits_to_f64, rel_fro, torch_bf16_to_bits

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def nsm():
    import torch
    if not torch.cuda.is_available():
        pytest.fail("no GPU visible: the gpu-marked tests must run on an MI355X")
    import newton_schulz_muon_amd as m
    m.load_library()
    return m


def _run(nsm, bits, **kw):
    import torch
    x = workloads.to_device_bf16(bits)
    out = nsm.ns_orthogonalize_batched(x, **kw)
    torch.cuda.synchronize()
    return torch_bf16_to_bits(out)


def _oracle_batch(bits, view_blocks=1, steps=5, coeffs=oracle.NS_COEFFS):
    return oracle.ns_batched(bits_to_f64(bits), view_blocks=view_blocks, steps=steps, coeffs=coeffs)


# Shapes span several 128-tiles, ragged tails (padding), tall blocks (transposed
# orientation), the small-block path (m <= 64 and m n <= 8192: every 16-row
# tile count, ragged k, 16-byte and element-wise global access, wide and tall)
# and the smallest MFMA-path blocks beside its limits (m = 65; m = 64 with
# m n = 8256).
SHAPES = [(64, 128), (128, 128), (256, 640), (640, 256), (300, 700), (700, 300), (33, 70), (70, 33),
          (96, 1000), (1, 12), (16, 200), (32, 128), (12, 1), (65, 130), (64, 129), (129, 64), (8, 1024),
          (1, 8192), (37, 221), (221, 37), (128, 64), (1024, 8), (48, 168), (4, 2048)]


@pytest.mark.parametrize("shape", SHAPES)
def test_ns_parity_default(nsm, shape):
    print(f"[ns parity] shape={shape}", flush=True)
    bits = workloads.gaussian_bits((3,) + shape, seed=shape[0] * 1000 + shape[1])
    got = bits_to_f64(_run(nsm, bits))
    ref = _oracle_batch(bits)
    for i in range(3):
        assert_ns_close(got[i], ref[i], label=f"{shape}[{i}]")


# Batches large enough for 256-wide tiles with a partial last round, which is
# finished by a second launch of 128-wide quadrants.  50 blocks of 768 x 768:
# the symmetric products run as 128-wide tiles (at K = 768 two 128-wide rounds
# cost what one 256-wide round does), the 450 B X tiles as 256 + 194.  24 of
# 768 x 1536: 144 symmetric tiles (all 128-wide) and 432 B X tiles (256 + 176).
# 50 of 768 x 3072: 300 upper-triangle Gram tiles at K = 3072 (256 + 44, the
# 44 including diagonal tiles whose lower quadrant is skipped; blocks 42 and
# 43 straddle the launch boundary) and 1800 B X tiles (1792 + 8, block 49).
# Blocks on both sides of each launch boundary, and the first and last, are
# checked.
@pytest.mark.parametrize("batch,shape,check", [
    (50, (768, 768), (0, 28, 29, 42, 43, 49)),
    (24, (768, 1536), (0, 14, 15, 23)),
    (24, (1536, 768), (0, 14, 15, 23)),
    (50, (768, 3072), (0, 42, 43, 49)),
])
def test_ns_parity_tail_split(nsm, batch, shape, check):
    print(f"[ns tail split] batch={batch} shape={shape}", flush=True)
    bits = workloads.gaussian_bits((batch,) + shape, seed=batch * 7 + shape[1])
    got = bits_to_f64(_run(nsm, bits))
    ref = _oracle_batch(bits[list(check)])
    for k, i in enumerate(check):
        assert_ns_close(got[i], ref[k], label=f"{shape}[{i}]")


@pytest.mark.parametrize("coeffs", [(1.0, 0.0, 0.0), (0.0, 1.0, 0.0), (0.0, 0.0, 1.0), oracle.NS_COEFFS])
@pytest.mark.parametrize("shape", [(256, 640), (300, 200)])
def test_ns_single_iteration_terms(nsm, coeffs, shape):
    # One iteration with one coefficient at a time isolates the Gram, polynomial
    # and B X kernels (and the normalisation folded into their epilogues).
    print(f"[ns one step] shape={shape} coeffs={coeffs}", flush=True)
    bits = workloads.gaussian_bits((2,) + shape, seed=7)
    got = bits_to_f64(_run(nsm, bits, ns_steps=1, coeffs=coeffs))
    ref = _oracle_batch(bits, steps=1, coeffs=coeffs)
    for i in range(2):
        assert rel_fro(got[i], ref[i]) < 1e-2, (coeffs, i, rel_fro(got[i], ref[i]))


@pytest.mark.parametrize("shape", [(200, 300), (1, 12)])
def test_ns_zero_steps_is_normalisation(nsm, shape):
    bits = workloads.gaussian_bits((2,) + shape, seed=3, std=7.0)
    got = bits_to_f64(_run(nsm, bits, ns_steps=0))
    ref = _oracle_batch(bits, steps=0)
    for i in range(2):
        assert rel_fro(got[i], ref[i]) < 4e-3


def test_ns_attn_view(nsm):
    # stored 96 x 384 read as 4 contiguous 96 x 96 blocks
    bits = workloads.gaussian_bits((3, 96, 384), seed=11)
    got = _run(nsm, bits, view_blocks=4)
    ref = _oracle_batch(bits, view_blocks=4)
    for i in range(3):
        assert_ns_close(bits_to_f64(got[i]), ref[i], view_blocks=4, label=f"view[{i}]")
    # identical to running the [12, 96, 96] reinterpretation without the view
    flat = _run(nsm, bits.reshape(12, 96, 96))
    np.testing.assert_array_equal(got.reshape(12, 96, 96), flat)


def test_ns_transpose_is_bitwise(nsm):
    bits = workloads.gaussian_bits((2, 200, 520), seed=5)
    a = _run(nsm, bits)
    b = _run(nsm, np.ascontiguousarray(bits.transpose(0, 2, 1)))
    np.testing.assert_array_equal(a, b.transpose(0, 2, 1))


def test_ns_odd_within_rounding(nsm):
    # NS is odd in exact arithmetic, and every other step of this path is
    # sign-symmetric (the Gram product of -X equals that of X, scaling and
    # round-to-nearest-even casts commute with negation).  The matrix core's
    # fp32 accumulation does not: (A, -B, -C) gives the negated result of
    # (A, B, C) for only 74-93% of outputs (tests/test_gpu_mfma_rounding.py),
    # so -x and x agree to rounding level only; both must match the oracle.
    bits = workloads.gaussian_bits((2, 256, 384), seed=6)
    a = bits_to_f64(_run(nsm, bits))
    b = bits_to_f64(_run(nsm, bits ^ np.uint16(0x8000)))
    ref = _oracle_batch(bits)
    for i in range(2):
        assert_ns_close(a[i], ref[i], label=f"+x[{i}]")
        assert_ns_close(b[i], -ref[i], label=f"-x[{i}]")
        assert rel_fro(b[i], -a[i]) < 1e-2


def test_ns_batch_position_and_determinism(nsm):
    bits = workloads.gaussian_bits((5, 160, 416), seed=9)
    a = _run(nsm, bits)
    a2 = _run(nsm, bits)
    np.testing.assert_array_equal(a, a2)
    perm = [3, 0, 4, 1, 2]
    b = _run(nsm, bits[perm])
    np.testing.assert_array_equal(a[perm], b)
    single = _run(nsm, bits[2:3])
    np.testing.assert_array_equal(a[2:3], single)


def test_ns_in_place_alias(nsm):
    import torch
    bits = workloads.gaussian_bits((2, 130, 260), seed=12)
    ref = _run(nsm, bits)
    for steps in (1, 5):
        x = workloads.to_device_bf16(bits)
        nsm.ns_orthogonalize_batched(x, out=x, ns_steps=steps)
        torch.cuda.synchronize()
        if steps == 5:
            np.testing.assert_array_equal(torch_bf16_to_bits(x), ref)
        else:
            assert_ns_close(bits_to_f64(torch_bf16_to_bits(x))[0], _oracle_batch(bits, steps=1)[0],
                            tol=1e-2, label="alias one step")


def test_ns_zero_block(nsm):
    bits = np.zeros((2, 128, 256), np.uint16)
    bits[1] = workloads.gaussian_bits((128, 256), seed=1)
    got = _run(nsm, bits)
    assert np.all(got[0] == 0)
    assert_ns_close(bits_to_f64(got[1]), _oracle_batch(bits[1:])[0], label="nonzero neighbour")


def test_ns_scale_invariance(nsm):
    # NS normalises first, so scaling the input by a power of two changes nothing
    bits = workloads.gaussian_bits((2, 192, 320), seed=13)
    scaled = workloads.f32_to_bf16_bits(workloads.bf16_bits_to_f32(bits) * np.float32(64.0))
    np.testing.assert_array_equal(_run(nsm, bits), _run(nsm, scaled))


def test_ns_accurate_mode(nsm):
    bits = workloads.gaussian_bits((2, 256, 640), seed=14)
    fast = bits_to_f64(_run(nsm, bits))
    acc = bits_to_f64(_run(nsm, bits, precision="accurate"))
    ref = _oracle_batch(bits)
    for i in range(2):
        e_fast = rel_fro(fast[i], ref[i])
        e_acc = rel_fro(acc[i], ref[i])
        assert e_acc < 2e-2
        assert e_acc < e_fast, (e_acc, e_fast)


def test_ns_rejects_misaligned_and_small_workspace(nsm):
    import ctypes
    import torch
    lib = nsm.load_library()
    x = torch.zeros((2, 128, 128), dtype=torch.bfloat16, device="cuda")
    need = nsm.muon_workspace_bytes(2, 128, 128)
    ws = torch.empty(need + 512, dtype=torch.uint8, device="cuda")
    st = lib.ns_orthogonalize_batched(x.data_ptr(), x.data_ptr(), 2, 128, 128, 1, None,
                                      ws.data_ptr(), need - 1, None)
    assert st == 4
    st = lib.ns_orthogonalize_batched(x.data_ptr() + 2, x.data_ptr(), 2, 128, 128, 1, None,
                                      ws.data_ptr(), need, None)
    assert st == 3
    st = lib.ns_orthogonalize_batched(x.data_ptr(), x.data_ptr(), 2, 128, 128, 1, None,
                                      ws.data_ptr() + 64, need, None)
    assert st == 3
    assert nsm.muon_last_error()


@pytest.mark.timeout(400)
@pytest.mark.parametrize("group,index", [("sq", 0), ("wide", 7)])
def test_ns_parity_large_dense(nsm, group, index):
    # The large dense batch at full size (8 x 4096^2 and 8 x 4096x14336, decaying
    # spectrum sigma_i = 1/i, ACCURATE precision as the workload runs it): the
    # whole batch goes through the GPU and one matrix is checked against the
    # fp64 oracle on its bf16 input (the matrix the last 256-wide round of the
    # wide group covers, and the first square one).
    import torch
    wl = workloads.get_workload("large_dense")
    g = {gr.name: gr for gr in wl.groups}[group]
    print(f"[ns large_dense] group={group} {g.count}x{g.rows}x{g.cols} precision={g.precision} "
          f"check index {index}", flush=True)
    x = workloads.grads_device(wl, g, 0, torch.device("cuda:0"))
    out = nsm.ns_orthogonalize_batched(x, precision=g.precision)
    torch.cuda.synchronize()
    bits = torch_bf16_to_bits(x[index:index + 1])
    got = bits_to_f64(torch_bf16_to_bits(out[index:index + 1]))
    del x, out
    ref = _oracle_batch(bits)
    print("[ns large_dense] oracle done", flush=True)
    rel, sig = assert_ns_close(got[0], ref[0], label=f"large_dense {group}[{index}]")
    print(f"[ns large_dense] rel {rel:.3e} sigma {sig:.3e}", flush=True)


@pytest.mark.timeout(300)
@pytest.mark.parametrize("schedule", ["per_product", "persistent"])
def test_ns_parity_metric_batch(nsm, schedule):
    # The batch the throughput metric is quoted on, in the call the benchmark
    # times for it: 32 x 768x3072 bf16, N(0, 0.01^2), one ns_orthogonalize_batched
    # over the whole batch, per product (256-wide Gram round at K = 3072,
    # 128-wide polynomial, four 256-wide B X rounds plus a quadrant tail) and
    # in the persistent loop the automatic schedule settles on for it; the
    # first, a middle and the last block are checked against the fp64 oracle.
    import torch
    wl = workloads.get_workload("metric32")
    g = wl.groups[0]
    print(f"[ns metric batch] {schedule} {g.count}x{g.rows}x{g.cols}", flush=True)
    x = workloads.grads_device(wl, g, 0, torch.device("cuda:0"))
    nsm.muon_set_ns_schedule(schedule)
    try:
        out = nsm.ns_orthogonalize_batched(x)
        torch.cuda.synchronize()
    finally:
        nsm.muon_set_ns_schedule("auto")
    for i in (0, 17, g.count - 1):
        bits = torch_bf16_to_bits(x[i:i + 1])
        got = bits_to_f64(torch_bf16_to_bits(out[i:i + 1]))
        ref = _oracle_batch(bits)
        rel, sig = assert_ns_close(got[0], ref[0], label=f"metric32[{i}]")
        print(f"[ns metric batch] block {i}: rel {rel:.3e} sigma {sig:.3e}", flush=True)
