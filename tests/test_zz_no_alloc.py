"""GPU check of ns_orthogonalize_batched_noalloc, the entry point that
allocates nothing (its scratch is the library's static per-GPU array): called
through the C ABI, its output must equal ns_orthogonalize_batched's bit for
bit, on two calls in a row, the second with a smaller (ragged) input, and it
must reject a batch beyond its scratch before enqueueing anything."""
import ctypes

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
    return m


def _noalloc(nsm, x, out):
    import torch
    B, R, C = x.shape
    st = nsm.load_library().ns_orthogonalize_batched_noalloc(
        x.data_ptr(), out.data_ptr(), B, R, C, 1, None, torch.cuda.current_stream().cuda_stream)
    assert st == 0, nsm.muon_last_error()


def test_noalloc_matches_workspace_entry_point(nsm):
    import torch
    # first call: 8 x 512x1024 (tile-exact, read and written in place), then a
    # smaller ragged batch 3 x 300x700 (padded iterates), then a small-block batch
    for k, shape in enumerate([(8, 512, 1024), (3, 300, 700), (4, 64, 128)]):
        print(f"[noalloc] call {k}: {shape}", flush=True)
        bits = workloads.gaussian_bits(shape, seed=700 + k)
        x = workloads.to_device_bf16(bits)
        out = torch.full_like(x, float("nan"))
        _noalloc(nsm, x, out)
        ref = nsm.ns_orthogonalize_batched(x)
        torch.cuda.synchronize()
        got = torch_bf16_to_bits(out)
        np.testing.assert_array_equal(got, torch_bf16_to_bits(ref))
        # and the bar against the fp64 oracle on the first block
        want = oracle.ns_batched(bits_to_f64(bits[:1]))
        assert_ns_close(bits_to_f64(got[:1])[0], want[0], label=f"noalloc {shape}")


def test_noalloc_rejects_batches_beyond_its_scratch(nsm):
    import torch
    x = torch.zeros((32, 768, 3072), dtype=torch.bfloat16, device="cuda")
    out = torch.ones_like(x)
    need = nsm.muon_workspace_bytes(32, 768, 3072)
    assert need > nsm.NOALLOC_SCRATCH_BYTES
    st = nsm.load_library().ns_orthogonalize_batched_noalloc(
        x.data_ptr(), out.data_ptr(), 32, 768, 3072, 1, None, torch.cuda.current_stream().cuda_stream)
    assert st == 4
    assert "no-allocation" in nsm.muon_last_error()
    torch.cuda.synchronize()
    assert bool((out == 1).all())
