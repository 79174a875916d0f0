"""GPU checks of the persistent NS loop's failure path and of the status words
every call leaves in its workspace.

The loop bounds each dependency wait; a run that gives up must never return
results that pass for valid ones.  The failure is forced from the host
(muon_debug_set_loop_fault), so every kernel still exits normally:
  * mode 1 sets the loop's error word at its start: every workgroup leaves at
    its first item, every block is left incomplete, so every output is NaN and
    the status words count every block;
  * mode 2 makes every dependency wait that is not met at once time out: each
    block is then either complete (bitwise the normal result) or NaN, and the
    status words count the NaN blocks.
After the mode is reset, the next call with the same workspace reports (0, 0)
and gives the normal result.
"""
import numpy as np
import pytest

import workloads
from parity import torch_bf16_to_bits

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def nsm():
    import torch
    if not torch.cuda.is_available():
        pytest.fail("no GPU visible: the gpu-marked tests must run on an MI355X")
    import newton_schulz_muon_amd as m
    m.load_library()
    yield m
    m.muon_debug_set_loop_fault(0)
    m.muon_set_ns_schedule("auto")


def _ns_call(nsm, x, ws, out):
    import ctypes
    import torch
    lib = nsm.load_library()
    B, R, C = x.shape
    st = lib.ns_orthogonalize_batched(x.data_ptr(), out.data_ptr(), B, R, C, 1, None, ws.data_ptr(), ws.numel(),
                                      torch.cuda.current_stream().cuda_stream)
    assert st == 0, nsm.muon_last_error()


def _nan_blocks(bits):
    # bf16 NaN: exponent all ones, mantissa non-zero
    nan = ((bits & 0x7f80) == 0x7f80) & ((bits & 0x007f) != 0)
    return [bool(nan[i].all()) for i in range(bits.shape[0])]


@pytest.mark.parametrize("shape", [(8, 768, 3072), (6, 512, 512)])
def test_forced_abort_poisons_every_block_and_reports(nsm, shape):
    import torch
    print(f"[loop fault] abort at start, shape={shape}", flush=True)
    bits = workloads.gaussian_bits(shape, seed=shape[1] + 7)
    x = workloads.to_device_bf16(bits)
    ws = torch.empty(nsm.muon_workspace_bytes(*shape), dtype=torch.uint8, device="cuda")
    ref = torch.empty_like(x)
    nsm.muon_set_ns_schedule("persistent")
    try:
        _ns_call(nsm, x, ws, ref)
        assert nsm.muon_workspace_status(ws) == (0, 0)
        out = torch.empty_like(x)
        nsm.muon_debug_set_loop_fault(1)
        _ns_call(nsm, x, ws, out)
        nsm.muon_debug_set_loop_fault(0)
        incomplete, flags = nsm.muon_workspace_status(ws)
        got = torch_bf16_to_bits(out)
        assert incomplete == shape[0], (incomplete, flags)
        assert flags & 1 and flags & 2, flags
        assert all(_nan_blocks(got)), "every block must be NaN after a forced abort"
        # the status words are cleared by the next call, which completes normally
        out2 = torch.empty_like(x)
        _ns_call(nsm, x, ws, out2)
        assert nsm.muon_workspace_status(ws) == (0, 0)
        np.testing.assert_array_equal(torch_bf16_to_bits(out2), torch_bf16_to_bits(ref))
    finally:
        nsm.muon_debug_set_loop_fault(0)
        nsm.muon_set_ns_schedule("auto")


def test_forced_timeouts_leave_each_block_complete_or_nan(nsm):
    import torch
    shape = (16, 768, 3072)
    print(f"[loop fault] zero spin limit, shape={shape}", flush=True)
    bits = workloads.gaussian_bits(shape, seed=99)
    x = workloads.to_device_bf16(bits)
    ws = torch.empty(nsm.muon_workspace_bytes(*shape), dtype=torch.uint8, device="cuda")
    ref = torch.empty_like(x)
    out = torch.empty_like(x)
    nsm.muon_set_ns_schedule("persistent")
    try:
        _ns_call(nsm, x, ws, ref)
        nsm.muon_debug_set_loop_fault(2)
        _ns_call(nsm, x, ws, out)
        nsm.muon_debug_set_loop_fault(0)
        incomplete, flags = nsm.muon_workspace_status(ws)
    finally:
        nsm.muon_debug_set_loop_fault(0)
        nsm.muon_set_ns_schedule("auto")
    got, want = torch_bf16_to_bits(out), torch_bf16_to_bits(ref)
    nan = _nan_blocks(got)
    for i in range(shape[0]):
        if not nan[i]:
            np.testing.assert_array_equal(got[i], want[i])
    assert sum(nan) == incomplete
    assert (flags & 2 != 0) == (incomplete > 0)
    print(f"[loop fault] {incomplete} of {shape[0]} blocks left incomplete, flags {flags}", flush=True)


def test_forced_abort_in_a_step_poisons_params_not_momentum(nsm):
    import torch
    shape = (4, 512, 1024)
    print(f"[loop fault] muon_step_batched abort, shape={shape}", flush=True)
    gbits = workloads.gaussian_bits(shape, seed=5)
    g = workloads.to_device_bf16(gbits)
    P = torch.randn(shape, device="cuda") * 0.02
    P0 = P.clone()
    M = torch.zeros(shape, device="cuda")
    nsm.muon_set_ns_schedule("persistent")
    try:
        nsm.muon_debug_set_loop_fault(1)
        nsm.muon_step_batched(P, g, M, lr=0.02, weight_decay=0.0, momentum=0.95)
        nsm.muon_debug_set_loop_fault(0)
        incomplete, flags = nsm.last_call_status()
    finally:
        nsm.muon_debug_set_loop_fault(0)
        nsm.muon_set_ns_schedule("auto")
    torch.cuda.synchronize()
    assert incomplete == shape[0] and flags & 3 == 3, (incomplete, flags)
    assert torch.isnan(P).all()
    # the momentum update precedes the NS loop and is exact: (1 - mu) g from zero
    gf = g.float()
    assert torch.allclose(M, gf * (1 - np.float32(0.95)), rtol=1e-6, atol=0)
    del P0


@pytest.mark.parametrize("steps", [1, 2, 5])
def test_direct_io_alias_is_bitwise(nsm, steps):
    # 256 x 512 blocks are laid out in the caller's buffer exactly as the
    # padded iterate: NS-only calls read x in place and (except one step onto
    # itself) write the last iterate straight into out.  Aliasing out = x
    # must give the non-aliased result bit for bit, under both schedules.
    import torch
    bits = workloads.gaussian_bits((3, 256, 512), seed=40 + steps)
    for sched in ("per_product", "persistent"):
        nsm.muon_set_ns_schedule(sched)
        try:
            x = workloads.to_device_bf16(bits)
            ref = nsm.ns_orthogonalize_batched(x, ns_steps=steps)
            nsm.ns_orthogonalize_batched(x, out=x, ns_steps=steps)
            torch.cuda.synchronize()
        finally:
            nsm.muon_set_ns_schedule("auto")
        np.testing.assert_array_equal(torch_bf16_to_bits(x), torch_bf16_to_bits(ref))
        np.testing.assert_array_equal(workloads.gaussian_bits((3, 256, 512), seed=40 + steps), bits)
