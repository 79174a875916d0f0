"""What the build's LDS DMA hazard scan relies on: a vector memory load that
reads an SGPR five or more wait states after a VALU instruction wrote it sees
the new value.  The library's DMA is inline assembly, outside the compiler's
hazard recognizer; the build rejects any DMA closer than five wait states to a
VALU write of its SGPRs, and the one loader whose offset comes from
v_readfirstlane puts five wait states before its loads.  A test-only kernel
(tests/kernels/sgpr_hazard_probe.hip) counts which offset each load used,
for v_readfirstlane and for v_readlane (the restore of a spilled SGPR), with
0, 1, 2 and 5 instructions between the write and the load; only the last is
asserted, the others are printed (measured on gfx950: with none between,
40-76% of the loads used the old value, with one between 2-52%, varying from
run to run, with two or more none)."""
import ctypes
import os

import pytest

pytestmark = pytest.mark.gpu

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
PROBE = os.path.join(ROOT, "tests", "libsgpr_hazard_probe.so")
BLOCKS, REPS = 256, 32


@pytest.fixture(scope="module")
def probe():
    import torch
    if not torch.cuda.is_available():
        pytest.fail("no GPU visible: the gpu-marked tests must run on an MI355X")
    if not os.path.exists(PROBE):
        pytest.fail("tests/libsgpr_hazard_probe.so is not built: run __graft_entry__.build()")
    lib = ctypes.CDLL(PROBE)
    lib.sgpr_hazard_probe_launch.argtypes = [ctypes.c_void_p, ctypes.c_uint32, ctypes.c_void_p] + \
        [ctypes.c_int] * 4 + [ctypes.c_void_p]
    lib.sgpr_hazard_probe_launch.restype = ctypes.c_int
    return lib


def _run(probe, gap, kind):
    import torch
    src = torch.arange(8192, dtype=torch.int32, device="cuda")
    out = torch.zeros(2, dtype=torch.int32, device="cuda")
    st = torch.cuda.current_stream().cuda_stream
    assert probe.sgpr_hazard_probe_launch(src.data_ptr(), 8192, out.data_ptr(), gap, kind, BLOCKS, REPS, st) == 0
    torch.cuda.synchronize()
    new, old = (int(v) for v in out.cpu())
    return new, old


@pytest.mark.parametrize("kind", [0, 1], ids=["readfirstlane", "readlane"])
def test_five_wait_states_make_the_sgpr_write_visible(probe, kind):
    total = BLOCKS * 256 * REPS
    for gap in (0, 1, 2):
        new, old = _run(probe, gap, kind)
        print(f"[sgpr hazard] kind={kind} gap={gap}: new {new} old {old} of {total}", flush=True)
        assert new + old == total
    new, old = _run(probe, 5, kind)
    print(f"[sgpr hazard] kind={kind} gap=5: new {new} old {old} of {total}", flush=True)
    assert (new, old) == (total, 0)
