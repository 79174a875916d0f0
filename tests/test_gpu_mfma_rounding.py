"""How the matrix core rounds: one v_mfma_f32_32x32x16_bf16 per wave (the
instruction every NS product here is built from), run by a test-only kernel
(tests/kernels/mfma_probe.hip) on seeded bf16 fragments and fp32
accumulators.  The exact result of each output (16 bf16 products plus the
accumulator) is representable in float64 for the exponent ranges drawn here,
so the host knows it exactly and compares:
  * the hardware result against the exact sum correctly rounded to fp32;
  * the result for (A, -B, -C) against the negated result for (A, B, C).
The second one decides whether NS(-X) = -NS(X) can hold bit for bit."""
import ctypes
import os

import numpy as np
import pytest

import workloads

pytestmark = pytest.mark.gpu

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
PROBE = os.path.join(ROOT, "tests", "libmfma_probe.so")


@pytest.fixture(scope="module")
def probe():
    import torch
    if not torch.cuda.is_available():
        pytest.fail("no GPU visible: the gpu-marked tests must run on an MI355X")
    if not os.path.exists(PROBE):
        pytest.fail("tests/libmfma_probe.so is not built: run __graft_entry__.build()")
    lib = ctypes.CDLL(PROBE)
    lib.mfma_probe_launch.argtypes = [ctypes.c_void_p] * 4 + [ctypes.c_int, ctypes.c_void_p]
    lib.mfma_probe_launch.restype = ctypes.c_int
    return lib


def _run(probe, a_bits, b_bits, c0):
    import torch
    waves = a_bits.shape[0] // 512
    a = torch.from_numpy(a_bits.view(np.int16)).cuda()
    b = torch.from_numpy(b_bits.view(np.int16)).cuda()
    c = torch.from_numpy(c0).cuda()
    out = torch.empty_like(c)
    assert probe.mfma_probe_launch(a.data_ptr(), b.data_ptr(), c.data_ptr(), out.data_ptr(), waves,
                                   torch.cuda.current_stream().cuda_stream) == 0
    torch.cuda.synchronize()
    return out.cpu().numpy()


def _exact(a_bits, b_bits, c0):
    """(D, S) per output in the lanes' register layout (see the kernel's
    header): D = A B + C exactly (float64), S = |A| |B| + |C|, the magnitude
    the terms of each sum add up to."""
    w = a_bits.shape[0] // 512
    A = workloads.bf16_bits_to_f32(a_bits).astype(np.float64).reshape(w, 2, 32, 8)   # [w][l/32][i][k8]
    B = workloads.bf16_bits_to_f32(b_bits).astype(np.float64).reshape(w, 2, 32, 8)   # [w][l/32][j][k8]
    Am = A.transpose(0, 2, 1, 3).reshape(w, 32, 16)            # A[i][k], k = 8 (l/32) + e
    Bm = B.transpose(0, 1, 3, 2).reshape(w, 16, 32)            # B[k][j]
    # register r of lane l holds D[8 (r/4) + 4 (l/32) + r%4][l % 32]
    l = np.arange(64)[:, None]
    r = np.arange(16)[None, :]
    i = 8 * (r // 4) + 4 * (l // 32) + r % 4
    j = np.broadcast_to(l % 32, i.shape)
    D = (Am @ Bm)[:, i, j].reshape(-1) + c0.astype(np.float64)
    S = (np.abs(Am) @ np.abs(Bm))[:, i, j].reshape(-1) + np.abs(c0).astype(np.float64)
    return D, S


def _inputs(seed, waves, with_acc):
    rng = np.random.default_rng(seed)
    n = waves * 512
    # mantissa spread inside 2^-4 .. 2^4 keeps every exact sum within float64's 53 bits
    a = rng.standard_normal(n) * np.exp2(rng.integers(-4, 5, n))
    b = rng.standard_normal(n) * np.exp2(rng.integers(-4, 5, n))
    a_bits = workloads.f32_to_bf16_bits(a.astype(np.float32))
    b_bits = workloads.f32_to_bf16_bits(b.astype(np.float32))
    c0 = (rng.standard_normal(waves * 1024) * np.exp2(rng.integers(-4, 5, waves * 1024))).astype(np.float32)
    if not with_acc:
        c0[:] = 0.0
    return a_bits, b_bits, c0


@pytest.mark.parametrize("with_acc", [False, True])
def test_mfma_rounding_and_sign_symmetry(probe, with_acc):
    waves = 2048
    a_bits, b_bits, c0 = _inputs(31 + with_acc, waves, with_acc)
    pos = _run(probe, a_bits, b_bits, c0)
    neg = _run(probe, a_bits, b_bits ^ np.uint16(0x8000), -c0)
    exact, mag = _exact(a_bits, b_bits, c0)
    rne = exact.astype(np.float32)                      # the exact sum rounded once, to nearest even
    u = 2.0 ** -24
    err = np.abs(pos.astype(np.float64) - exact) / (u * mag)
    once = float(np.mean(pos == rne))
    asym = float(np.mean(neg != -pos))
    print(f"[mfma] accumulator {'random' if with_acc else 'zero'}: {pos.size} outputs; equal to the exact sum "
          f"rounded once: {once:.4f}; max error {err.max():.2f} u * sum|terms|; (A,-B,-C) != -(A,B,C): "
          f"{asym:.4f}; below the exact sum {float(np.mean(pos < exact)):.4f}, above "
          f"{float(np.mean(pos > exact)):.4f}", flush=True)
    # The layout reading is right and the sums are fp32-accurate: within the
    # recursive-summation bound of 17 terms, 17 u sum|terms|.
    assert err.max() <= 17.0
    # The accumulation rounds in more than one step (not once, to nearest) ...
    assert once < 0.99
    # ... and not symmetrically: negating B and C does not always negate the
    # result, by at most a rounding error of either sum.  Hence NS(-X) equals
    # -NS(X) only to rounding on this hardware, not bit for bit.
    assert asym > 0.0
    assert (np.abs(neg.astype(np.float64) + pos) / (u * mag)).max() <= 34.0
