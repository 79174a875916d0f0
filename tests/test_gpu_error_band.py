"""The GPU's measured error against the fp64 oracle, per configuration, must
land in the band the bf16 error model (tests/error_model.py) predicts for it.

The model performs the kernels' roundings with exact accumulation, so the GPU
output should sit close to the model's output and its error close to the
model's error.  Bands (relative Frobenius, per block):
  * error ratio GPU / model within [0.9, 1.1] (measured on MI355X: 0.996 to
    1.010 over these cases);
  * distance GPU - model at most the model's own error (measured 0.17 to
    0.83 of it: fp32 accumulation in another order flips a few bf16 roundings,
    and a flip propagates through later iterations).
Truncation instead of round-to-nearest (about 2x), a dropped lo pass in
ACCURATE (about 8x), or an extra or missing rounding moves the error by far
more than that (tests/test_error_model_cpu.py), even while it stays under the
2e-2 bar."""
import numpy as np
import pytest

import error_model as em
import oracle
import workloads
from parity import bits_to_f64, torch_bf16_to_bits

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def nsm():
    import torch
    if not torch.cuda.is_available():
        pytest.fail("no GPU visible: the gpu-marked tests must run on an MI355X")
    import newton_schulz_muon_amd as m
    m.load_library()
    return m


def _wl_bits(name, group, index):
    wl = workloads.get_workload(name)
    g = {gr.name: gr for gr in wl.groups}[group]
    return workloads.grad_bits_host(wl, g, 0, [index])[0]


def _spectral_bits(m, n, seed):
    rng = np.random.default_rng(seed)
    u, _ = np.linalg.qr(rng.standard_normal((m, m)))
    v, _ = np.linalg.qr(rng.standard_normal((n, m)))
    return workloads.f32_to_bf16_bits(((u * (1.0 / np.arange(1, m + 1))) @ v.T).astype(np.float32))


# (label, input bits factory, precision)
CASES = [
    ("gqa 512x512", lambda: workloads.gaussian_bits((512, 512), seed=1, std=1e-2), "fast"),
    ("gqa 512x256 (tall)", lambda: workloads.gaussian_bits((512, 256), seed=2, std=1e-2), "fast"),
    ("gqa 512x1024", lambda: workloads.gaussian_bits((512, 1024), seed=3, std=1e-2), "fast"),
    ("gqa 1024x512 (tall)", lambda: workloads.gaussian_bits((1024, 512), seed=4, std=1e-2), "fast"),
    ("124M mlp 768x3072", lambda: _wl_bits("gpt124m", "mlp", 0), "fast"),
    ("124M attn block 768x768", lambda: _wl_bits("gpt124m", "attn", 0)[:, :768].copy(), "fast"),
    ("gpt2-medium 1024x4096 heavy rows", lambda: _wl_bits("gpt2_medium", "wide", 3), "fast"),
    ("gpt2-medium 4096x1024 heavy rows (tall)", lambda: _wl_bits("gpt2_medium", "tall", 3), "fast"),
    ("ragged 300x700", lambda: workloads.gaussian_bits((300, 700), seed=5), "fast"),
    ("768x3072 accurate", lambda: _wl_bits("gpt124m", "mlp", 1), "accurate"),
    ("1/i spectrum 1024x3584 fast", lambda: _spectral_bits(1024, 3584, 6), "fast"),
    ("1/i spectrum 1024x3584 accurate", lambda: _spectral_bits(1024, 3584, 6), "accurate"),
    ("large dense 4096x4096 1/i accurate", lambda: _wl_bits("large_dense", "sq", 0), "accurate"),
]


@pytest.mark.timeout(300)
@pytest.mark.parametrize("label,make,precision", CASES, ids=[c[0] for c in CASES])
def test_gpu_error_in_predicted_band(nsm, label, make, precision):
    import torch
    print(f"[error band] {label} ({precision})", flush=True)
    bits = make()
    x = workloads.to_device_bf16(bits[None])
    out = nsm.ns_orthogonalize_batched(x, precision=precision)
    torch.cuda.synchronize()
    got = bits_to_f64(torch_bf16_to_bits(out))[0]
    Y = bits_to_f64(bits)
    ref = oracle.newton_schulz(Y)
    model = em.ns_model(Y, precision=precision)
    e_gpu, e_model = em.rel_fro(got, ref), em.rel_fro(model, ref)
    d = em.rel_fro(got, model)
    print(f"[error band] {label}: GPU {e_gpu:.4e}, model {e_model:.4e} (ratio {e_gpu / e_model:.3f}), "
          f"GPU vs model {d:.3e} ({d / e_model:.3f} of the model's error)", flush=True)
    assert 0.9 <= e_gpu / e_model <= 1.1, (label, e_gpu, e_model)
    assert d <= e_model, (label, d, e_model)
