"""GPU parity of muon_step_batched against the fp64 oracle on the seeded
workloads: the tiny 4 x 64x128 batch, the 9-layer d=512 GQA matrices, the
124M custom-sizing set (gates + attn view + mlp), and a sampled check of the
96-matrix GPT-2-medium-like batch with heavy-tailed rows (stored wide and
tall)."""
import numpy as np
import pytest

import oracle
import workloads
from parity import (MOMENTUM_TOL, NS_REL_TOL, assert_ns_close, bits_to_f64, rel_fro,
                    torch_bf16_to_bits)

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def nsm():
    import torch
    if not torch.cuda.is_available():
        pytest.fail("no GPU visible: the gpu-marked tests must run on an MI355X")
    import newton_schulz_muon_amd as m
    m.load_library()
    return m


def _run_host_workload(nsm, wl, steps=None, sigma_every=True):
    """Runs `steps` optimizer steps of every group on the GPU and in the oracle,
    checking O, M and P after every step."""
    import torch
    steps = wl.steps if steps is None else steps
    worst = {"ns": 0.0, "mom": 0.0, "param": 0.0}
    for grp in wl.groups:
        P_host = workloads.param_init_host(wl, grp)
        P = torch.from_numpy(P_host).cuda()
        M = torch.zeros_like(P)
        O = torch.empty(P.shape, dtype=torch.bfloat16, device="cuda")
        P_ref = P_host.astype(np.float64)
        M_ref = np.zeros_like(P_ref)
        bound = 0.0
        for t in range(steps):
            mu = wl.momentum_at(t)
            gbits = workloads.grad_bits_host(wl, grp, t)
            print(f"[step parity] {wl.name}/{grp.name} {grp.count}x{grp.rows}x{grp.cols} "
                  f"view={grp.view_blocks} step={t}", flush=True)
            G = workloads.to_device_bf16(gbits)
            nsm.muon_step_batched(P, G, M, lr=wl.lr, weight_decay=wl.weight_decay, momentum=mu,
                                  view_blocks=grp.view_blocks, ns_steps=wl.ns_steps,
                                  precision=grp.precision, update_out=O)
            torch.cuda.synchronize()
            P_new, M_new, O_ref = oracle.muon_step(P_ref, bits_to_f64(gbits), M_ref, lr=wl.lr,
                                                   weight_decay=wl.weight_decay, momentum=mu,
                                                   view_blocks=grp.view_blocks, ns_steps=wl.ns_steps)
            O_got = bits_to_f64(torch_bf16_to_bits(O))
            M_got = M.cpu().numpy().astype(np.float64)
            P_got = P.cpu().numpy().astype(np.float64)
            lr_eff = float(np.float32(wl.lr)) * oracle.aspect_factor(grp.rows, grp.cols)
            for i in range(grp.count):
                r, s = assert_ns_close(O_got[i], O_ref[i], grp.view_blocks, sigma=sigma_every or t == 0,
                                       label=f"{grp.name}[{i}] step {t}")
                worst["ns"] = max(worst["ns"], r)
                em = rel_fro(M_got[i], M_new[i])
                assert em <= MOMENTUM_TOL, f"momentum {grp.name}[{i}] step {t}: {em:.3e}"
                worst["mom"] = max(worst["mom"], em)
            bound += NS_REL_TOL * lr_eff * np.linalg.norm(O_ref) + 4 * 2.0 ** -24 * np.linalg.norm(P_new)
            ep = np.linalg.norm(P_got - P_new)
            assert ep <= bound, f"params {grp.name} step {t}: {ep:.3e} > {bound:.3e}"
            worst["param"] = max(worst["param"], ep / bound)
            P_ref, M_ref = P_new, M_new
    print(f"[step parity] {wl.name} worst: {worst}", flush=True)
    return worst


def test_step_tiny(nsm):
    _run_host_workload(nsm, workloads.get_workload("tiny"))


def test_step_tiny_plain_momentum_and_multipliers(nsm):
    import torch
    wl = workloads.get_workload("tiny")
    grp = wl.groups[0]
    P_host = workloads.param_init_host(wl, grp)
    P = torch.from_numpy(P_host).cuda()
    M = torch.full_like(P, 0.25)
    gbits = workloads.grad_bits_host(wl, grp, 0)
    O = torch.empty(P.shape, dtype=torch.bfloat16, device="cuda")
    nsm.muon_step_batched(P, workloads.to_device_bf16(gbits), M, lr=0.1, weight_decay=0.3,
                          momentum=0.9, nesterov=False, lr_mul=0.5, wd_mul=2.0, update_out=O)
    torch.cuda.synchronize()
    P_ref, M_ref, O_ref = oracle.muon_step(P_host, bits_to_f64(gbits), np.full(P_host.shape, 0.25),
                                           lr=0.1, weight_decay=0.3, momentum=0.9, nesterov=False,
                                           lr_mul=0.5, wd_mul=2.0)
    for i in range(grp.count):
        assert_ns_close(bits_to_f64(torch_bf16_to_bits(O))[i], O_ref[i], label=f"plain[{i}]")
        assert rel_fro(M.cpu().numpy()[i], M_ref[i]) <= MOMENTUM_TOL
    bound = NS_REL_TOL * 0.05 * np.linalg.norm(O_ref) + 4 * 2.0 ** -24 * np.linalg.norm(P_ref)
    assert np.linalg.norm(P.cpu().numpy() - P_ref) <= bound


def test_step_gqa_small(nsm):
    _run_host_workload(nsm, workloads.get_workload("gqa_small"), sigma_every=False)


def test_step_gpt124m(nsm):
    _run_host_workload(nsm, workloads.get_workload("gpt124m"), sigma_every=False)


@pytest.mark.timeout(900)
def test_step_gpt2_medium_sampled(nsm):
    """96 matrices (48 wide 1024x4096, 48 stored tall 4096x1024), heavy-tailed
    rows, 20 steps on the GPU.  The oracle follows 8 of the 96 (4 wide, 4 tall)
    through all 20 steps (parameters every step, NS output at the first and the
    last step) and checks the momentum buffer of all 96 matrices after every
    step."""
    import torch
    wl = workloads.get_workload("gpt2_medium")
    sample = {0: [0, 17, 33, 47], 1: [5, 30, 41, 47]}
    for gi, grp in enumerate(wl.groups):
        P = workloads.params_device(wl, grp)
        M = torch.zeros_like(P)
        O = torch.empty(P.shape, dtype=torch.bfloat16, device="cuda")
        idx = sample[gi]
        P_ref = P[idx].cpu().numpy().astype(np.float64)
        M_all = np.zeros((grp.count, grp.rows, grp.cols), np.float64)   # the oracle's buffers of every matrix
        bound = 0.0
        worst_m = 0.0
        for t in range(wl.steps):
            print(f"[step parity] gpt2_medium/{grp.name} step={t}", flush=True)
            G = workloads.grads_device(wl, grp, t)
            g_bits = torch_bf16_to_bits(G)
            nsm.muon_step_batched(P, G, M, lr=wl.lr, weight_decay=wl.weight_decay,
                                  momentum=wl.momentum, update_out=O)
            torch.cuda.synchronize()
            need_ns = t in (0, wl.steps - 1)
            M_gpu = M.cpu().numpy()
            U_s = {}
            for i in range(grp.count):
                M_all[i], U = oracle.nesterov_momentum(bits_to_f64(g_bits[i]), M_all[i], wl.momentum)
                em = rel_fro(M_gpu[i], M_all[i])
                assert em <= MOMENTUM_TOL, f"momentum {grp.name}[{i}] step {t}: {em:.3e}"
                worst_m = max(worst_m, em)
                if i in idx:
                    U_s[i] = U
            O_ref = np.stack([oracle.newton_schulz(U_s[i]) for i in idx])
            P_new = np.stack([oracle.muon_update(P_ref[k], O_ref[k], wl.lr, wl.weight_decay)
                              for k in range(len(idx))])
            if need_ns:
                O_bits = torch_bf16_to_bits(O[idx])
                for k in range(len(idx)):
                    assert_ns_close(bits_to_f64(O_bits[k]), O_ref[k], label=f"{grp.name}[{idx[k]}] step {t}")
            lr_eff = float(np.float32(wl.lr)) * oracle.aspect_factor(grp.rows, grp.cols)
            bound += NS_REL_TOL * lr_eff * np.linalg.norm(O_ref) + 4 * 2.0 ** -24 * np.linalg.norm(P_new)
            ep = np.linalg.norm(P[idx].cpu().numpy() - P_new)
            assert ep <= bound, (t, ep, bound)
            P_ref = P_new
            del G
        print(f"[step parity] gpt2_medium/{grp.name}: worst momentum {worst_m:.3e} over {grp.count} matrices",
              flush=True)


@pytest.mark.timeout(900)
def test_step_large_dense_accurate(nsm):
    """The large dense batch (8 x 4096^2 and 8 x 4096x14336, spectra 1/i) as
    full Muon steps in ACCURATE precision, 2 steps: the momentum buffers of all
    16 matrices against the oracle after each step, and one matrix per group
    (2 of 16) followed through both steps by the oracle (NS output, params)."""
    import torch
    wl = workloads.get_workload("large_dense")
    sample = {"sq": 3, "wide": 6}
    for grp in wl.groups:
        P = workloads.params_device(wl, grp)
        M = torch.zeros_like(P)
        O = torch.empty(P.shape, dtype=torch.bfloat16, device="cuda")
        k = sample[grp.name]
        P_ref = P[k].cpu().numpy().astype(np.float64)
        M_all = np.zeros((grp.count, grp.rows, grp.cols), np.float64)
        bound = 0.0
        for t in range(wl.steps):
            print(f"[step parity] large_dense/{grp.name} {grp.count}x{grp.rows}x{grp.cols} {grp.precision} "
                  f"step={t}", flush=True)
            G = workloads.grads_device(wl, grp, t)
            g_bits = torch_bf16_to_bits(G)
            nsm.muon_step_batched(P, G, M, lr=wl.lr, weight_decay=wl.weight_decay, momentum=wl.momentum,
                                  precision=grp.precision, update_out=O)
            torch.cuda.synchronize()
            M_gpu = M.cpu().numpy()
            U_k = None
            for i in range(grp.count):
                M_all[i], U = oracle.nesterov_momentum(bits_to_f64(g_bits[i]), M_all[i], wl.momentum)
                em = rel_fro(M_gpu[i], M_all[i])
                assert em <= MOMENTUM_TOL, f"momentum {grp.name}[{i}] step {t}: {em:.3e}"
                if i == k:
                    U_k = U
            del M_gpu, g_bits
            O_ref = oracle.newton_schulz(U_k)
            print(f"[step parity] large_dense/{grp.name}[{k}] step {t}: oracle done", flush=True)
            rel, sig = assert_ns_close(bits_to_f64(torch_bf16_to_bits(O[k])), O_ref,
                                       label=f"large_dense {grp.name}[{k}] step {t}")
            print(f"[step parity] large_dense/{grp.name}[{k}] step {t}: rel {rel:.3e} sigma {sig:.3e}", flush=True)
            P_new = oracle.muon_update(P_ref, O_ref, wl.lr, wl.weight_decay)
            lr_eff = float(np.float32(wl.lr)) * oracle.aspect_factor(grp.rows, grp.cols)
            bound += NS_REL_TOL * lr_eff * np.linalg.norm(O_ref) + 4 * 2.0 ** -24 * np.linalg.norm(P_new)
            ep = np.linalg.norm(P[k].cpu().numpy() - P_new)
            assert ep <= bound, (grp.name, t, ep, bound)
            P_ref = P_new
            del G
        del P, M, O


@pytest.mark.parametrize("group", ["attn", "mlp"])
def test_step_rank_share(nsm, group):
    """One GPU's share of the 124M set under 8-way sharding by whole matrices,
    as the benchmark runs it: 2 stored 768x3072 matrices per muon_step_batched
    call (attn: viewed as 8 blocks of 768x768), 3 steps against the oracle."""
    import torch
    wl = workloads.get_workload("gpt124m")
    grp = {g.name: g for g in wl.groups}[group]
    P_host = workloads.param_init_host(wl, grp, [0, 1])
    P = torch.from_numpy(P_host).cuda()
    M = torch.zeros_like(P)
    O = torch.empty(P.shape, dtype=torch.bfloat16, device="cuda")
    P_ref, M_ref = P_host.astype(np.float64), np.zeros(P_host.shape)
    bound = 0.0
    for t in range(wl.steps):
        print(f"[step parity] rank share {group} step={t}", flush=True)
        gbits = workloads.grad_bits_host(wl, grp, t, [0, 1])
        nsm.muon_step_batched(P, workloads.to_device_bf16(gbits), M, lr=wl.lr, weight_decay=wl.weight_decay,
                              momentum=wl.momentum, view_blocks=grp.view_blocks, update_out=O)
        torch.cuda.synchronize()
        P_ref, M_ref, O_ref = oracle.muon_step(P_ref, bits_to_f64(gbits), M_ref, lr=wl.lr,
                                               weight_decay=wl.weight_decay, momentum=wl.momentum,
                                               view_blocks=grp.view_blocks)
        O_got = bits_to_f64(torch_bf16_to_bits(O))
        for i in range(2):
            assert_ns_close(O_got[i], O_ref[i], grp.view_blocks, label=f"share {group}[{i}] step {t}")
            assert rel_fro(M.cpu().numpy()[i], M_ref[i]) <= MOMENTUM_TOL
        lr_eff = float(np.float32(wl.lr)) * oracle.aspect_factor(grp.rows, grp.cols)
        bound += NS_REL_TOL * lr_eff * np.linalg.norm(O_ref) + 4 * 2.0 ** -24 * np.linalg.norm(P_ref)
        assert np.linalg.norm(P.cpu().numpy() - P_ref) <= bound


# Wide blocks go through the element-wise kernels in row strips of 4096
# elements whose width is the widest of 1024, 512, 256, 128 columns dividing
# the padded columns: one shape per width, row counts that leave a ragged
# last strip, an attn view and ACCURATE precision.
STRIP_CASES = [
    (3, 200, 640, 1, "fast"),       # padded columns 640: 128-wide strips (32 rows)
    (2, 130, 1280, 1, "accurate"),  # 1280: 256-wide (16 rows)
    (2, 260, 2560, 1, "fast"),      # 2560: 512-wide (8 rows)
    (2, 102, 2048, 1, "fast"),      # 2048: 1024-wide (4 rows)
    (2, 256, 3072, 4, "fast"),      # attn view: 256 x 768 blocks, 256-wide
]


@pytest.mark.parametrize("b,r,c,v,precision", STRIP_CASES)
def test_step_row_strip_widths(nsm, b, r, c, v, precision):
    import torch
    rng = np.random.default_rng(1000 + r + c)
    P_host = (rng.standard_normal((b, r, c)) / np.sqrt(c)).astype(np.float32)
    M_host = (rng.standard_normal((b, r, c)) * 1e-3).astype(np.float32)
    gbits = workloads.gaussian_bits((b, r, c), seed=77 + r, std=1e-2)
    P = torch.from_numpy(P_host).cuda()
    M = torch.from_numpy(M_host).cuda()
    O = torch.empty((b, r, c), dtype=torch.bfloat16, device="cuda")
    print(f"[strip parity] {b}x{r}x{c} view={v} {precision}", flush=True)
    nsm.muon_step_batched(P, workloads.to_device_bf16(gbits), M, lr=0.05, weight_decay=0.01, momentum=0.95,
                          view_blocks=v, precision=precision, update_out=O)
    torch.cuda.synchronize()
    P_ref, M_ref, O_ref = oracle.muon_step(P_host.astype(np.float64), bits_to_f64(gbits),
                                           M_host.astype(np.float64), lr=0.05, weight_decay=0.01,
                                           momentum=0.95, view_blocks=v)
    O_got = bits_to_f64(torch_bf16_to_bits(O))
    for i in range(b):
        assert_ns_close(O_got[i], O_ref[i], v, label=f"strip {r}x{c}[{i}]")
        assert rel_fro(M.cpu().numpy()[i], M_ref[i]) <= MOMENTUM_TOL
    lr_eff = float(np.float32(0.05)) * oracle.aspect_factor(r, c)
    bound = NS_REL_TOL * lr_eff * np.linalg.norm(O_ref) + 4 * 2.0 ** -24 * np.linalg.norm(P_ref)
    assert np.linalg.norm(P.cpu().numpy() - P_ref) <= bound
