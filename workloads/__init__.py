"""Seeded synthetic inputs for the batched Muon step.

This module is shared by the tests, the benchmark and the CPU oracle's callers.
It draws random numbers and encodes them; it performs none of the optimizer's
arithmetic (no momentum, no normalisation, no Newton-Schulz, no update).

Sources of the workload shapes (the pages have no datasets or weights here, so
every gradient is a seeded random stand-in with the shapes the pages describe):

* Muon Custom Sizing page (modded-nanogpt record 2025-09-23), section 2 (all
  attn and mlp weights stored with one shape; 10 attn + 22 mlp matrices;
  smear_gate / attn_gate small params), section 3.1 (qkvo weight stored as
  (hdim, 4*dim) and viewed as (4, hdim, dim)), section 4 (Muon defaults
  lr 0.02 / wd 0.01 / momentum 0.95 and the record run's lr 0.05 / wd 0).
* parameter-golf train_gpt.py walkthrough, the starter model description
  (9 layers, width 512, 8 heads with 4 KV heads) and Part 1 (matrix_lr 0.04,
  momentum warm-up from 0.85 to 0.95 over the first 500 steps).
* AdamW workload: the same Custom Sizing page, section 4 (a DistAdam steps the
  scalar, head and embedding parameters with lr 0.008, betas (0.8, 0.95),
  eps 1e-8) and the model it trains (vocab_size 50257, model_dim 768,
  num_layers 12).  The pages give no scalar count and no Adam weight decay:
  48 scalars (4 per layer) and weight decay 0 are this workload's readings.

bf16 values are carried as raw uint16 bit patterns.  The float32 -> bf16
encoder below is IEEE round-to-nearest-even on the upper 16 bits, written from
that definition.
"""
from __future__ import annotations

import dataclasses
import hashlib
from typing import Callable, Dict, List, Optional, Sequence, Tuple

import numpy as np

__all__ = [
    "f32_to_bf16_bits", "bf16_bits_to_f32", "Group", "Workload", "WORKLOADS",
    "get_workload", "grad_bits_host", "param_init_host", "momentum_warmup",
    "grads_device", "params_device", "gaussian_bits", "to_device_bf16",
    "AdamWorkload", "ADAM_WORKLOADS", "adam_grad_bits_host", "adam_param_host", "adam_grads_device",
    "adam_params_device",
]


# --------------------------------------------------------------------------
# bf16 encoding (round to nearest, ties to even)
# --------------------------------------------------------------------------
def f32_to_bf16_bits(x) -> np.ndarray:
    """float32 -> bf16 bit pattern with round-to-nearest-even; NaN -> quiet NaN."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32).astype(np.uint64)
    lsb = (u >> np.uint64(16)) & np.uint64(1)
    r = ((u + np.uint64(0x7FFF) + lsb) >> np.uint64(16)).astype(np.uint32)
    out = (r & np.uint32(0xFFFF)).astype(np.uint16)
    nan = np.isnan(x)
    if nan.any():
        out = np.where(nan, ((u >> np.uint64(16)).astype(np.uint16) | np.uint16(0x0040)), out)
    return out


def bf16_bits_to_f32(b) -> np.ndarray:
    b = np.ascontiguousarray(b, dtype=np.uint16)
    return (b.astype(np.uint32) << np.uint32(16)).view(np.float32)


# --------------------------------------------------------------------------
# Workload descriptions
# --------------------------------------------------------------------------
@dataclasses.dataclass(frozen=True)
class Group:
    """`count` same-shaped stored matrices of shape rows x cols.

    view_blocks > 1 means each stored matrix is re-read, row-major, as
    view_blocks contiguous blocks of shape rows x (cols / view_blocks) before
    Newton-Schulz (the attention-weight view).
    """
    name: str
    count: int
    rows: int
    cols: int
    view_blocks: int = 1
    first_id: int = 0          # global matrix index of the first matrix (seeding)
    precision: str = "fast"    # "fast" or "accurate"

    @property
    def block_shape(self) -> Tuple[int, int]:
        return self.rows, self.cols // self.view_blocks

    @property
    def n_blocks(self) -> int:
        return self.count * self.view_blocks


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    description: str
    groups: Tuple[Group, ...]
    steps: int
    lr: float
    weight_decay: float
    momentum: float                 # constant value, or the warm-up start
    momentum_warmup_steps: int      # 0: constant momentum
    grad_kind: str                  # "gauss", "heavy", "spectral"
    grad_std: float
    seed: int
    ns_steps: int = 5

    def momentum_at(self, step: int) -> float:
        if self.momentum_warmup_steps <= 0:
            return self.momentum
        return momentum_warmup(step, self.momentum, 0.95, self.momentum_warmup_steps)

    @property
    def n_matrices(self) -> int:
        return sum(g.count for g in self.groups)


def momentum_warmup(step: int, start: float, end: float, warmup_steps: int) -> float:
    """Linear momentum warm-up from `start` at step 0 to `end` at `warmup_steps`.

    parameter-golf walkthrough, Part 1, momentum warm-up paragraph (0.85 -> 0.95
    over the first 500 steps).  This is a hyper-parameter schedule handed to the
    optimizer as a scalar input, not part of the step's arithmetic.
    """
    frac = min(step / float(warmup_steps), 1.0)
    return (1.0 - frac) * start + frac * end


def _groups(spec: Sequence[Tuple[str, int, int, int, int, str]]) -> Tuple[Group, ...]:
    out, gid = [], 0
    for name, count, rows, cols, view, prec in spec:
        out.append(Group(name, count, rows, cols, view, gid, prec))
        gid += count
    return tuple(out)


def _gqa_groups() -> Tuple[Group, ...]:
    # 9 layers of d=512, 8 heads / 4 KV heads (head_dim 64 -> K/V width 256),
    # MLP 2x.  Grouped by shape, one launch group per unique shape.
    per_layer = [("c_q", 512, 512), ("c_k", 512, 256), ("c_v", 512, 256),
                 ("proj", 512, 512), ("fc", 512, 1024), ("mlp_proj", 1024, 512)]
    by_shape: Dict[Tuple[int, int], int] = {}
    for _, r, c in per_layer:
        by_shape[(r, c)] = by_shape.get((r, c), 0) + 9
    spec = [(f"{r}x{c}", n, r, c, 1, "fast") for (r, c), n in by_shape.items()]
    return _groups(spec)


WORKLOADS: Dict[str, Workload] = {
    "tiny": Workload(
        name="tiny",
        description="4 matrices 64x128, bf16 grads ~N(0,1), fp32 momentum zero-init, "
                    "Nesterov 0.95, 5 NS steps, lr 0.02, wd 0.01",
        groups=_groups([("w", 4, 64, 128, 1, "fast")]),
        steps=3, lr=0.02, weight_decay=0.01, momentum=0.95, momentum_warmup_steps=0,
        grad_kind="gauss", grad_std=1.0, seed=20251202),
    "gqa_small": Workload(
        name="gqa_small",
        description="9-layer d=512 GQA (8 heads / 4 KV heads) matrices grouped by shape; "
                    "bf16 grads ~N(0,1e-2); momentum warm-up from 0.85; 10 steps; lr 0.04, wd 0",
        groups=_gqa_groups(),
        steps=10, lr=0.04, weight_decay=0.0, momentum=0.85, momentum_warmup_steps=500,
        grad_kind="gauss", grad_std=1e-2, seed=20251203),
    "gpt124m": Workload(
        name="gpt124m",
        description="124M GPT custom sizing: 11 gates 1x12 first, then 10 attn 768x3072 "
                    "(each viewed as 4 x 768x768) and 22 mlp 768x3072; bf16 grads ~N(0,1e-2); "
                    "momentum 0.95; lr 0.05, wd 0",
        groups=_groups([("gate", 11, 1, 12, 1, "accurate"),
                        ("attn", 10, 768, 3072, 4, "fast"),
                        ("mlp", 22, 768, 3072, 1, "fast")]),
        steps=3, lr=0.05, weight_decay=0.0, momentum=0.95, momentum_warmup_steps=0,
        grad_kind="gauss", grad_std=1e-2, seed=20251204),
    "metric32": Workload(
        name="metric32",
        description="32 matrices 768x3072, bf16 grads ~N(0,1e-2), momentum 0.95, lr 0.05, wd 0",
        groups=_groups([("w", 32, 768, 3072, 1, "fast")]),
        steps=3, lr=0.05, weight_decay=0.0, momentum=0.95, momentum_warmup_steps=0,
        grad_kind="gauss", grad_std=1e-2, seed=20251204),
    "gpt2_medium": Workload(
        name="gpt2_medium",
        description="96 matrices 1024x4096 (48 stored transposed as 4096x1024), bf16 grads "
                    "~N(0,1e-2) with 1% of rows scaled x100; 20 steps; lr 0.02, wd 0.01",
        groups=_groups([("wide", 48, 1024, 4096, 1, "fast"),
                        ("tall", 48, 4096, 1024, 1, "fast")]),
        steps=20, lr=0.02, weight_decay=0.01, momentum=0.95, momentum_warmup_steps=0,
        grad_kind="heavy", grad_std=1e-2, seed=20251205),
    "large_dense": Workload(
        name="large_dense",
        description="8 matrices 4096x4096 + 8 matrices 4096x14336, grads U diag(1/i) V^T "
                    "from seeded random orthogonal U, V; 2 steps; lr 0.02, wd 0.01",
        groups=_groups([("sq", 8, 4096, 4096, 1, "accurate"),
                        ("wide", 8, 4096, 14336, 1, "accurate")]),
        steps=2, lr=0.02, weight_decay=0.01, momentum=0.95, momentum_warmup_steps=0,
        grad_kind="spectral", grad_std=1.0, seed=20251206),
}


def get_workload(name: str) -> Workload:
    return WORKLOADS[name]


# --------------------------------------------------------------------------
# Host (numpy) generation: one independent stream per (seed, step, matrix)
# --------------------------------------------------------------------------
def _rng(seed: int, step: int, matrix_id: int, salt: int = 0) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence([seed, salt, step, matrix_id])))


def _haar(rng: np.random.Generator, rows: int, cols: int) -> np.ndarray:
    """rows x cols (rows >= cols) matrix with orthonormal columns, Haar distributed."""
    z = rng.standard_normal((rows, cols))
    q, r = np.linalg.qr(z)
    return q * np.sign(np.diag(r))[None, :]


def grad_f32_host(wl: Workload, group: Group, step: int, index: int) -> np.ndarray:
    """float32 gradient (before bf16 encoding) for matrix `index` of `group`."""
    mid = group.first_id + index
    rng = _rng(wl.seed, step, mid)
    R, C = group.rows, group.cols
    if wl.grad_kind in ("gauss", "heavy"):
        g = rng.standard_normal((R, C), dtype=np.float32) * np.float32(wl.grad_std)
        if wl.grad_kind == "heavy":
            n_out = int(round(0.01 * R))
            rows = rng.permutation(R)[:n_out]
            g[rows, :] *= np.float32(100.0)
        return g
    if wl.grad_kind == "spectral":
        m = min(R, C)
        u = _haar(rng, R, m)
        v = _haar(rng, C, m)
        s = 1.0 / np.arange(1, m + 1, dtype=np.float64)
        return ((u * s[None, :]) @ v.T).astype(np.float32)
    raise ValueError(wl.grad_kind)


def grad_bits_host(wl: Workload, group: Group, step: int,
                   indices: Optional[Sequence[int]] = None) -> np.ndarray:
    """bf16 bit patterns, shape [len(indices), rows, cols]."""
    idx = range(group.count) if indices is None else indices
    return np.stack([f32_to_bf16_bits(grad_f32_host(wl, group, step, i)) for i in idx])


def param_init_host(wl: Workload, group: Group,
                    indices: Optional[Sequence[int]] = None) -> np.ndarray:
    """float32 initial parameters ~ N(0, 1/cols), shape [len(indices), rows, cols]."""
    idx = range(group.count) if indices is None else indices
    out = []
    for i in idx:
        rng = _rng(wl.seed, 0, group.first_id + i, salt=1)
        out.append(rng.standard_normal((group.rows, group.cols), dtype=np.float32)
                   * np.float32(1.0 / np.sqrt(group.cols)))
    return np.stack(out)


# --------------------------------------------------------------------------
# Device (torch) generation for the large batches.  The same bits are copied
# back to the host when the oracle needs them.
# --------------------------------------------------------------------------
def _torch_seed(*parts: int) -> int:
    h = hashlib.sha256(("/".join(str(p) for p in parts)).encode()).digest()
    return int.from_bytes(h[:8], "little") & ((1 << 63) - 1)


def grads_device(wl: Workload, group: Group, step: int, device="cuda"):
    """bf16 gradients [count, rows, cols] drawn on `device` from a seeded torch generator."""
    import torch
    gen = torch.Generator(device=device)
    gen.manual_seed(_torch_seed(wl.seed, step, group.first_id, group.count))
    R, C, n = group.rows, group.cols, group.count
    if wl.grad_kind in ("gauss", "heavy"):
        g = torch.randn((n, R, C), generator=gen, device=device, dtype=torch.float32)
        g.mul_(wl.grad_std)
        if wl.grad_kind == "heavy":
            n_out = int(round(0.01 * R))
            keys = torch.rand((n, R), generator=gen, device=device)
            rows = keys.argsort(dim=1)[:, :n_out]
            scale = torch.ones((n, R), device=device)
            scale.scatter_(1, rows, 100.0)
            g.mul_(scale[:, :, None])
        return g.to(torch.bfloat16)
    if wl.grad_kind == "spectral":
        m = min(R, C)
        s = 1.0 / torch.arange(1, m + 1, device=device, dtype=torch.float32)
        out = torch.empty((n, R, C), device=device, dtype=torch.bfloat16)
        for i in range(n):
            zu = torch.randn((R, m), generator=gen, device=device, dtype=torch.float32)
            zv = torch.randn((C, m), generator=gen, device=device, dtype=torch.float32)
            qu, ru = torch.linalg.qr(zu)
            qv, rv = torch.linalg.qr(zv)
            qu = qu * torch.sign(torch.diagonal(ru))[None, :]
            qv = qv * torch.sign(torch.diagonal(rv))[None, :]
            out[i] = ((qu * s[None, :]) @ qv.T).to(torch.bfloat16)
        return out
    raise ValueError(wl.grad_kind)


def params_device(wl: Workload, group: Group, device="cuda"):
    import torch
    gen = torch.Generator(device=device)
    gen.manual_seed(_torch_seed(wl.seed, "param", group.first_id, group.count))
    p = torch.randn((group.count, group.rows, group.cols), generator=gen, device=device,
                    dtype=torch.float32)
    return p.mul_(1.0 / float(np.sqrt(group.cols)))


def gaussian_bits(shape, seed: int, std: float = 1.0) -> np.ndarray:
    """bf16 bits of seeded N(0, std^2) samples of any shape (ad-hoc test inputs)."""
    rng = np.random.Generator(np.random.PCG64(np.random.SeedSequence([seed, 0xAD40C])))
    return f32_to_bf16_bits(rng.standard_normal(shape, dtype=np.float32) * np.float32(std))


def to_device_bf16(bits: np.ndarray, device="cuda"):
    """Uploads bf16 bit patterns as a torch.bfloat16 tensor."""
    import torch
    t = torch.from_numpy(np.ascontiguousarray(bits).view(np.int16))
    return t.to(device).view(torch.bfloat16)


# --------------------------------------------------------------------------
# AdamW workloads (the non-matrix parameters of the same models)
# --------------------------------------------------------------------------
@dataclasses.dataclass(frozen=True)
class AdamWorkload:
    name: str
    description: str
    tensors: Tuple[Tuple[str, Tuple[int, ...]], ...]   # (name, shape)
    lr: float
    betas: Tuple[float, float]
    eps: float
    weight_decay: float
    grad_std: float
    seed: int

    @property
    def numel(self) -> int:
        return sum(int(np.prod(shape)) for _, shape in self.tensors)


ADAM_WORKLOADS: Dict[str, AdamWorkload] = {
    "gpt124m_adam": AdamWorkload(
        name="gpt124m_adam",
        description="124M record's DistAdam params: embed 50257x768, lm_head 50257x768, 48 scalars; "
                    "bf16 grads ~N(0,1e-3^2); lr 0.008, betas (0.8, 0.95), eps 1e-8, wd 0",
        tensors=(("embed", (50257, 768)), ("lm_head", (50257, 768)), ("scalars", (48,))),
        lr=0.008, betas=(0.8, 0.95), eps=1e-8, weight_decay=0.0, grad_std=1e-3, seed=20251205),
}


def adam_grad_bits_host(wl: AdamWorkload, index: int, step: int, numel: Optional[int] = None) -> np.ndarray:
    """bf16 bits of the gradient of tensor `index` (flattened; first `numel` elements)."""
    shape = wl.tensors[index][1]
    n = int(np.prod(shape)) if numel is None else numel
    rng = _rng(wl.seed, step, index, salt=2)
    return f32_to_bf16_bits(rng.standard_normal(n, dtype=np.float32) * np.float32(wl.grad_std))


def adam_param_host(wl: AdamWorkload, index: int, numel: Optional[int] = None) -> np.ndarray:
    shape = wl.tensors[index][1]
    n = int(np.prod(shape)) if numel is None else numel
    rng = _rng(wl.seed, 0, index, salt=3)
    return rng.standard_normal(n, dtype=np.float32) * np.float32(0.02)


def adam_grads_device(wl: AdamWorkload, index: int, step: int, device="cuda"):
    """bf16 gradient of tensor `index`, with its shape, drawn on `device`."""
    import torch
    gen = torch.Generator(device=device)
    gen.manual_seed(_torch_seed(wl.seed, "adam-grad", step, index))
    shape = wl.tensors[index][1]
    g = torch.randn(shape, generator=gen, device=device, dtype=torch.float32).mul_(wl.grad_std)
    return g.to(torch.bfloat16)


def adam_params_device(wl: AdamWorkload, index: int, device="cuda"):
    import torch
    gen = torch.Generator(device=device)
    gen.manual_seed(_torch_seed(wl.seed, "adam-param", index))
    shape = wl.tensors[index][1]
    return torch.randn(shape, generator=gen, device=device, dtype=torch.float32).mul_(0.02)
