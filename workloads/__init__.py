"""Seeded synthetic inputs for the Muon / Dimuon step.

This module only draws inputs.  It holds none of the optimizer's arithmetic,
and both the HIP path's tests and the oracle read the tensors it returns.

Every draw comes from ``numpy.random.default_rng(SeedSequence([config,
matrix, role]))`` (host) or from a ``torch.Generator`` seeded from that same
SeedSequence (device); the square set's orthogonal factors are always
float64 QRs on the host.  Roles are G = 0, previous momentum = 1, W = 2,
U = 3, V = 4, and structure = 5.  Structure covers channel scales, outlier
channels, token counts and zero rows.  Host draws are float64 and are then
cast to the storage dtype.

The five workloads follow the benchmark configurations.  Every size is a
parameter, so tests can draw smaller instances of the same recipe.
"""

from __future__ import annotations

import os
from dataclasses import dataclass, field
from typing import List, Optional

import numpy as np
import torch

G_ROLE, MPREV_ROLE, W_ROLE, U_ROLE, V_ROLE, STRUCT_ROLE = 0, 1, 2, 3, 4, 5

_TORCH_DTYPES = {"f32": torch.float32, "bf16": torch.bfloat16}


def host_rng(config: int, matrix: int, role: int) -> np.random.Generator:
    return np.random.default_rng(np.random.SeedSequence([config, matrix, role]))


def device_generator(config: int, matrix: int, role: int, device) -> torch.Generator:
    seed = int(np.random.SeedSequence([config, matrix, role]).generate_state(1, np.uint64)[0])
    gen = torch.Generator(device=device)
    gen.manual_seed(seed & ((1 << 63) - 1))
    return gen


@dataclass
class MatrixInput:
    """One 2-D parameter with its gradient and previous momentum."""
    w: torch.Tensor
    g: torch.Tensor
    m_prev: torch.Tensor

    @property
    def shape(self):
        return tuple(self.w.shape)


@dataclass
class Workload:
    name: str
    mats: List[MatrixInput]
    w_dtype: str
    g_dtype: str
    mom_dtype: str
    ns_dtype: str
    lr: float
    mu: float
    variant: str                  # "muon" or "dimuon"
    ns_steps: int = 5
    notes: dict = field(default_factory=dict)

    @property
    def count(self) -> int:
        return len(self.mats)

    def elements(self) -> int:
        return sum(int(np.prod(m.shape)) for m in self.mats)


def _to(x: np.ndarray, dtype: str, device) -> torch.Tensor:
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float64))
    return t.to(_TORCH_DTYPES[dtype]).to(device).contiguous()


def _normal(config, matrix, role, shape, device, std=1.0) -> torch.Tensor:
    """Standard-normal draw (times ``std``), float64 on host or float32 on device."""
    if device is None or str(device) == "cpu":
        return torch.from_numpy(host_rng(config, matrix, role).standard_normal(shape) * std)
    gen = device_generator(config, matrix, role, device)
    return torch.randn(shape, generator=gen, device=device, dtype=torch.float32) * std


def _cast(t: torch.Tensor, dtype: str, device) -> torch.Tensor:
    dev = "cpu" if device is None else device
    return t.to(_TORCH_DTYPES[dtype]).to(dev).contiguous()


# ---------------------------------------------------------------------------
# Config 1: LoRA factor A, 4 x 16 fp32, log-spaced column scales 0.1 .. 10
# ---------------------------------------------------------------------------

def toy_column_scales(n: int = 16) -> np.ndarray:
    """s_j = 10**(-1 + 2 j / (n - 1)): n values evenly spaced in log, 0.1..10."""
    j = np.arange(n, dtype=np.float64)
    return 10.0 ** (-1.0 + 2.0 * j / (n - 1))


def lora_toy(seed: int = 0, rank: int = 4, n: int = 16, device=None) -> Workload:
    s2 = toy_column_scales(n) ** 2
    cfg = 1000 + seed
    g = _normal(cfg, 0, G_ROLE, (rank, n), None) * torch.from_numpy(s2)[None, :]
    mp = _normal(cfg, 0, MPREV_ROLE, (rank, n), None) * torch.from_numpy(s2)[None, :]
    w = _normal(cfg, 0, W_ROLE, (rank, n), None, std=0.02)
    mats = [MatrixInput(_cast(w, "f32", device), _cast(g, "f32", device),
                        _cast(mp, "f32", device))]
    return Workload("lora_toy_4x16_f32", mats, "f32", "f32", "f32", "f32",
                    lr=0.01, mu=0.95, variant="dimuon",
                    notes={"column_scales": toy_column_scales(n)})


# ---------------------------------------------------------------------------
# Config 2: LoRA batch, pairs of A (r x d) and B (d x r), fp32 master
# ---------------------------------------------------------------------------

def lora_batch(pairs: int = 64, rank: int = 8, d: int = 4096, outliers: int = 6,
               outlier_factor: float = 20.0, seed: int = 0, device=None) -> Workload:
    """Channel scales s_j ~ lognormal(0, 1) over the d channels, ``outliers``
    of them (without replacement) multiplied by ``outlier_factor``.  G and the
    previous momentum are N(0,1) * s_j^2 along the d axis of both factors."""
    cfg = 2000 + seed
    mats = []
    for p in range(pairs):
        srng = host_rng(cfg, p, STRUCT_ROLE)
        s = np.exp(srng.standard_normal(d))
        s[srng.choice(d, size=min(outliers, d), replace=False)] *= outlier_factor
        s2 = torch.from_numpy(s * s)
        if device is not None and str(device) != "cpu":
            s2 = s2.to(device=device, dtype=torch.float32)
        for side in range(2):
            idx = 2 * p + side
            shape = (rank, d) if side == 0 else (d, rank)
            scale = s2[None, :] if side == 0 else s2[:, None]
            g = _normal(cfg, idx, G_ROLE, shape, device) * scale
            mp = _normal(cfg, idx, MPREV_ROLE, shape, device) * scale
            w = _normal(cfg, idx, W_ROLE, shape, device, std=0.02)
            mats.append(MatrixInput(_cast(w, "f32", device), _cast(g, "f32", device),
                                    _cast(mp, "f32", device)))
    return Workload(f"lora_batch_{pairs}x({rank}x{d}+{d}x{rank})_f32", mats,
                    "f32", "f32", "f32", "bf16", lr=0.02, mu=0.95, variant="dimuon")


# ---------------------------------------------------------------------------
# Config 3: GPT-2-small hidden matrices, bf16, Muon
# ---------------------------------------------------------------------------

def gpt2_hidden(layers: int = 12, d_model: int = 768, seed: int = 0,
                device=None) -> Workload:
    """Per layer: qkv (d x 3d), attention proj (d x d), fc (d x 4d),
    mlp proj (4d x d).  G ~ N(0, 0.02^2); the previous momentum is the
    previous synthetic step's gradient, drawn the same way."""
    cfg = 3000 + seed
    shapes = [(d_model, 3 * d_model), (d_model, d_model),
              (d_model, 4 * d_model), (4 * d_model, d_model)]
    mats = []
    for layer in range(layers):
        for k, shape in enumerate(shapes):
            idx = 4 * layer + k
            g = _normal(cfg, idx, G_ROLE, shape, device, std=0.02)
            mp = _normal(cfg, idx, MPREV_ROLE, shape, device, std=0.02)
            w = _normal(cfg, idx, W_ROLE, shape, device, std=0.02)
            mats.append(MatrixInput(_cast(w, "bf16", device), _cast(g, "bf16", device),
                                    _cast(mp, "bf16", device)))
    return Workload(f"gpt2_small_{layers}x4_bf16", mats, "bf16", "bf16", "bf16",
                    "bf16", lr=0.02, mu=0.95, variant="muon")


# ---------------------------------------------------------------------------
# Config 4: square matrices with a prescribed spectrum, bf16
# ---------------------------------------------------------------------------

def square_spectrum(n: int, s_max: float = 20.0, s_min: float = 1e-3) -> np.ndarray:
    """n singular values evenly spaced in log from s_max down to s_min."""
    if n == 1:
        return np.array([s_max])
    return np.exp(np.linspace(np.log(s_max), np.log(s_min), n))


def haar_orthogonal(config: int, matrix: int, role: int, n: int) -> np.ndarray:
    """Haar-random orthogonal n x n, float64 on the host: Householder QR of
    a Gaussian draw, columns sign-fixed so that R has a positive diagonal."""
    a = host_rng(config, matrix, role).standard_normal((n, n))
    q, r = np.linalg.qr(a)
    sign = np.sign(np.diag(r))
    sign[sign == 0] = 1.0
    return q * sign[None, :]


def _haar_many(jobs, workers: int = 0):
    """haar_orthogonal for every (config, matrix, role, n) of ``jobs``, several
    QRs at a time (LAPACK's QR uses few cores well; a few concurrent ones with
    two BLAS threads each finish sooner)."""
    from concurrent.futures import ThreadPoolExecutor
    if len(jobs) <= 1 or jobs[0][3] < 512:
        return [haar_orthogonal(*j) for j in jobs]
    cores = os.cpu_count() or 2
    workers = workers or max(1, min(len(jobs), min(cores, 16) // 2))
    try:
        from threadpoolctl import threadpool_limits
        limit = threadpool_limits(2)
    except Exception:  # pragma: no cover
        limit = None
    try:
        with ThreadPoolExecutor(workers) as ex:
            return list(ex.map(lambda j: haar_orthogonal(*j), jobs))
    finally:
        if limit is not None:
            limit.restore_original_limits()


def square_batch(count: int = 8, n: int = 4096, seed: int = 0, device=None,
                 variant: str = "dimuon", with_factors: bool = False,
                 zero_prev: bool = False) -> Workload:
    """G = U diag(sigma) V^T with Haar U, V and sigma log-spaced 20 .. 1e-3.
    The previous momentum is an independent draw of the same kind (the
    step-0 gradient: after a step from zero momentum, M equals it), or zero
    with ``zero_prev`` (the step from zero momentum, whose exact result is
    U f(sigma / ||sigma||) V^T with f the iteration's scalar polynomial).

    U and V always come from a float64 QR on the host; the products
    U diag(sigma) V^T are float64, on ``device`` when one is given (there
    they are plain matrix products), then rounded to bf16."""
    cfg = 4000 + seed
    sigma = square_spectrum(n)
    jobs = []
    for i in range(count):
        jobs += [(cfg, i, U_ROLE, n), (cfg, i, V_ROLE, n)]
        if not zero_prev:
            jobs += [(cfg + 500, i, U_ROLE, n), (cfg + 500, i, V_ROLE, n)]
    qs = _haar_many(jobs)
    on_dev = device is not None and str(device) != "cpu"
    dev = device if on_dev else "cpu"

    def product(u, v):
        ut = torch.from_numpy(u).to(dev)
        vt = torch.from_numpy(v).to(dev)
        st = torch.from_numpy(sigma).to(dev)
        return (ut * st[None, :]) @ vt.T

    mats, factors = [], []
    per = 2 if zero_prev else 4
    for i in range(count):
        u, v = qs[per * i], qs[per * i + 1]
        g = product(u, v)
        if zero_prev:
            mp = torch.zeros((n, n), dtype=torch.float64, device=dev)
        else:
            mp = product(qs[per * i + 2], qs[per * i + 3])
        w = _normal(cfg, i, W_ROLE, (n, n), device, std=0.02)
        mats.append(MatrixInput(_cast(w, "bf16", device), _cast(g, "bf16", device),
                                _cast(mp, "bf16", device)))
        if with_factors:
            factors.append((u, v))
        del g, mp
    wl = Workload(f"square_{count}x{n}x{n}_bf16", mats, "bf16", "bf16", "bf16", "bf16",
                  lr=0.02, mu=0.95, variant=variant,
                  notes={"sigma": sigma})
    if with_factors:
        wl.notes["factors"] = factors
    return wl


# ---------------------------------------------------------------------------
# Config 5: MoE expert set, mixed up/down shapes, bf16, Dimuon
# ---------------------------------------------------------------------------

def moe_experts(experts: int = 64, d_model: int = 2048, d_ff: int = 1408,
                tokens_mean: float = 32.0, zero_row_frac: float = 0.10,
                seed: int = 0, device=None) -> Workload:
    """Per expert an up (d_model x d_ff) and a down (d_ff x d_model) matrix.
    G_ij = N(0,1) * k_i with k_i ~ Poisson(tokens_mean) per row; the previous
    momentum is drawn the same way with ``zero_row_frac`` of its rows (chosen
    uniformly per matrix) set to zero."""
    cfg = 5000 + seed
    mats = []
    for e in range(experts):
        for side, shape in enumerate([(d_model, d_ff), (d_ff, d_model)]):
            idx = 2 * e + side
            srng = host_rng(cfg, idx, STRUCT_ROLE)
            rows = shape[0]
            k_g = torch.from_numpy(srng.poisson(tokens_mean, rows).astype(np.float64))
            k_m = torch.from_numpy(srng.poisson(tokens_mean, rows).astype(np.float64))
            zero = srng.choice(rows, size=int(round(zero_row_frac * rows)), replace=False)
            k_m[torch.from_numpy(zero)] = 0.0
            if device is not None and str(device) != "cpu":
                k_g = k_g.to(device=device, dtype=torch.float32)
                k_m = k_m.to(device=device, dtype=torch.float32)
            g = _normal(cfg, idx, G_ROLE, shape, device) * k_g[:, None]
            mp = _normal(cfg, idx, MPREV_ROLE, shape, device) * k_m[:, None]
            w = _normal(cfg, idx, W_ROLE, shape, device, std=0.02)
            mats.append(MatrixInput(_cast(w, "bf16", device), _cast(g, "bf16", device),
                                    _cast(mp, "bf16", device)))
    return Workload(f"moe_{experts}x({d_model}x{d_ff}+{d_ff}x{d_model})_bf16", mats,
                    "bf16", "bf16", "bf16", "bf16", lr=0.02, mu=0.95, variant="dimuon")


# ---------------------------------------------------------------------------
# Generic random batch for edge-case tests
# ---------------------------------------------------------------------------

def random_batch(shapes, dtype: str = "bf16", ns_dtype: Optional[str] = None,
                 seed: int = 0, variant: str = "muon", zero_prev: bool = False,
                 device=None, grad_std: float = 1.0) -> Workload:
    cfg = 9000 + seed
    mats = []
    for i, shape in enumerate(shapes):
        g = _normal(cfg, i, G_ROLE, shape, device, std=grad_std)
        if zero_prev:
            mp = torch.zeros(shape, dtype=torch.float64)
        else:
            mp = _normal(cfg, i, MPREV_ROLE, shape, device, std=grad_std)
        w = _normal(cfg, i, W_ROLE, shape, device, std=0.02)
        mats.append(MatrixInput(_cast(w, dtype, device), _cast(g, dtype, device),
                                _cast(mp, dtype, device)))
    return Workload(f"random_{len(shapes)}_{dtype}", mats, dtype, dtype, dtype,
                    ns_dtype or dtype, lr=0.02, mu=0.95, variant=variant)


CONFIG_BUILDERS = {
    "c1": lora_toy,
    "c2": lora_batch,
    "c3": gpt2_hidden,
    "c4": square_batch,
    "c5": moe_experts,
}
