"""Parity at the full benchmark sizes, through the plan API that bench.py
times (same launch configuration).  The oracle recomputes sampled matrices
of each batch in full (float64); energies and momentum of the sampled
matrices are checked bit for bit.  Inputs are drawn on the device by the
seeded generators and copied to the host for the oracle."""

import sys

import numpy as np
import pytest
import torch

import dimuon_newton_schulz_amd as D
import workloads as W
from parity import check_matrix, run_gpu, run_oracle, to64, GpuResult

pytestmark = pytest.mark.gpu


def announce(msg):
    print(f"[case] {msg}", flush=True)


_SQUARE = {}


def square_inputs():
    """The 8 x 4096^2 batch, built once per session (its 32 float64 QRs run
    on the host); each test steps clones of its tensors."""
    if "wl" not in _SQUARE:
        _SQUARE["wl"] = W.square_batch(device="cuda")
    return _SQUARE["wl"]


def run_plan(wl, variant, sample):
    """One plan step over the whole batch (on clones of the workload's
    tensors); O and energies captured for `sample`."""
    cfg = D.StepConfig(lr=wl.lr, momentum=wl.mu, ns_steps=wl.ns_steps, w_dtype=wl.w_dtype,
                       g_dtype=wl.g_dtype, mom_dtype=wl.mom_dtype, ns_dtype=wl.ns_dtype)
    host = {}
    params = []
    for i, m in enumerate(wl.mats):
        if i in sample:
            host[i] = (m.w.cpu().clone(), m.g.cpu().clone(), m.m_prev.cpu().clone())
        rows, cols = m.shape
        params.append(D.Param(
            w=m.w.clone(), g=m.g.clone(), mom=m.m_prev.clone(),
            o_out=torch.full((rows, cols), float("nan"), device=m.w.device) if i in sample else None,
            energy_out=(torch.full((rows + cols,), float("nan"), device=m.w.device)
                        if (i in sample and variant == "dimuon") else None)))
    plan = D.Plan(params, cfg, dimuon=(variant == "dimuon"))
    plan.step()
    torch.cuda.synchronize()
    plan.close()
    return cfg, params, host


def compare(wl, variant, cfg, params, host, sample):
    # Rebuild a small host workload holding the sampled matrices' inputs.
    sub = W.Workload(wl.name, [W.MatrixInput(*host[i]) for i in sample], wl.w_dtype, wl.g_dtype,
                     wl.mom_dtype, wl.ns_dtype, wl.lr, wl.mu, variant)
    gpu = GpuResult(w=[to64(params[i].w) for i in sample], m=[to64(params[i].mom) for i in sample],
                    o=[to64(params[i].o_out) for i in sample],
                    e=[params[i].energy_out.cpu().numpy() if params[i].energy_out is not None else None
                       for i in sample])
    errs = []
    for j, i in enumerate(sample):
        announce(f"oracle on matrix {i} {sub.mats[j].shape}")
        ref = run_oracle(sub, variant, cfg, j)
        errs.append(check_matrix(gpu, ref, j, cfg, variant, sub))
    return errs


def test_fullsize_lora_batch_dimuon():
    wl = W.lora_batch(device="cuda")
    announce(f"{wl.name} dimuon, all {wl.count} matrices")
    sample = list(range(0, wl.count, 5)) + [wl.count - 1]
    cfg, params, host = run_plan(wl, "dimuon", set(sample))
    compare(wl, "dimuon", cfg, params, host, sample)


def test_fullsize_gpt2_muon():
    wl = W.gpt2_hidden(device="cuda")
    announce(f"{wl.name} muon")
    sample = [0, 1, 2, 3, 46, 47]          # every shape, first and last layer
    cfg, params, host = run_plan(wl, "muon", set(sample))
    compare(wl, "muon", cfg, params, host, sample)


@pytest.mark.parametrize("variant", ["dimuon", "muon"])
def test_fullsize_square_4096(variant):
    wl = square_inputs()
    announce(f"{wl.name} {variant}")
    sample = [0, 7]
    cfg, params, host = run_plan(wl, variant, set(sample))
    compare(wl, variant, cfg, params, host, sample)


def test_fullsize_moe_dimuon():
    wl = W.moe_experts(device="cuda")
    announce(f"{wl.name} dimuon")
    sample = [0, 1, 126, 127]              # up and down, first and last expert
    cfg, params, host = run_plan(wl, "dimuon", set(sample))
    compare(wl, "dimuon", cfg, params, host, sample)


@pytest.mark.parametrize("variant", ["dimuon", "muon"])
def test_fullsize_fp32_products(variant):
    # The fp32 Newton-Schulz products at the largest shapes of the sets: one
    # 4096^2 matrix of the square recipe and one MoE expert pair (2048 x 1408
    # and 1408 x 2048), each within the fp32 bound of 1e-5 relative (measured
    # 4.5e-6 and 3-4e-6).
    for wl in (W.square_batch(count=1, n=4096, seed=3, device="cuda", variant=variant),
               W.moe_experts(experts=1, device="cuda")):
        cfg = D.StepConfig(lr=wl.lr, momentum=wl.mu, ns_steps=wl.ns_steps, w_dtype=wl.w_dtype,
                           g_dtype=wl.g_dtype, mom_dtype=wl.mom_dtype, ns_dtype="f32")
        announce(f"{wl.name} {variant}, fp32 products")
        gpu = run_gpu(wl, variant, cfg)
        for i in range(wl.count):
            announce(f"oracle on matrix {i} {wl.mats[i].shape}")
            check_matrix(gpu, run_oracle(wl, variant, cfg, i), i, cfg, variant, wl)


@pytest.mark.parametrize("name", ["lora", "gpt2", "square", "moe"])
def test_fullsize_plan_steps_repeatable(name):
    # A plan step over the full benchmark batch, run twice from the same
    # inputs, gives the same W and M bit for bit (every matrix; compared on
    # the device).
    wl, variant = {"lora": lambda: (W.lora_batch(device="cuda"), "dimuon"),
                   "gpt2": lambda: (W.gpt2_hidden(device="cuda"), "muon"),
                   "square": lambda: (square_inputs(), "dimuon"),
                   "moe": lambda: (W.moe_experts(device="cuda"), "dimuon")}[name]()
    cfg = D.StepConfig(lr=wl.lr, momentum=wl.mu, ns_steps=wl.ns_steps, w_dtype=wl.w_dtype,
                       g_dtype=wl.g_dtype, mom_dtype=wl.mom_dtype, ns_dtype=wl.ns_dtype)
    announce(f"{wl.name} {variant}: two plan steps from the same inputs")
    runs = []
    for _ in range(2):
        params = [D.Param(w=m.w.clone(), g=m.g.clone(), mom=m.m_prev.clone()) for m in wl.mats]
        plan = D.Plan(params, cfg, dimuon=(variant == "dimuon"))
        plan.step()
        torch.cuda.synchronize()
        plan.close()
        runs.append(params)
    for i, (a, b) in enumerate(zip(*runs)):
        assert torch.equal(a.w, b.w), f"matrix {i}: W differs between identical steps"
        assert torch.equal(a.mom, b.mom), f"matrix {i}: M differs between identical steps"
