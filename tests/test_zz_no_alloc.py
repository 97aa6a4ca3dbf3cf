"""The allocation-free entry point (muon_step_noalloc) against the entry
point with a caller workspace (muon_step / dimuon_step): the same kernels on
the same inputs, so every output must agree bit for bit.  Two calls in a row
share the library's static scratch, the second with a smaller batch."""

import sys

import numpy as np
import pytest
import torch

import dimuon_newton_schulz_amd as D
import workloads as W

pytestmark = pytest.mark.gpu


def announce(msg):
    print(f"[case] {msg}", flush=True)
    sys.stdout.flush()


def params_of(wl, device="cuda"):
    out = []
    for m in wl.mats:
        rows, cols = m.shape
        out.append(D.Param(w=m.w.to(device).clone(), g=m.g.to(device).clone(), mom=m.m_prev.to(device).clone(),
                           o_out=torch.full((rows, cols), float("nan"), device=device),
                           energy_out=torch.full((rows + cols,), float("nan"), device=device)))
    return out


def compare(a, b, ctx):
    for i, (pa, pb) in enumerate(zip(a, b)):
        for name in ("w", "mom", "o_out", "energy_out"):
            np.testing.assert_array_equal(getattr(pa, name).float().cpu().numpy(),
                                          getattr(pb, name).float().cpu().numpy(),
                                          err_msg=f"{ctx}: matrix {i} {name}")


def run_both(wl, variant):
    cfg = D.StepConfig(lr=wl.lr, momentum=wl.mu, ns_steps=wl.ns_steps, w_dtype=wl.w_dtype, g_dtype=wl.g_dtype,
                       mom_dtype=wl.mom_dtype, ns_dtype=wl.ns_dtype)
    shapes = [m.shape for m in wl.mats]
    announce(f"no-alloc vs workspace entry point: {variant} {shapes}")
    ref = params_of(wl)
    (D.dimuon_step if variant == "dimuon" else D.muon_step)(ref, cfg)
    got = params_of(wl)
    D.muon_step_noalloc(got, cfg, dimuon=(variant == "dimuon"))
    torch.cuda.synchronize()
    compare(ref, got, f"{variant} {shapes}")
    return got


def test_noalloc_matches_workspace_entry_point():
    big = [(8, 4096), (4096, 8), (300, 700), (700, 300), (33, 500), (256, 1024)]
    small = [(16, 2048), (130, 260)]
    for variant in ("dimuon", "muon"):
        run_both(W.random_batch(big, dtype="bf16", ns_dtype="bf16", seed=31, variant=variant), variant)
        # The second call: a smaller batch over the same scratch.
        run_both(W.random_batch(small, dtype="bf16", ns_dtype="bf16", seed=32, variant=variant), variant)
    # fp32 storage and products, thin and general
    wl = W.random_batch([(8, 1024), (200, 333)], dtype="f32", ns_dtype="f32", seed=33, variant="dimuon")
    run_both(wl, "dimuon")


def test_noalloc_rejects_batches_beyond_the_scratch():
    t = torch.zeros((4096, 4096), dtype=torch.bfloat16, device="cuda")
    p = D.Param(w=t, g=t.clone(), mom=t.clone())
    need = D.muon_workspace_bytes([p], D.StepConfig())
    assert need > D.NOALLOC_MAX_BYTES
    with pytest.raises(D.MuonError) as e:
        D.muon_step_noalloc([p], D.StepConfig(), dimuon=False)
    assert e.value.status == 3 and "static scratch" in str(e.value)
    assert torch.count_nonzero(p.w).item() == 0
