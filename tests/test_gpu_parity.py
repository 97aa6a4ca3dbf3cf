"""GPU parity: the HIP path through the C ABI against the float64 oracle.

Each case prints its name, shapes and variant before touching the GPU.
Inputs come from the seeded generators in ``workloads``; expected values
come only from ``oracle``."""

import ctypes
import sys

import numpy as np
import pytest
import torch

import dimuon_newton_schulz_amd as D
import workloads as W
from parity import check_matrix, f32, run_gpu, run_oracle, to64

pytestmark = pytest.mark.gpu


def announce(msg):
    print(f"[case] {msg}", flush=True)
    sys.stdout.flush()


def cfg_of(wl, **kw):
    base = dict(lr=wl.lr, momentum=wl.mu, ns_steps=wl.ns_steps, w_dtype=wl.w_dtype, g_dtype=wl.g_dtype,
                mom_dtype=wl.mom_dtype, ns_dtype=wl.ns_dtype)
    base.update(kw)
    return D.StepConfig(**base)


def run_case(wl, variant, cfg, indices=None, scales=None, o_tol=None):
    announce(f"{wl.name} {variant} ns={cfg.ns_dtype} count={wl.count} "
             f"shapes={sorted(set(m.shape for m in wl.mats))}")
    gpu = run_gpu(wl, variant, cfg, scales=scales)
    idx = range(wl.count) if indices is None else indices
    errs = []
    for i in idx:
        ref = run_oracle(wl, variant, cfg, i, 1.0 if scales is None else scales[i])
        errs.append(check_matrix(gpu, ref, i, cfg, variant, wl, 1.0 if scales is None else scales[i], o_tol))
    return gpu, errs


def launch_kinds(step):
    """Kinds of the kernel launches one call of step() makes (the library's launch-event hook)."""
    lib = D.load_library()
    cap = 64
    events = [torch.cuda.Event(enable_timing=True) for _ in range(cap)]
    for e in events:
        e.record()
    torch.cuda.synchronize()
    handles = (ctypes.c_void_p * cap)(*[e.cuda_event for e in events])
    kinds = (ctypes.c_int32 * cap)()
    lib.muon_set_launch_events(handles, kinds, cap)
    try:
        step()
    finally:
        n = lib.muon_set_launch_events(None, None, 0)
    torch.cuda.synchronize()
    return [D.LAUNCH_KINDS[kinds[i]] for i in range(1, n)]


# ---------------------------------------------------------------------------
# Thin path (Gram side <= 32): two launches per padded Gram side
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("variant", ["muon", "dimuon"])
def test_lora_toy_4x16_f32(variant):
    wl = W.lora_toy(seed=0)
    run_case(wl, variant, cfg_of(wl))


def test_lora_toy_column_share_report():
    # The toy's report quantity (share of the squared step in the four
    # largest-scale columns) from the GPU step equals the oracle's, and
    # Dimuon lowers it below Muon's on every seed.
    def share(o):
        col = (o ** 2).sum(0)
        return col[-4:].sum() / col.sum()
    for seed in range(8):
        wl = W.lora_toy(seed=seed)
        cfg = cfg_of(wl)
        got = {}
        for variant in ("muon", "dimuon"):
            announce(f"{wl.name} seed {seed} {variant}: column share")
            gpu = run_gpu(wl, variant, cfg)
            ref = run_oracle(wl, variant, cfg, 0)
            got[variant] = share(gpu.o[0])
            assert abs(got[variant] - share(ref.o)) < 1e-5, (seed, variant, got[variant], share(ref.o))
        assert got["dimuon"] < got["muon"], (seed, got)


@pytest.mark.parametrize("variant", ["muon", "dimuon"])
@pytest.mark.parametrize("ns", ["bf16", "f32"])
def test_lora_batch_small(variant, ns):
    wl = W.lora_batch(pairs=6, rank=8, d=4096, seed=1)
    run_case(wl, variant, cfg_of(wl, ns_dtype=ns))


@pytest.mark.parametrize("shape", [(1, 40), (40, 1), (3, 1000), (1000, 3), (5, 333), (16, 2048), (2048, 16),
                                   (32, 1024), (1024, 32), (2, 9000), (9000, 2), (7, 4093)])
@pytest.mark.parametrize("variant", ["muon", "dimuon"])
def test_thin_ragged_shapes(shape, variant):
    for dt in ("f32", "bf16"):
        wl = W.random_batch([shape], dtype=dt, ns_dtype="f32", seed=hash(shape) % 97, variant=variant)
        run_case(wl, variant, cfg_of(wl))


@pytest.mark.parametrize("pairs,seed", [(150, 3), (64, 0)])
@pytest.mark.parametrize("variant", ["muon", "dimuon"])
def test_thin_large_batch(variant, pairs, seed):
    # 150 LoRA pairs: 2400 slices, more workgroups than the GPU holds at once;
    # 64 pairs: the full LoRA batch.  Every matrix is checked: the outlier
    # columns make some of them ill-conditioned, and those amplify Gram errors.
    wl = W.lora_batch(pairs=pairs, rank=8, d=4096, seed=seed)
    cfg = cfg_of(wl)
    params = [D.Param(w=m.w.cuda(), g=m.g.cuda(), mom=m.m_prev.cuda()) for m in wl.mats]
    fn = D.dimuon_step if variant == "dimuon" else D.muon_step
    announce(f"{wl.name} {variant}: launch kinds")
    kinds = launch_kinds(lambda: fn(params, cfg))
    assert kinds.count("thin_a") == 1 and kinds.count("thin_b") == 1, kinds
    del params
    run_case(wl, variant, cfg)


# ---------------------------------------------------------------------------
# General path (bf16 MFMA and fp32 GEMMs)
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("variant", ["muon", "dimuon"])
@pytest.mark.parametrize("ns", ["bf16", "f32"])
def test_general_ragged_mixed_batch(variant, ns):
    shapes = [(300, 700), (700, 300), (256, 256), (130, 1000), (1000, 130), (33, 500), (129, 129)]
    wl = W.random_batch(shapes, dtype="bf16", ns_dtype=ns, seed=3, variant=variant)
    run_case(wl, variant, cfg_of(wl))


@pytest.mark.parametrize("variant", ["muon", "dimuon"])
def test_general_f32_storage(variant):
    shapes = [(200, 333), (333, 200), (64, 1024)]
    wl = W.random_batch(shapes, dtype="f32", ns_dtype="f32", seed=4, variant=variant)
    run_case(wl, variant, cfg_of(wl))


@pytest.mark.parametrize("variant", ["muon", "dimuon"])
def test_maximum_extent(variant):
    # Long sides at the supported maximum of 65536, wide and tall: thin Gram
    # sides 8 and 32 (128 and 256 slices, the most a matrix may have) and a
    # general Gram side of 33 (padded to 128; its Gram is a product over
    # K = 65536), next to the thin path's largest Gram side.
    shapes = [(8, 65536), (65536, 32), (33, 65536), (65536, 40)]
    wl = W.random_batch(shapes, dtype="bf16", ns_dtype="bf16", seed=11, variant=variant)
    run_case(wl, variant, cfg_of(wl))


def test_gpt2_shapes_scaled():
    wl = W.gpt2_hidden(layers=1, d_model=256, seed=5)
    run_case(wl, "muon", cfg_of(wl))


@pytest.mark.parametrize("variant", ["muon", "dimuon"])
def test_square_spectrum_scaled(variant):
    wl = W.square_batch(count=2, n=512, seed=6, variant=variant)
    run_case(wl, variant, cfg_of(wl))


@pytest.mark.parametrize("variant", ["muon", "dimuon"])
def test_symmetric_tail_tiles(variant):
    # 8 x 2048^2: 288 upper 256-tiles, one full round on 256 CUs and a tail
    # of 32, which the planner runs as 128 x 128 tiles in a second launch of
    # each symmetric product.  The tail belongs to the last matrix.
    wl = W.square_batch(count=8, n=2048, seed=9, variant=variant)
    cfg = cfg_of(wl)
    params = [D.Param(w=m.w.cuda(), g=m.g.cuda(), mom=m.m_prev.cuda()) for m in wl.mats]
    fn = D.dimuon_step if variant == "dimuon" else D.muon_step
    announce(f"{wl.name} {variant}: launch kinds")
    kinds = launch_kinds(lambda: fn(params, cfg))
    assert kinds.count("gram") == 2 * cfg.ns_steps and kinds.count("poly") == 2 * cfg.ns_steps, kinds
    del params
    run_case(wl, variant, cfg, indices=[0, wl.count - 1])


@pytest.mark.parametrize("variant", ["muon", "dimuon"])
def test_combine_tail_tiles(variant):
    # 9 x (256 x 7936): 279 combine tiles of 256 x 256, one full round and a
    # tail of 23 that the planner runs as 128 x 128 tiles in a second launch.
    # The last matrix mixes both sizes, so its Dimuon norm partials come from
    # both launches.
    wl = W.random_batch([(256, 7936)] * 9, dtype="bf16", ns_dtype="bf16", seed=10, variant=variant)
    cfg = cfg_of(wl)
    params = [D.Param(w=m.w.cuda(), g=m.g.cuda(), mom=m.m_prev.cuda()) for m in wl.mats]
    fn = D.dimuon_step if variant == "dimuon" else D.muon_step
    announce(f"{wl.name} {variant}: launch kinds")
    kinds = launch_kinds(lambda: fn(params, cfg))
    assert kinds.count("combine") == 2 * cfg.ns_steps, kinds
    del params
    run_case(wl, variant, cfg, indices=[0, wl.count - 1])


@pytest.mark.parametrize("variant", ["muon", "dimuon"])
def test_combine_256x128_tiles(variant):
    # Gram side 512 (a multiple of 256), long side 1408 (an odd multiple of
    # 128): the combine runs 256 x 128 tiles (eight waves, one 32-column
    # block per wave), wide and tall matrices alike.
    shapes = [(512, 1408)] * 4 + [(1408, 512)] * 2
    wl = W.random_batch(shapes, dtype="bf16", ns_dtype="bf16", seed=12, variant=variant)
    run_case(wl, variant, cfg_of(wl), indices=[0, 3, 4, 5])


@pytest.mark.parametrize("steps", [5, 1, 0])
@pytest.mark.parametrize("variant", ["muon", "dimuon"])
def test_combine_padded_rows(variant, steps):
    # Gram sides 1152 and 1408 (odd multiples of 128): the combine runs on
    # 256 x 256 tiles over rows rounded up to 256, and the last iteration
    # stores and sums only the rows below the Gram side (with one iteration,
    # the first combine is also the last; with none, the exact-row combine
    # reads the padded iterate buffers); a matrix with a small Gram side
    # shares the batch.
    shapes = [(1152, 2048), (2048, 1152), (1408, 1536), (300, 700)]
    wl = W.random_batch(shapes, dtype="bf16", ns_dtype="bf16", seed=21, variant=variant)
    run_case(wl, variant, cfg_of(wl, ns_steps=steps))


@pytest.mark.parametrize("variant", ["muon", "dimuon"])
def test_moe_expert_full_size(variant):
    # One MoE expert at full size: 2048 x 1408 and 1408 x 2048.  The Gram
    # side 1408 is an odd multiple of 128, so the combine runs 128 x 256
    # tiles (eight waves) and the symmetric products 128 x 128 ones.
    wl = W.moe_experts(experts=1, d_model=2048, d_ff=1408, seed=11)
    run_case(wl, variant, cfg_of(wl))


def test_moe_scaled_zero_rows():
    wl = W.moe_experts(experts=2, d_model=384, d_ff=264, seed=7)
    gpu, _ = run_case(wl, "dimuon", cfg_of(wl))


# ---------------------------------------------------------------------------
# Method properties on the GPU
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("shapes", [[(8, 4096), (4096, 8), (4, 16)], [(300, 700), (700, 300), (256, 256)]])
def test_first_step_dimuon_equals_muon_bitwise(shapes):
    wl = W.random_batch(shapes, dtype="bf16", ns_dtype="bf16", seed=8, zero_prev=True)
    cfg = cfg_of(wl)
    announce(f"first-step identity {shapes}")
    a = run_gpu(wl, "muon", cfg)
    b = run_gpu(wl, "dimuon", cfg)
    for i in range(wl.count):
        np.testing.assert_array_equal(a.o[i], b.o[i])
        np.testing.assert_array_equal(a.w[i], b.w[i])
        np.testing.assert_array_equal(a.m[i], b.m[i])
        m, n = wl.mats[i].shape
        assert np.all(b.e[i] == 0)


def test_extensions_nesterov_decay_schedule_scale():
    shapes = [(8, 1024), (1024, 8), (200, 300), (300, 200)]
    # A stable schedule: each odd polynomial maps [0, 1] into a bounded band.
    sched = [(3.4445, -4.7750, 2.0315), (3.0, -3.2, 1.2), (2.6, -2.4, 0.8), (2.0, -1.5, 0.5), (1.5, -0.5, 0.0)]
    scales = [0.5, 2.0, 1.5, 0.25]
    for variant in ("muon", "dimuon"):
        wl = W.random_batch(shapes, dtype="bf16", ns_dtype="bf16", seed=9, variant=variant)
        cfg = cfg_of(wl, nesterov=True, weight_decay=0.1, coeff_schedule=sched)
        run_case(wl, variant, cfg, scales=scales)


@pytest.mark.parametrize("steps", [0, 1, 7])
def test_other_iteration_counts(steps):
    shapes = [(8, 512), (160, 300)]
    wl = W.random_batch(shapes, dtype="bf16", ns_dtype="bf16", seed=10)
    run_case(wl, "muon", cfg_of(wl, ns_steps=steps))


def test_zero_gradient_and_momentum_gives_zero_step():
    wl = W.random_batch([(8, 256), (130, 260)], dtype="bf16", ns_dtype="bf16", seed=11, zero_prev=True,
                        grad_std=0.0)
    for variant in ("muon", "dimuon"):
        gpu = run_gpu(wl, variant, cfg_of(wl))
        for i in range(wl.count):
            assert np.all(gpu.o[i] == 0)
            np.testing.assert_array_equal(gpu.w[i], to64(wl.mats[i].w))


def test_repeated_steps_track_oracle():
    # Three consecutive steps with fresh gradients; momentum carried on device.
    shapes = [(8, 2048), (256, 384)]
    wl = W.random_batch(shapes, dtype="f32", ns_dtype="f32", seed=12, variant="dimuon")
    cfg = cfg_of(wl)
    import oracle as O
    params = [D.Param(w=m.w.cuda().clone(), g=m.g.cuda().clone(), mom=m.m_prev.cuda().clone(),
                      o_out=torch.empty(m.shape, device="cuda")) for m in wl.mats]
    ws = D.workspace_for(params, cfg)
    ref_w = [to64(m.w) for m in wl.mats]
    ref_m = [to64(m.m_prev) for m in wl.mats]
    for step in range(3):
        grads = W.random_batch(shapes, dtype="f32", seed=100 + step)
        for p, gm in zip(params, grads.mats):
            p.g.copy_(gm.g.cuda())
        announce(f"repeated step {step}")
        D.dimuon_step(params, cfg, workspace=ws)
        torch.cuda.synchronize()
        for i, p in enumerate(params):
            r = O.dimuon_step(ref_w[i], to64(grads.mats[i].g), ref_m[i], lr=f32(cfg.lr), mu=f32(cfg.momentum),
                              mom_dtype="f32", w_dtype="f32", eps=f32(cfg.dimuon_eps))
            o = to64(p.o_out)
            rel = np.linalg.norm(o - r.o) / np.linalg.norm(r.o)
            assert rel < 1e-5, (step, i, rel)
            ref_w[i], ref_m[i] = to64(p.w), to64(p.mom)   # follow the GPU state


def test_plan_matches_stateless_step_bitwise():
    shapes = [(8, 4096), (4096, 8), (300, 700), (700, 300)]
    wl = W.random_batch(shapes, dtype="bf16", ns_dtype="bf16", seed=13, variant="dimuon")
    cfg = cfg_of(wl)
    announce(f"plan vs stateless {shapes}")
    ref = run_gpu(wl, "dimuon", cfg)
    params = [D.Param(w=m.w.cuda().clone(), g=m.g.cuda().clone(), mom=m.m_prev.cuda().clone(),
                      o_out=torch.empty(m.shape, device="cuda"),
                      energy_out=torch.empty(m.shape[0] + m.shape[1], device="cuda")) for m in wl.mats]
    plan = D.Plan(params, cfg, dimuon=True)
    plan.step()
    torch.cuda.synchronize()
    for i, p in enumerate(params):
        np.testing.assert_array_equal(to64(p.o_out), ref.o[i])
        np.testing.assert_array_equal(to64(p.w), ref.w[i])
        np.testing.assert_array_equal(to64(p.mom), ref.m[i])
        np.testing.assert_array_equal(p.energy_out.cpu().numpy(), ref.e[i])
    # a second step with a new learning rate follows the oracle from the GPU state
    w1 = [to64(p.w) for p in params]
    m1 = [to64(p.mom) for p in params]
    plan.set_lr(0.005)
    plan.step()
    torch.cuda.synchronize()
    import oracle as O
    for i, p in enumerate(params):
        r = O.dimuon_step(w1[i], to64(wl.mats[i].g), m1[i], lr=f32(0.005), mu=f32(cfg.momentum),
                          mom_dtype="bf16", w_dtype="bf16", eps=f32(cfg.dimuon_eps))
        assert np.max(np.abs(to64(p.o_out) - r.o)) < 2e-2
    plan.close()


@pytest.mark.parametrize("shapes", [[(8, 4096), (4096, 8), (3, 1000), (16, 2048)], [(300, 700), (8, 300)]])
def test_plan_steps_with_cached_energies_match_stateless(shapes):
    # A Dimuon plan reuses the energies its previous step computed; three plan
    # steps must equal three stateless steps bit for bit, and a reset must be
    # harmless.
    wl = W.random_batch(shapes, dtype="f32", ns_dtype="bf16", seed=14, variant="dimuon")
    cfg = cfg_of(wl)
    announce(f"cached energies {shapes}")
    def fresh():
        return [D.Param(w=m.w.cuda().clone(), g=m.g.cuda().clone(), mom=m.m_prev.cuda().clone(),
                        o_out=torch.empty(m.shape, device="cuda"),
                        energy_out=torch.empty(m.shape[0] + m.shape[1], device="cuda")) for m in wl.mats]
    a, b = fresh(), fresh()
    plan = D.Plan(a, cfg, dimuon=True)
    for step in range(3):
        if step == 2:
            plan.reset()
        plan.step()
        D.dimuon_step(b, cfg)
        torch.cuda.synchronize()
        for pa, pb in zip(a, b):
            for name in ("w", "mom", "o_out", "energy_out"):
                np.testing.assert_array_equal(getattr(pa, name).cpu().numpy(), getattr(pb, name).cpu().numpy(),
                                              err_msg=f"step {step} {name}")
    plan.close()
