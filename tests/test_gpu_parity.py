"""GPU parity: the HIP path through the C ABI against the float64 oracle.

Each case prints its name, shapes and variant before touching the GPU.
Inputs come from the seeded generators in ``workloads``; expected values
come only from ``oracle``."""

import ctypes
import os
import sys

import numpy as np
import pytest
import torch

import dimuon_newton_schulz_amd as D
import workloads as W
from parity import RECORDS, check_matrix, f32, run_gpu, run_oracle, to64

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


@pytest.mark.parametrize("wdt", ["bf16", "f32"])
def test_muon_streaming_passes_fused(wdt):
    # The momentum update runs inside the prescale launch (M_t is not read
    # back).  Dimuon's factors need the energies of M_{t-1} first: a
    # stateless call computes them in a pass of their own, a plan step reads
    # the ones its previous step left (the fused pass computes those of M_t),
    # and a reset brings the extra pass back.  Ragged and whole 16-byte runs,
    # wide and tall, f32 and bf16 storage.
    shapes = [(200, 333), (333, 200), (256, 1024), (1000, 130), (8, 512)]
    wl = W.random_batch(shapes, dtype=wdt, ns_dtype="bf16", seed=17)
    cfg = cfg_of(wl)
    params = [D.Param(w=m.w.cuda().clone(), g=m.g.cuda().clone(), mom=m.m_prev.cuda().clone()) for m in wl.mats]
    announce(f"fused streaming passes {wdt}: launch kinds")
    kinds = launch_kinds(lambda: D.muon_step(params, cfg))
    assert kinds.count("momentum_prescale") == 1 and kinds.count("update") == 1, kinds
    assert not {"momentum", "prescale"} & set(kinds), kinds
    f32 = launch_kinds(lambda: D.muon_step(params, cfg_of(wl, ns_dtype="f32")))
    assert "momentum_prescale" in f32 and "momentum" not in f32, f32
    dim = launch_kinds(lambda: D.dimuon_step(params, cfg))
    assert dim.count("energy") == 1 and dim.count("momentum_prescale") == 1, dim
    assert not {"momentum", "prescale"} & set(dim), dim
    plan = D.Plan(params, cfg, dimuon=True)
    first, second = launch_kinds(plan.step), launch_kinds(plan.step)
    plan.reset()
    third = launch_kinds(plan.step)
    plan.close()
    assert "energy" in first and "energy" not in second and "energy" in third, (first, second, third)
    del params
    run_case(wl, "muon", cfg)
    run_case(wl, "muon", cfg_of(wl, nesterov=True, weight_decay=0.1), scales=[0.5, 2.0, 1.0, 1.5, 0.25])


def test_muon_update_in_last_combine():
    # Muon with bf16 weights: for a matrix whose rows are whole 8-element
    # runs, the last combine applies the update (O rounded to bf16 as the last
    # iterate is stored), and the update pass runs only for the others.  Wide
    # and tall, rows beyond the Gram side's padding, a ragged long side, with
    # and without weight decay and per-matrix scales, against the oracle.
    # (The first-step identity test checks it bit for bit against Dimuon,
    # which always takes the update pass.)
    shapes = [(384, 1024), (1024, 384), (300, 696), (700, 296), (129, 136)]
    wl = W.random_batch(shapes, dtype="bf16", ns_dtype="bf16", seed=21)
    cfg = cfg_of(wl)
    params = [D.Param(w=m.w.cuda().clone(), g=m.g.cuda().clone(), mom=m.m_prev.cuda().clone()) for m in wl.mats]
    announce("update in the last combine: launch kinds")
    assert "update" not in launch_kinds(lambda: D.muon_step(params, cfg))
    assert launch_kinds(lambda: D.dimuon_step(params, cfg)).count("update") == 1
    mixed = params + [D.Param(w=params[0].w[:, :999].contiguous(), g=params[0].g[:, :999].contiguous(),
                              mom=params[0].mom[:, :999].contiguous())]
    assert launch_kinds(lambda: D.muon_step(mixed, cfg)).count("update") == 1
    assert launch_kinds(lambda: D.muon_step(params, cfg_of(wl, ns_dtype="f32"))).count("update") == 1
    del params, mixed
    run_case(wl, "muon", cfg)
    run_case(wl, "muon", cfg_of(wl, nesterov=True, weight_decay=0.1), scales=[0.5, 2.0, 1.0, 1.5, 0.25])


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


def scalar_iteration(x, steps, coeffs):
    """The quintic's action on one singular value, applied `steps` times."""
    a, b, c = coeffs
    for _ in range(steps):
        x = a * x + b * x ** 3 + c * x ** 5
    return x


@pytest.mark.parametrize("variant", ["muon", "dimuon"])
def test_square_closed_form_from_zero_momentum(variant):
    # The orthogonaliser keeps the singular vectors and maps every singular
    # value through the scalar quintic (sitech.ge Muon blog, "SVD-ի փոխարեն՝
    # Newton–Schulz"; "Muon Optimizer 정리", "Newton-Schulz 직교화").  From
    # zero momentum, G = U diag(sigma) V^T therefore gives
    # O = U f^5(sigma / ||sigma||_2) V^T, up to the bf16 rounding of G; a zero
    # previous momentum switches Dimuon's conditioning off ("Dimuon: LoRA 에
    # 맞춰 다시 짠 Muon", "왜 「지난」 모멘텀인가").  Checked against the closed
    # form itself, not the oracle: 2048 x 2048, sigma log-spaced 20 .. 1e-3.
    n = 2048
    wl = W.square_batch(count=1, n=n, seed=7, device="cuda", variant=variant, with_factors=True,
                        zero_prev=True)
    cfg = cfg_of(wl)
    announce(f"closed form {n}x{n} {variant}")
    gpu = run_gpu(wl, variant, cfg)
    u, v = wl.notes["factors"][0]
    sigma = wl.notes["sigma"]
    coeffs = tuple(f32(x) for x in (cfg.a, cfg.b, cfg.c))
    expect = (u * scalar_iteration(sigma / np.linalg.norm(sigma), cfg.ns_steps, coeffs)[None, :]) @ v.T
    o = gpu.o[0]
    err = float(np.max(np.abs(o - expect)))
    rel = float(np.linalg.norm(o - expect) / np.linalg.norm(expect))
    print(f"[parity] closed form {n}x{n} {variant}: max|O - U f5(s) V^T| = {err:.3e}, rel F {rel:.2e}, "
          f"max|O| {np.abs(expect).max():.3f}", flush=True)
    RECORDS.append({"case": f"closed form U f5(sigma) V^T {n}x{n} ({variant})", "max_abs_dO": err, "rel_F_dO": rel,
                    "norm_ratio_m1": float(np.linalg.norm(o) / np.linalg.norm(expect) - 1.0),
                    "max_abs_O": float(np.abs(expect).max()), "ns": cfg.ns_dtype, "variant": variant,
                    "test": os.environ.get("PYTEST_CURRENT_TEST", "").split(" ")[0]})
    assert err <= 2e-2, err
    np.testing.assert_array_equal(gpu.m[0], to64(wl.mats[0].g))   # M = mu * 0 + G exactly


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
    # Two experts at half the configured sides (1024 x 704 and 704 x 1024),
    # 10% zero rows in the previous momentum (factor exactly 10 on those rows).
    # The contract bound is stated at the configured sizes: on much smaller
    # experts the entries of O grow while the bf16 error of the iteration
    # does not shrink with them, and rows conditioned by 10 carry ten times
    # the error (at 264 x 384 the GPU's max |dO| is 2.04e-2, the same as a
    # CPU emulation of the kernels' rounding points).
    wl = W.moe_experts(experts=2, d_model=1024, d_ff=704, seed=7)
    gpu, _ = run_case(wl, "dimuon", cfg_of(wl))
    for i, m in enumerate(wl.mats):
        zero = (m.m_prev.float().abs().sum(1) == 0).sum().item()
        assert zero == round(0.1 * m.shape[0]), (i, zero)


# ---------------------------------------------------------------------------
# Method properties on the GPU
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("shapes", [[(8, 4096), (4096, 8), (4, 16)], [(300, 700), (700, 300), (256, 256)],
                                    [(384, 1024), (1024, 384), (300, 696), (700, 296)]])
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


@pytest.mark.parametrize("variant", ["muon", "dimuon"])
def test_degenerate_shapes(variant):
    # One-element and one-row matrices (thin path, Gram side 1) and the
    # smallest general-path Gram side (33), f32 and bf16 storage.
    shapes = [(1, 1), (1, 2), (2, 1), (1, 7), (33, 33), (33, 40), (40, 33)]
    for dt in ("f32", "bf16"):
        wl = W.random_batch(shapes, dtype=dt, ns_dtype="bf16", seed=29, variant=variant)
        run_case(wl, variant, cfg_of(wl))


def _batch_params(wl, idx):
    return [D.Param(w=wl.mats[i].w.cuda().clone(), g=wl.mats[i].g.cuda().clone(),
                    mom=wl.mats[i].m_prev.cuda().clone(),
                    o_out=torch.full(wl.mats[i].shape, float("nan"), device="cuda")) for i in idx]


@pytest.mark.parametrize("variant", ["muon", "dimuon"])
def test_matrices_independent_of_batch(variant):
    # A matrix's step does not depend on the other matrices of its batch:
    # each matrix stepped alone equals the same matrix in a mixed batch, bit
    # for bit (the batch changes tile lists and their order, not the
    # arithmetic of any matrix).
    shapes = [(8, 4096), (300, 700), (4096, 8), (700, 300), (256, 1024), (5, 333)]
    wl = W.random_batch(shapes, dtype="bf16", ns_dtype="bf16", seed=31, variant=variant)
    cfg = cfg_of(wl)
    fn = D.dimuon_step if variant == "dimuon" else D.muon_step
    announce(f"batch independence {variant}")
    together = _batch_params(wl, range(wl.count))
    fn(together, cfg)
    for i in range(wl.count):
        alone = _batch_params(wl, [i])
        fn(alone, cfg)
        torch.cuda.synchronize()
        for name in ("w", "mom", "o_out"):
            np.testing.assert_array_equal(getattr(alone[0], name).float().cpu().numpy(),
                                          getattr(together[i], name).float().cpu().numpy(),
                                          err_msg=f"matrix {i} {name}")


@pytest.mark.parametrize("variant", ["muon", "dimuon"])
def test_round_interleave_bit_identical(variant):
    # A batch of one shape whose one-per-CU tile lists fill whole rounds on
    # all XCDs (8 x 2048^2: 512 combine tiles, 256 symmetric ones after the
    # tail split) has its rounds dealt across the XCDs; a matrix stepped alone
    # keeps the plain order.  Tile order changes no arithmetic: bit for bit.
    shapes = [(2048, 2048)] * 8
    wl = W.random_batch(shapes, dtype="bf16", ns_dtype="bf16", seed=41, variant=variant)
    cfg = cfg_of(wl)
    fn = D.dimuon_step if variant == "dimuon" else D.muon_step
    announce(f"round interleave {variant}")
    together = _batch_params(wl, range(wl.count))
    fn(together, cfg)
    for i in (0, 5):
        alone = _batch_params(wl, [i])
        fn(alone, cfg)
        torch.cuda.synchronize()
        for name in ("w", "mom", "o_out"):
            np.testing.assert_array_equal(getattr(alone[0], name).float().cpu().numpy(),
                                          getattr(together[i], name).float().cpu().numpy(),
                                          err_msg=f"matrix {i} {name}")


@pytest.mark.parametrize("variant", ["muon", "dimuon"])
def test_repeated_steps_bit_identical(variant):
    # The same step on the same inputs gives the same bits every time.  The
    # 8 x 1024^2 batch runs its combine on 512 tiles of 128 x 128 (the planner
    # prefers them to 128 tiles of 256 x 256): with two such workgroups per
    # CU this once differed between runs in about a thousand elements of X'.
    shapes = [(1024, 1024)] * 8
    wl = W.random_batch(shapes, dtype="bf16", ns_dtype="bf16", seed=47, variant=variant)
    cfg = cfg_of(wl)
    fn = D.dimuon_step if variant == "dimuon" else D.muon_step
    announce(f"repeated steps {variant}")
    runs = []
    for _ in range(3):
        ps = _batch_params(wl, range(wl.count))
        fn(ps, cfg)
        torch.cuda.synchronize()
        runs.append([(p.w.float().cpu().numpy(), p.mom.float().cpu().numpy(), p.o_out.cpu().numpy()) for p in ps])
    for r in runs[1:]:
        for i in range(wl.count):
            for k, name in enumerate(("w", "mom", "o_out")):
                np.testing.assert_array_equal(r[i][k], runs[0][i][k], err_msg=f"matrix {i} {name}")


@pytest.mark.parametrize("variant", ["muon", "dimuon"])
def test_two_plans_on_two_streams_match_one_plan(variant):
    # A batch split into two plans stepped on two streams (their kernels may
    # then share CUs) gives what one plan over the whole batch gives, bit for
    # bit.  8 x 1024^2 runs 128 x 128 combine tiles, GPT-2 shapes 256 x 256.
    for wl in (W.random_batch([(1024, 1024)] * 8, dtype="bf16", ns_dtype="bf16", seed=49, variant=variant),
               W.gpt2_hidden(layers=4, seed=1, device="cuda")):
        cfg = cfg_of(wl)
        dimuon = variant == "dimuon"
        announce(f"two plans on two streams {variant} {wl.name}")
        one = _batch_params(wl, range(wl.count))
        plan = D.Plan(one, cfg, dimuon)
        plan.step()
        torch.cuda.synchronize()
        plan.close()
        two = _batch_params(wl, range(wl.count))
        p0, p1 = D.Plan(two[0::2], cfg, dimuon), D.Plan(two[1::2], cfg, dimuon)
        main, side = torch.cuda.current_stream(), torch.cuda.Stream()
        fork = torch.cuda.Event()
        fork.record(main)
        side.wait_event(fork)
        p0.step(main)
        p1.step(side)
        join = torch.cuda.Event()
        join.record(side)
        main.wait_event(join)
        torch.cuda.synchronize()
        p0.close()
        p1.close()
        for i, (a, b) in enumerate(zip(one, two)):
            for name in ("w", "mom", "o_out"):
                assert torch.equal(getattr(a, name), getattr(b, name)), f"{wl.name} matrix {i} {name}"


@pytest.mark.parametrize("variant", ["muon", "dimuon"])
def test_symmetric_ring_depths_bit_identical(variant):
    # 8 x 1024^2: the symmetric products run 128 x 128 tiles, 36 per matrix.
    # The batch's 288 tiles exceed one per CU and take the two-buffer ring; a
    # matrix alone (36 tiles) takes the four-buffer ring.  The two rings run
    # the same MFMAs in the same k order: bit for bit.
    shapes = [(1024, 1024)] * 8
    wl = W.random_batch(shapes, dtype="bf16", ns_dtype="bf16", seed=43, variant=variant)
    cfg = cfg_of(wl)
    fn = D.dimuon_step if variant == "dimuon" else D.muon_step
    announce(f"ring depths {variant}")
    together = _batch_params(wl, range(wl.count))
    fn(together, cfg)
    for i in (0, 5):
        alone = _batch_params(wl, [i])
        fn(alone, cfg)
        torch.cuda.synchronize()
        for name in ("w", "mom", "o_out"):
            np.testing.assert_array_equal(getattr(alone[0], name).float().cpu().numpy(),
                                          getattr(together[i], name).float().cpu().numpy(),
                                          err_msg=f"matrix {i} {name}")


@pytest.mark.parametrize("variant", ["muon", "dimuon"])
def test_nonfinite_gradient_stays_in_its_matrix(variant):
    # NaN propagates as IEEE arithmetic does (no status word): a NaN in one
    # element of a gradient gives a NaN in that element of M_t and a
    # non-finite step for that matrix (its norm is NaN), and leaves every
    # other matrix of the batch bit-identical to a batch without it.
    shapes = [(8, 1024), (300, 700), (1024, 8), (256, 256)]
    wl = W.random_batch(shapes, dtype="bf16", ns_dtype="bf16", seed=37, variant=variant)
    cfg = cfg_of(wl)
    fn = D.dimuon_step if variant == "dimuon" else D.muon_step
    for bad in (0, 1):
        announce(f"NaN in gradient of matrix {bad} ({variant})")
        clean = _batch_params(wl, range(wl.count))
        dirty = _batch_params(wl, range(wl.count))
        dirty[bad].g[3, 5] = float("nan")
        fn(clean, cfg)
        fn(dirty, cfg)
        torch.cuda.synchronize()
        m = dirty[bad].mom.float().cpu().numpy()
        assert np.isnan(m[3, 5]) and np.isfinite(np.delete(m.ravel(), 3 * m.shape[1] + 5)).all()
        assert not np.isfinite(dirty[bad].o_out.cpu().numpy()).any()
        for i in range(wl.count):
            if i == bad:
                continue
            for name in ("w", "mom", "o_out"):
                np.testing.assert_array_equal(getattr(clean[i], name).float().cpu().numpy(),
                                              getattr(dirty[i], name).float().cpu().numpy(),
                                              err_msg=f"matrix {i} {name}")


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


@pytest.mark.parametrize("variant", ["muon", "dimuon"])
def test_plan_graph_replays_match_eager(variant):
    # A plan replaying its launch sequence as a HIP graph equals a plan
    # launching eagerly, bit for bit, step after step: graphs captured in
    # both energy-cache states (Dimuon), eager device work and host
    # synchronisations between the replays, and a learning-rate change
    # (which discards the graphs).
    shapes = [(8, 4096), (4096, 8), (300, 700), (700, 300), (16, 2048)]
    wl = W.random_batch(shapes, dtype="bf16", ns_dtype="bf16", seed=23, variant=variant)
    cfg = cfg_of(wl)
    def fresh():
        return [D.Param(w=m.w.cuda().clone(), g=m.g.cuda().clone(), mom=m.m_prev.cuda().clone(),
                        o_out=torch.empty(m.shape, device="cuda")) for m in wl.mats]
    a, b = fresh(), fresh()
    pa, pb = D.Plan(a, cfg, dimuon=(variant == "dimuon")), D.Plan(b, cfg, dimuon=(variant == "dimuon"))
    pb.set_graph(True)
    junk = torch.ones(1 << 20, device="cuda")
    for step in range(6):
        if step == 4:
            pa.set_lr(0.01)
            pb.set_lr(0.01)
        announce(f"graph replay {variant} step {step}")
        pa.step()
        pb.step()
        junk.mul_(1.0001)          # the program's own eager work between replays
        torch.cuda.synchronize()
        for i, (x, y) in enumerate(zip(a, b)):
            for name in ("w", "mom", "o_out"):
                np.testing.assert_array_equal(getattr(x, name).float().cpu().numpy(),
                                              getattr(y, name).float().cpu().numpy(),
                                              err_msg=f"step {step} matrix {i} {name}")
    pa.close()
    pb.close()


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
