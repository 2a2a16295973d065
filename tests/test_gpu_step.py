"""End-to-end parity of qi21_prefill + qi21_step against the CPU oracle (needs a GPU).

The tiny model (2 blocks, dim 256, f32 weights that the library rounds to
f16 planes) runs through the C ABI on seeded inputs; its velocity must be
within 1e-3 relative L2 of the oracle's prefill + step on the same inputs.
Also: a condition-image prefix (block-causal mask over several key tiles),
a CFG pair of unequal prefixes as one batched step, determinism, the
range-guard settings, the non-finite refusal, and the error paths.
"""
import dataclasses

import numpy as np
import pytest

import bench
from inputs import CONFIGS
from inputs.configs import TINY_MODEL, Workload
from oracle import SynthModel, workload_inputs
from oracle import qi21_oracle as O
from parity import ROW_FACTOR, assert_close, rel, rowrel

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu
V_TOL = 1e-3


def Q():
    from diffusion_transformer_denoiser_qi21_amd import qi21
    return qi21


def rel_rows(a, b):
    """The whole tensor's relative L2 and the largest one row's own"""
    return rel(a, b), rowrel(a, b)


@pytest.fixture(scope="module")
def tiny_gpu():
    m = bench.build_model(TINY_MODEL)
    yield m
    Q().qi21_model_destroy(m)


@pytest.fixture(scope="module")
def tiny_cpu():
    return SynthModel(TINY_MODEL)


def oracle_v(model, w, prefix=0):
    d = workload_inputs(w, prefix)
    lay = O.Layout(w.layout(prefix))
    pre = O.prefill(model, d["x_prefix"], lay)
    return O.step(model, pre, d["tok"], d["mods"], d["final_scale"])


def gpu_v(m, w, key=1, prefix=0):
    d = bench.workload_tensors(w, prefix)
    bench.prefill(m, key, d)
    out = torch.full((d["n"], 64), 7.0, device="cuda")
    Q().qi21_step(m, key, d["tok"], d["mods"], d["fs"], out)
    return out.cpu().numpy(), d


def test_tiny_prefill_step_parity(tiny_gpu, tiny_cpu):
    w = CONFIGS["tiny"]
    v, _ = gpu_v(tiny_gpu, w)
    want = oracle_v(tiny_cpu, w)
    err, row = rel_rows(v, want)
    print(f"tiny v rel L2 {err:.3e}")
    assert err < V_TOL and row < ROW_FACTOR * V_TOL


@pytest.mark.parametrize("segs,target", [
    ((("text", 22), ("image", 12, 12)), (16, 16)),
    ((("text", 5), ("image", 3, 4), ("text", 2), ("image", 9, 9)), (7, 9)),
    ((("text", 1),), (1, 1)),
])
def test_condition_prefix_parity(tiny_gpu, tiny_cpu, segs, target):
    w = Workload("t", TINY_MODEL, 33, target, (tuple(segs),))
    v, _ = gpu_v(tiny_gpu, w, key=2)
    want = oracle_v(tiny_cpu, w)
    err, row = rel_rows(v, want)
    print(f"{segs} -> {target}: v rel L2 {err:.3e}")
    assert err < V_TOL and row < ROW_FACTOR * V_TOL


def test_cfg_pair_unequal_prefixes_batched(tiny_gpu, tiny_cpu):
    w = Workload("cfg", TINY_MODEL, 44, (10, 12), ((("text", 18),), (("text", 9), ("image", 2, 3))),
                 prefix_seeds=(44, 45))
    q = Q()
    ds = [bench.workload_tensors(w, p) for p in range(2)]
    for p in range(2):
        bench.prefill(tiny_gpu, 10 + p, ds[p])
    outs = [torch.zeros(d["n"], 64, device="cuda") for d in ds]
    q.qi21_step_batch(tiny_gpu, [10, 11], [d["tok"] for d in ds], ds[0]["mods"], ds[0]["fs"], outs)
    for p in range(2):
        # the oracle's prefix p, with the step inputs of the shared workload
        d = workload_inputs(w, p)
        lay = O.Layout(w.layout(p))
        pre = O.prefill(tiny_cpu, d["x_prefix"], lay)
        want = O.step(tiny_cpu, pre, d["tok"], d["mods"], d["final_scale"])
        err, row = rel_rows(outs[p].cpu().numpy(), want)
        print(f"cfg prefix {p}: v rel L2 {err:.3e}")
        assert err < V_TOL and row < ROW_FACTOR * V_TOL
    # batched == one program at a time
    single = torch.zeros_like(outs[1])
    q.qi21_step(tiny_gpu, 11, ds[1]["tok"], ds[1]["mods"], ds[1]["fs"], single)
    assert_close(single.cpu().numpy(), outs[1].cpu().numpy(), 1e-6, row_tol=2e-5)  # summation order, as below


@pytest.fixture(scope="module")
def wide_gpu():
    """One block at the full width (32 heads of 128), so the attention grids
    reach the sizes at which the launch forms change."""
    from inputs.configs import FULL_MODEL
    m = bench.build_model(dataclasses.replace(FULL_MODEL, layers=1))
    yield m
    Q().qi21_model_destroy(m)


@pytest.fixture(scope="module")
def wide_cpu():
    from inputs.configs import FULL_MODEL
    return SynthModel(dataclasses.replace(FULL_MODEL, layers=1))


# Target rows per program -> the attention form of the two programs' shared
# launch on 256 CUs: 512 -> key-split blocks, 1024 -> 4-wave blocks, 2048 ->
# 8-wave blocks (while each program alone would take the key-split, key-split
# and 4-wave forms).
@pytest.mark.parametrize("target", [(16, 32), (32, 32), (32, 64)])
def test_cfg_pair_shared_attention_launch(wide_gpu, wide_cpu, target):
    """The two programs' rows in one attention launch, against the oracle's
    step of each program (unequal prefixes, so the second segment's key
    count differs from the first's)."""
    from inputs.configs import FULL_MODEL
    w = Workload("cfgw", dataclasses.replace(FULL_MODEL, layers=1), 51, target,
                 ((("text", 18),), (("text", 7), ("image", 2, 2))), prefix_seeds=(51, 52))
    q = Q()
    ds = [bench.workload_tensors(w, p) for p in range(2)]
    for p in range(2):
        bench.prefill(wide_gpu, 20 + p, ds[p])
    outs = [torch.zeros(d["n"], 64, device="cuda") for d in ds]
    q.qi21_step_batch(wide_gpu, [20, 21], [d["tok"] for d in ds], ds[0]["mods"], ds[0]["fs"], outs)
    for p in range(2):
        got = outs[p].cpu().numpy()
        assert np.isfinite(got).all()
        err, row = rel_rows(got, oracle_v(wide_cpu, w, p))
        single = torch.zeros_like(outs[p])
        q.qi21_step(wide_gpu, 20 + p, ds[p]["tok"], ds[p]["mods"], ds[p]["fs"], single)
        print(f"{target} program {p}: v rel L2 {err:.3e} (alone vs batched "
              f"{rel(single.cpu().numpy(), got):.3e})")
        assert err < V_TOL and row < ROW_FACTOR * V_TOL


# The seeded rows are Irwin-Hall(4) draws, cut at 3.46 sigma; trained
# activations have heavier tails.  Plant far larger values (a whole prefix
# row at 40x, single entries at 25-60 sigma in the prefix and the latent
# tokens) and check that the f16 sites' range guards still carry them: v
# stays finite and within the bar of the oracle on the same inputs.
OUTLIERS = (("x_prefix", (3, slice(None)), 40.0, "scale"), ("x_prefix", (7, 5), 25.0, "set"),
            ("x_prefix", (0, 200), -60.0, "set"), ("tok", (11, 3), 30.0, "set"), ("tok", (200, slice(None)), 12.0,
                                                                                   "scale"))


def _plant(host, dev):
    for name, idx, val, how in OUTLIERS:
        key = "x" if name == "x_prefix" else name
        if idx[0] >= host[name].shape[0]:
            continue
        if how == "scale":
            host[name][idx] *= val
            dev[key][idx] *= val
        else:
            host[name][idx] = val
            dev[key][idx] = val


@pytest.mark.parametrize("which", ["tiny", "wide"])
def test_outliers_beyond_the_synthetic_tails(which, tiny_gpu, tiny_cpu, wide_gpu, wide_cpu):
    from inputs.configs import FULL_MODEL
    spec = TINY_MODEL if which == "tiny" else dataclasses.replace(FULL_MODEL, layers=1)
    m, cpu = (tiny_gpu, tiny_cpu) if which == "tiny" else (wide_gpu, wide_cpu)
    w = Workload("tails", spec, 77, (16, 16), ((("text", 18),),))
    d = bench.workload_tensors(w)
    dd = workload_inputs(w)
    _plant(dd, d)
    assert float(np.abs(dd["x_prefix"]).max()) >= 60.0 and float(np.abs(dd["tok"]).max()) >= 30.0
    bench.prefill(m, 31, d)
    out = torch.full((d["n"], 64), 7.0, device="cuda")
    Q().qi21_step(m, 31, d["tok"], d["mods"], d["fs"], out)
    v = out.cpu().numpy()
    pre = O.prefill(cpu, dd["x_prefix"], O.Layout(w.layout()))
    want = O.step(cpu, pre, dd["tok"], dd["mods"], dd["final_scale"])
    err, row = rel_rows(v, want)
    print(f"{which} with planted outliers: v rel L2 {err:.3e}, worst row {row:.3e}, |v| max {np.abs(v).max():.2f}")
    assert np.isfinite(v).all()
    assert err < V_TOL and row < ROW_FACTOR * V_TOL
    Q().qi21_release_key(m, 31)


def test_step_is_deterministic(tiny_gpu):
    w = CONFIGS["tiny"]
    d = bench.workload_tensors(w)
    bench.prefill(tiny_gpu, 3, d)
    a = torch.zeros(d["n"], 64, device="cuda")
    b = torch.zeros(d["n"], 64, device="cuda")
    Q().qi21_step(tiny_gpu, 3, d["tok"], d["mods"], d["fs"], a)
    Q().qi21_step(tiny_gpu, 3, d["tok"], d["mods"], d["fs"], b)
    assert torch.equal(a, b)


def test_profile_sampling_counts_and_leaves_v_alone(tiny_gpu):
    """Events around one launch in `every` of a profiled class: the launch
    counts follow, and v is bit-identical with and without the events."""
    q = Q()
    w = CONFIGS["tiny"]
    d = bench.workload_tensors(w)
    bench.prefill(tiny_gpu, 4, d)
    ref = torch.zeros(d["n"], 64, device="cuda")
    q.qi21_step(tiny_gpu, 4, d["tok"], d["mods"], d["fs"], ref)
    blocks = TINY_MODEL.layers
    with pytest.raises(RuntimeError):
        q.qi21_set_profile_every(tiny_gpu, 0)
    q.qi21_profile_read(tiny_gpu)
    q.qi21_set_profile(tiny_gpu, (1 << 4) | (1 << 5))
    for every, steps in ((1, 2), (3, 5)):
        q.qi21_set_profile_every(tiny_gpu, every)
        for _ in range(steps):
            out = torch.zeros(d["n"], 64, device="cuda")
            q.qi21_step(tiny_gpu, 4, d["tok"], d["mods"], d["fs"], out)
            assert torch.equal(out, ref)
        torch.cuda.synchronize()
        ms, n = q.qi21_profile_read(tiny_gpu)
        want = -(-steps * blocks // every)  # launches 0, every, 2 every, ... of steps * blocks
        assert n[4] == want and n[5] == want, (every, n)
        assert ms[4] > 0 and ms[5] > 0
    q.qi21_set_profile(tiny_gpu, 0)
    q.qi21_set_profile_every(tiny_gpu, 1)


@pytest.mark.parametrize("shifts", [(0, 0, 0, 0, 0), (4, 8, 2, 4, 10)])
def test_range_guard_settings(tiny_cpu, shifts):
    q = Q()
    opt = q.qi21_default_options()
    opt.shift_attn, opt.shift_qkv, opt.shift_ao, opt.shift_ffn, opt.shift_hid = shifts
    m = bench.build_model(TINY_MODEL, opt)
    try:
        w = CONFIGS["tiny"]
        v, _ = gpu_v(m, w)
        assert_close(v, oracle_v(tiny_cpu, w), V_TOL)
    finally:
        q.qi21_model_destroy(m)


@pytest.mark.parametrize("mode", ["pair", "lo8", "lo4"])
def test_ffn_mode_option(tiny_cpu, tiny_gpu, mode):
    """ffn_mode PAIR (FFN input and hidden as f16 pairs), LO8 and LO4 (f16
    plus a scaled fp8 / fp4 residual): the result to the bar, on the single
    step and on a batched CFG pair, and no larger error than single f16"""
    q = Q()
    opt = q.qi21_default_options()
    opt.ffn_mode = {"pair": q.QI21_FFN_PAIR, "lo8": q.QI21_FFN_LO8, "lo4": q.QI21_FFN_LO4}[mode]
    m = bench.build_model(TINY_MODEL, opt)
    try:
        w = CONFIGS["tiny"]
        v, _ = gpu_v(m, w)
        want = oracle_v(tiny_cpu, w)
        err, row = rel_rows(v, want)
        base = rel(gpu_v(tiny_gpu, w, key=5)[0], want)
        print(f"tiny v rel L2 ffn_mode {mode} {err:.3e}, single f16 {base:.3e}")
        assert err < V_TOL and row < ROW_FACTOR * V_TOL and err < base
        ds = [bench.workload_tensors(w) for _ in range(2)]
        bench.prefill(m, 2, ds[0])
        outs = [torch.zeros(ds[0]["n"], 64, device="cuda") for _ in range(2)]
        q.qi21_step_batch(m, [1, 2], [d["tok"] for d in ds], ds[0]["mods"], ds[0]["fs"], outs)
        # batched and single passes sum in different orders; where that moves
        # an f32 value across an f16 rounding boundary at a storage site, one
        # element of a row moves by 2^-11 of itself, so a row's figure may
        # reach several times the whole tensor's
        for o in outs:
            assert_close(o.cpu().numpy(), v, 1e-6, row_tol=2e-5)
    finally:
        q.qi21_model_destroy(m)


def test_nonfinite_velocity_is_refused_and_out_untouched(tiny_gpu):
    q = Q()
    w = CONFIGS["tiny"]
    d = bench.workload_tensors(w)
    bench.prefill(tiny_gpu, 4, d)
    mods = d["mods"].clone()
    mods[:TINY_MODEL.dim] = 1e5  # (1 + s1) * LN(x) overflows the f16 attention input
    out = torch.full((d["n"], 64), 7.0, device="cuda")
    with pytest.raises(q.Qi21Error) as e:
        q.qi21_step(tiny_gpu, 4, d["tok"], mods, d["fs"], out)
    assert e.value.code == q.QI21_ENONFINITE
    assert torch.all(out == 7.0)
    # the model still works afterwards
    q.qi21_step(tiny_gpu, 4, d["tok"], d["mods"], d["fs"], out)
    assert torch.all(torch.isfinite(out))


def test_batched_step_after_a_refused_nonfinite_step(tiny_gpu, tiny_cpu):
    """A refused non-finite step leaves non-finite values behind in the
    shared activations.  A later batched step whose programs leave gap rows
    between them (target 120 rows: the second program starts at row 128)
    and V^T padding past the last key (248 rows in a 256-row pass) reads
    both with zero weight, so they must have been rewritten: the step is
    finite and matches the oracle ([WG] step refuses a non-finite velocity
    and the program stays usable)."""
    q = Q()
    w0 = CONFIGS["tiny"]
    d0 = bench.workload_tensors(w0)
    bench.prefill(tiny_gpu, 20, d0)
    mods = d0["mods"].clone()
    mods[:TINY_MODEL.dim] = 1e5  # (1 + s1) * LN(x) overflows the f16 attention input
    out = torch.zeros(d0["n"], 64, device="cuda")
    with pytest.raises(q.Qi21Error) as e:
        q.qi21_step(tiny_gpu, 20, d0["tok"], mods, d0["fs"], out)
    assert e.value.code == q.QI21_ENONFINITE
    q.qi21_release_key(tiny_gpu, 20)
    w = Workload("cfg", TINY_MODEL, 44, (10, 12), ((("text", 18),), (("text", 9), ("image", 2, 3))),
                 prefix_seeds=(44, 45))
    ds = [bench.workload_tensors(w, p) for p in range(2)]
    for p in range(2):
        bench.prefill(tiny_gpu, 21 + p, ds[p])
    outs = [torch.zeros(d["n"], 64, device="cuda") for d in ds]
    q.qi21_step_batch(tiny_gpu, [21, 22], [d["tok"] for d in ds], ds[0]["mods"], ds[0]["fs"], outs)
    for p in range(2):
        d = workload_inputs(w, p)
        pre = O.prefill(tiny_cpu, d["x_prefix"], O.Layout(w.layout(p)))
        want = O.step(tiny_cpu, pre, d["tok"], d["mods"], d["final_scale"])
        got = outs[p].cpu().numpy()
        assert np.isfinite(got).all()
        assert_close(got, want, V_TOL)
    for p in range(2):
        q.qi21_release_key(tiny_gpu, 21 + p)


def test_torch_pool_and_enomem_leave_the_model_usable(tiny_cpu):
    # every device byte comes from torch's caching allocator through the
    # alloc/free hook; a refused allocation in prefill gives ENOMEM with the
    # accounting intact, and the same model then steps to the oracle's v
    q = Q()
    pool = q.DeviceAllocator()
    m = bench.build_model(TINY_MODEL, pool.install(q.qi21_default_options()))
    try:
        b0 = q.qi21_model_bytes(m)
        assert b0 > 0 and pool.live_bytes == b0
        w = CONFIGS["tiny"]
        d = bench.workload_tensors(w)
        pool.budget = b0  # nothing more fits: the activations are refused
        with pytest.raises(q.Qi21Error) as e:
            bench.prefill(m, 1, d)
        assert e.value.code == q.QI21_ENOMEM and pool.failed >= 1
        assert q.qi21_model_bytes(m) == pool.live_bytes == b0
        out = torch.zeros(d["n"], 64, device="cuda")
        with pytest.raises(q.Qi21Error) as e:
            q.qi21_step(m, 1, d["tok"], d["mods"], d["fs"], out)
        assert e.value.code == q.QI21_ENOKEY  # the refused program was not kept
        pool.budget = None
        bench.prefill(m, 1, d)
        q.qi21_step(m, 1, d["tok"], d["mods"], d["fs"], out)
        v1 = out.cpu().numpy()
        err, row = rel_rows(v1, oracle_v(tiny_cpu, w))
        print(f"torch pool: v rel L2 {err:.3e}")
        assert err < V_TOL and row < ROW_FACTOR * V_TOL
        # a larger second program needs more activation rows than exist
        big = Workload("big", TINY_MODEL, 9, (24, 24), ((("text", 40),),))
        db = bench.workload_tensors(big)
        pool.budget = pool.live_bytes
        with pytest.raises(q.Qi21Error) as e:
            bench.prefill(m, 2, db)
        assert e.value.code == q.QI21_ENOMEM
        assert q.qi21_model_bytes(m) == pool.live_bytes
        pool.budget = None
        out2 = torch.zeros_like(out)
        q.qi21_step(m, 1, d["tok"], d["mods"], d["fs"], out2)  # program 1 survived
        assert np.array_equal(out2.cpu().numpy(), v1)
    finally:
        q.qi21_model_destroy(m)
    assert pool.live == {}


def test_error_paths_and_eviction(tiny_gpu):
    q = Q()
    w = CONFIGS["tiny"]
    d = bench.workload_tensors(w)
    out = torch.zeros(d["n"], 64, device="cuda")
    with pytest.raises(q.Qi21Error) as e:
        q.qi21_step(tiny_gpu, 999, d["tok"], d["mods"], d["fs"], out)
    assert e.value.code == q.QI21_ENOKEY
    for bad in (d["vis"].flip(0), torch.zeros_like(d["vis"]), d["vis"] + 1):
        dd = dict(d, vis=bad.contiguous())
        with pytest.raises(q.Qi21Error) as e:
            bench.prefill(tiny_gpu, 5, dd)
        assert e.value.code == q.QI21_EINVAL
    # max_programs = 2: a third prefix evicts the oldest
    for k in (21, 22, 23):
        bench.prefill(tiny_gpu, k, d)
    with pytest.raises(q.Qi21Error) as e:
        q.qi21_step(tiny_gpu, 21, d["tok"], d["mods"], d["fs"], out)
    assert e.value.code == q.QI21_ENOKEY
    q.qi21_step(tiny_gpu, 23, d["tok"], d["mods"], d["fs"], out)
    q.qi21_release_key(tiny_gpu, 23)
    with pytest.raises(q.Qi21Error) as e:
        q.qi21_release_key(tiny_gpu, 23)
    assert e.value.code == q.QI21_ENOKEY
    # a model whose blocks were never set refuses to prefill
    spec = dataclasses.replace(TINY_MODEL, layers=1)
    m2 = q.qi21_model_create(bench.geom_of(spec), None, 1, torch.zeros(256, 64, device="cuda"),
                             torch.zeros(64, 256, device="cuda"))
    try:
        with pytest.raises(q.Qi21Error) as e:
            bench.prefill(m2, 1, d)
        assert e.value.code == q.QI21_EINVAL
    finally:
        q.qi21_model_destroy(m2)


# ───────────────────────────── time path and sampler ─────────────────────────────

@pytest.fixture(scope="module")
def tiny_time():
    m = bench.build_model(TINY_MODEL, time_path=True)
    yield m
    Q().qi21_model_destroy(m)


@pytest.mark.parametrize("t", [0.0, 0.37, 1.0])
def test_time_mods_match_oracle(tiny_time, tiny_cpu, t):
    q = Q()
    h = TINY_MODEL.dim
    mods = torch.zeros(4 * h, device="cuda")
    fs = torch.zeros(h, device="cuda")
    q.qi21_time_mods(tiny_time, t, mods, fs)
    torch.cuda.synchronize()
    want_m, want_f = O.time_mods(tiny_cpu.time(), t)
    assert_close(mods.cpu().numpy(), want_m, 1e-5)
    assert_close(fs.cpu().numpy(), 1.0 + want_f, 1e-6)


def test_step_t_against_oracle(tiny_time, tiny_cpu):
    w = CONFIGS["tiny"]
    d = bench.workload_tensors(w)
    bench.prefill(tiny_time, 7, d)
    out = torch.zeros(d["n"], 64, device="cuda")
    Q().qi21_step_t(tiny_time, 7, d["tok"], 0.55, out)
    dd = workload_inputs(w)
    pre = O.prefill(tiny_cpu, dd["x_prefix"], O.Layout(w.layout()))
    mods, fsc = O.time_mods(tiny_cpu.time(), 0.55)
    err, row = rel_rows(out.cpu().numpy(), O.step(tiny_cpu, pre, dd["tok"], mods, fsc))
    print(f"step_t v rel L2 {err:.3e}")
    assert err < V_TOL and row < ROW_FACTOR * V_TOL


def test_sampler_against_oracle(tiny_time, tiny_cpu):
    w = CONFIGS["tiny"]
    d = bench.workload_tensors(w)
    bench.prefill(tiny_time, 8, d)
    times = [1.0, 0.75, 0.5, 0.25]
    x = d["tok"].clone()
    Q().qi21_sample(tiny_time, 8, x, times)
    dd = workload_inputs(w)
    pre = O.prefill(tiny_cpu, dd["x_prefix"], O.Layout(w.layout()))
    want = O.sample(tiny_cpu, pre, dd["tok"], times)
    err, row = rel_rows(x.cpu().numpy(), want)
    print(f"3-step sample rel L2 {err:.3e}")
    assert err < V_TOL and row < ROW_FACTOR * V_TOL
    # no time elapses, x unchanged; zero steps are a no-op
    y = d["tok"].clone()
    Q().qi21_sample(tiny_time, 8, y, [0.4, 0.4])
    Q().qi21_sample(tiny_time, 8, y, [0.4])
    assert torch.equal(y, d["tok"])


def test_time_path_errors(tiny_gpu, tiny_time):
    q = Q()
    x = torch.zeros(256, 64, device="cuda")
    bench.prefill(tiny_gpu, 9, bench.workload_tensors(CONFIGS["tiny"]))
    with pytest.raises(q.Qi21Error) as e:  # no time weights in this model
        q.qi21_sample(tiny_gpu, 9, x, [1.0, 0.5])
    assert e.value.code == q.QI21_EINVAL
    with pytest.raises(q.Qi21Error) as e:
        q.qi21_sample(tiny_time, 12345, x, [1.0, 0.5])
    assert e.value.code == q.QI21_ENOKEY
    with pytest.raises(q.Qi21Error):
        q.qi21_time_mods(tiny_time, float("nan"), x, x)


# ───────────────────────────── txt_in front ─────────────────────────────

@pytest.fixture(scope="module")
def tiny_txt():
    m = bench.build_model(TINY_MODEL, txt_in=True)
    yield m
    Q().qi21_model_destroy(m)


def _feats(n, c, seed=5):
    import inputs
    from inputs.configs import TID_TXT_FEATS
    return inputs.host_array(seed, TID_TXT_FEATS, (n, c), 1.0)


@pytest.mark.parametrize("n", [1, 18, 22, 300])
def test_txt_in_matches_oracle(tiny_txt, tiny_cpu, n):
    h = TINY_MODEL.dim
    f = _feats(n, h)
    out = torch.full((n, h), 7.0, device="cuda")
    Q().qi21_txt_in(tiny_txt, n, torch.from_numpy(f).cuda(), out)
    torch.cuda.synchronize()
    t = tiny_cpu.txt()
    want = O.embed_text(f, t["txt_norm"], t["txt_in1"], t["txt_in2"], TINY_MODEL.eps)
    err, row = rel_rows(out.cpu().numpy(), want)
    print(f"txt_in n {n}: rel L2 {err:.3e}")
    assert err < 2e-3 and row < ROW_FACTOR * 2e-3  # the normalised features and the GELU output are f16


def test_txt_in_feeds_prefill(tiny_txt, tiny_cpu):
    # a text-only prefix whose rows come from txt_in, then a step
    w = CONFIGS["tiny"]
    d = bench.workload_tensors(w)
    f = _feats(d["lp"], TINY_MODEL.dim, seed=6)
    Q().qi21_txt_in(tiny_txt, d["lp"], torch.from_numpy(f).cuda(), d["x"])
    bench.prefill(tiny_txt, 4, d)
    out = torch.zeros(d["n"], 64, device="cuda")
    Q().qi21_step(tiny_txt, 4, d["tok"], d["mods"], d["fs"], out)
    dd = workload_inputs(w)
    t = tiny_cpu.txt()
    xp = O.embed_text(f, t["txt_norm"], t["txt_in1"], t["txt_in2"], TINY_MODEL.eps)
    pre = O.prefill(tiny_cpu, xp, O.Layout(w.layout()))
    want = O.step(tiny_cpu, pre, dd["tok"], dd["mods"], dd["final_scale"])
    err, row = rel_rows(out.cpu().numpy(), want)
    print(f"txt_in prefix -> step: v rel L2 {err:.3e}")
    assert err < V_TOL and row < ROW_FACTOR * V_TOL


def test_txt_in_requires_weights(tiny_gpu):
    q = Q()
    z = torch.zeros(4, 256, device="cuda")
    with pytest.raises(q.Qi21Error) as e:
        q.qi21_txt_in(tiny_gpu, 4, z, z)
    assert e.value.code == q.QI21_EINVAL
