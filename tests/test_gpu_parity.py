"""GPU parity: the HIP path through the C ABI against the CPU oracle.

All twelve workload problems at full size, in the launch configuration the
benchmark times (automatic kernel choice), plus every problem on the
generic kernel family, integer-exact (bit-for-bit) runs, sentinel / guard /
determinism checks, a non-default stream, and seeded fuzz over layouts,
dtypes, groups, strides, dilations and padding for each kernel family.

The large bf16 case (dY 16x1x256x2048, W 2048x1x2x2048) is checked element
by element on sampled outputs the oracle computes one at a time and on
every output against one call of the oracle over the whole problem (about a
second on the host's threads, shared by the tests of its seeded operands).
"""
import random

import numpy as np
import pytest
import torch

import dnn_conv2d_bwd_amd as cbd
import oracle
from cbd_inputs import GROUPED_SWEEP, PROBLEMS, small_ints, uniform
from cbd_inputs.problems import NCHW, NHWC, Problem

from parity import DeviceRun, check, check_bf16, check_f32, exact_expected_bits, operands, \
    plan_for, to_device

pytestmark = pytest.mark.gpu

SMALL = [p.name for p in PROBLEMS if p.name != "c4"]


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    yield


def by_name(name):
    return [p for p in PROBLEMS if p.name == name][0]


_FULL_REF = {}


def oracle_full(p, kind="dist"):
    """The oracle's whole dX of a workload problem's seeded operands (one
    call each, kept for the tests that share it: about a second for the
    headline problem on the host's threads)."""
    key = (p.name, kind, p.n, p.hi, p.wi)
    if key not in _FULL_REF:
        dy, w = operands(p, kind)
        _FULL_REF[key] = oracle.bwd_data(p, dy, w)
    return _FULL_REF[key]


def unreached_mask(p):
    """Positions (h, w) of dX that no tap reaches (brute force)."""
    ho_n, wo_n = oracle.out_hw(p)

    def reach(i, pad, dil, taps, s, on):
        return any((i + pad - t * dil) >= 0 and (i + pad - t * dil) % s == 0
                   and (i + pad - t * dil) // s < on for t in range(taps))
    rh = np.array([reach(h, p.ph, p.dh, p.y, p.sh, ho_n) for h in range(p.hi)])
    rw = np.array([reach(w, p.pw, p.dw, p.x, p.sw, wo_n) for w in range(p.wi)])
    return ~(rh[:, None] & rw[None, :])


def spatial(p, a):
    """(N, C, H, W) view of a layout-ordered dX array."""
    return a if p.layout == NCHW else np.transpose(a, (0, 3, 1, 2))


# --------------------------------------------------------------- workload ---

@pytest.mark.parametrize("name", SMALL)
@pytest.mark.parametrize("force", [cbd.KERNEL_AUTO, cbd.KERNEL_GENERIC, cbd.KERNEL_NCHW_ROWS])
def test_workload_vs_oracle(name, force):
    p = by_name(name)
    if force == cbd.KERNEL_NCHW_ROWS and p.layout != NCHW:
        pytest.skip("the row-block family serves NCHW problems only")
    print(f"[parity] {name} force={force} kernel={plan_for(p, force).info().kernel}", flush=True)
    dy, w = operands(p)
    ref = oracle.bwd_data(p, dy, w)
    pl = plan_for(p, force)
    run = DeviceRun(p, pl, to_device(dy, p), to_device(w, p))()
    ok, info = check(p, run, ref)
    assert ok, info
    assert run.guards_intact()
    got = run.result_f32()
    assert not np.isnan(got).any()
    z = unreached_mask(p)
    if z.any():
        assert np.all(spatial(p, got)[:, :, z] == 0.0)
    if name == "c3b":
        assert np.count_nonzero(got == 0.0) >= got.size * 3 // 4
    bits1 = run.result_bits().copy()
    run()
    assert np.array_equal(bits1, run.result_bits()), "not deterministic"


# Generic family with 64x64 tiles (the planner takes them only for grids of
# at least 1024 such tiles): a 1x1 stride-1 and a 3x3 stride-2 fp32 problem,
# and a bf16 NHWC one forced onto the generic family.
GENERIC64 = [
    Problem("g64-1x1", 16, 1, 64, 64, 64, 64, 1, 1, 1, 1, 0, 0, 1, 1, NCHW, "f32", "u", "u", 0, 0),
    Problem("g64-3x3s2", 16, 1, 64, 64, 72, 72, 3, 3, 2, 2, 1, 1, 1, 1, NCHW, "f32", "u", "u", 0, 0),
    Problem("g64-nhwc", 16, 1, 64, 64, 64, 64, 1, 1, 1, 1, 0, 0, 1, 1, NHWC, "bf16", "n1", "n0.05", 0, 0),
]


@pytest.mark.parametrize("idx", range(len(GENERIC64)))
def test_generic_64_tiles_vs_oracle(idx):
    p = GENERIC64[idx]
    print(f"[parity] {p.name}", flush=True)
    dy, w = operands(p)
    pl = plan_for(p, cbd.KERNEL_GENERIC)
    assert (pl.info().tile_m, pl.info().tile_n) == (64, 64)
    run = DeviceRun(p, pl, to_device(dy, p), to_device(w, p))()
    ok, info = check(p, run, oracle.bwd_data(p, dy, w))
    assert ok, info
    assert run.guards_intact()


# ------------------------------------------------------------ maximum sizes ---
# dX just under 2^31 bytes, the library's limit for 32-bit buffer offsets,
# with three of four phases unreached (1x1 filter, stride 2): the GEMM kernels
# and both zero-fill paths (standalone NHWC 16-byte chunks, folded NCHW
# elements) run at the largest offsets the planner accepts.  Small-integer
# operands make every expected value exact; checked at the corners of the
# tensor, the last elements and random points, plus every unreached element
# exactly zero and no NaN sentinel left anywhere in dX.
MAXSIZE = [
    Problem("max-nhwc-bf16", 15, 1, 256, 256, 512, 512, 1, 1, 2, 2, 0, 0, 1, 1, NHWC, "bf16",
            "int", "int", 0, 0),
    Problem("max-nchw-f32", 8, 1, 64, 64, 1000, 1000, 1, 1, 2, 2, 0, 0, 1, 1, NCHW, "f32",
            "int", "int", 0, 0),
]


@pytest.mark.parametrize("idx", range(len(MAXSIZE)))
def test_max_size_integer_exact(idx):
    p = MAXSIZE[idx]
    print(f"[max-size] {p.name}", flush=True)
    pl = plan_for(p)
    sh = pl.shapes()
    es = 4 if p.dtype == "f32" else 2
    assert 2 ** 31 * 15 // 16 <= int(np.prod(sh["dx"])) * es < 2 ** 31
    assert pl.info().num_zero_regions == 3
    dy = small_ints(1, sh["dy"])
    w = small_ints(2, sh["w"])
    run = DeviceRun(p, pl, to_device(dy, p), to_device(w, p))()
    torch.cuda.synchronize()
    dx = run.dx
    assert not bool(torch.isnan(dx).any())
    assert run.guards_intact()
    odd = [dx[:, :, 1::2, :], dx[:, :, :, 1::2]] if p.layout == NCHW else \
          [dx[:, 1::2, :, :], dx[:, :, 1::2, :]]
    for v in odd:
        assert bool((v == 0).all())
    rng = np.random.default_rng(77)
    pts = [(n, c, h, x) for n in (0, p.n - 1) for c in (0, 1, p.c - 1)
           for h in (0, 1, p.hi - 2, p.hi - 1) for x in (0, 1, p.wi - 2, p.wi - 1)]
    pts += list(zip(rng.integers(0, p.n, 3000), rng.integers(0, p.c, 3000),
                    rng.integers(0, p.hi, 3000), rng.integers(0, p.wi, 3000)))
    pts = np.array(pts, dtype=np.int64)
    want = exact_expected_bits(p, oracle.bwd_data_at(p, dy, w, pts))
    i = torch.from_numpy(pts).cuda()
    got = dx[i[:, 0], i[:, 1], i[:, 2], i[:, 3]] if p.layout == NCHW else \
        dx[i[:, 0], i[:, 2], i[:, 3], i[:, 1]]
    got = got.cpu()
    got_bits = got.view(torch.int32).numpy().view(np.uint32) if p.dtype == "f32" else \
        got.view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(got_bits, want), int(np.count_nonzero(got_bits != want))


@pytest.mark.parametrize("name", [p.name for p in PROBLEMS])
def test_workload_integer_exact(name):
    p = by_name(name)
    print(f"[exact] {name}", flush=True)
    dy, w = operands(p, "int")
    pl = plan_for(p)
    run = DeviceRun(p, pl, to_device(dy, p), to_device(w, p))()
    got = run.result_f32()
    ref = oracle_full(p, "int")
    want = oracle.bf16_bits_to_f32(exact_expected_bits(p, ref)) if p.dtype == "bf16" \
        else exact_expected_bits(p, ref).view(np.float32)
    assert np.array_equal(got, want.reshape(got.shape))
    assert run.guards_intact()


def test_c4_full_size():
    """The headline bf16 problem: sampled oracle outputs (tile corners and
    random points, one at a time) and every output against one call of the
    oracle's fp64 loop nest over the whole problem."""
    p = by_name("c4")
    print("[parity] c4 full size", flush=True)
    dy, w = operands(p)
    pl = plan_for(p)
    assert pl.info().kernel == cbd.KERNEL_NHWC_BF16
    run = DeviceRun(p, pl, to_device(dy, p), to_device(w, p))()
    bits = run.result_bits().reshape(p.n, p.hi, p.wi, p.c)
    assert run.guards_intact()
    # sampled outputs, one by one, from the oracle: every tile corner plus random points
    rng = np.random.default_rng(44)
    pts = [(n, c, 0, wi) for n in (0, p.n - 1) for c in (0, 255, 256, p.c - 1)
           for wi in (0, 1, 510, 511)]
    pts += list(zip(rng.integers(0, p.n, 4000), rng.integers(0, p.c, 4000),
                    np.zeros(4000, dtype=np.int64), rng.integers(0, p.wi, 4000)))
    pts = np.array(pts, dtype=np.int64)
    ref_pts = oracle.bwd_data_at(p, dy, w, pts)
    got_pts = bits[pts[:, 0], pts[:, 2], pts[:, 3], pts[:, 1]]
    ok, info = check_bf16(got_pts, ref_pts)
    assert ok, info
    # every output against the oracle over the whole problem
    ref = oracle_full(p).reshape(bits.shape)
    ok, info = check_bf16(bits, ref)
    print("[parity] c4", info, flush=True)
    assert ok, info
    bits1 = bits.copy()
    run()
    assert np.array_equal(bits1, run.result_bits().reshape(bits1.shape))


@pytest.mark.parametrize("ksplit", [2, 3, 8])
def test_c4_ksplit(ksplit):
    """Split-K on the headline problem: every output against the oracle,
    and equal to itself on a second call."""
    p = by_name("c4")
    print(f"[ksplit] c4 ksplit={ksplit}", flush=True)
    dy, w = operands(p)
    pl = plan_for(p, ksplit=ksplit)
    assert pl.info().ksplit == ksplit
    ws = torch.empty(pl.workspace_size(), dtype=torch.uint8, device="cuda")
    run = DeviceRun(p, pl, to_device(dy, p), to_device(w, p), workspace=ws)()
    bits = run.result_bits().reshape(p.n, p.hi, p.wi, p.c)
    assert run.guards_intact()
    ok, info = check_bf16(bits, oracle_full(p).reshape(bits.shape))
    print("[ksplit] c4", info, flush=True)
    assert ok, info
    bits1 = bits.copy()
    run()
    assert np.array_equal(bits1, run.result_bits().reshape(bits1.shape))


@pytest.mark.parametrize("n,ksplit", [(2, 8), (1, 16), (4, 4)])
def test_c4_shard_ksplit_integer_exact(n, ksplit):
    """One GPU's batch shard of the headline problem with split-K, on
    integer-valued operands: bit-exact against the oracle."""
    p = by_name("c4").with_(n=n)
    print(f"[ksplit] c4 n={n} ksplit={ksplit}", flush=True)
    dy, w = operands(p, "int")
    pl = plan_for(p, ksplit=ksplit)
    ws = torch.empty(pl.workspace_size(), dtype=torch.uint8, device="cuda")
    run = DeviceRun(p, pl, to_device(dy, p), to_device(w, p), workspace=ws)()
    want = oracle.bf16_bits_to_f32(exact_expected_bits(p, oracle.bwd_data(p, dy, w)))
    got = run.result_f32()
    assert np.array_equal(got, want.reshape(got.shape))
    assert run.guards_intact()


@pytest.mark.parametrize("seed,count", [(19, 40)])
def test_fuzz_ksplit_integer_exact(seed, count):
    rng = random.Random(seed + 7)
    for i, p in enumerate(fuzz_problems(seed, count, family=cbd.KERNEL_NHWC_BF16)):
        ksplit = rng.choice([2, 3, 5, 16])
        pl = plan_for(p, cbd.KERNEL_NHWC_BF16, ksplit=ksplit)
        print(f"[fuzz-ksplit] i={i} ksplit={ksplit}->{pl.info().ksplit} {p}", flush=True)
        sh = oracle.shapes(p)
        dy = small_ints(5000 * seed + 3 * i + 1, sh["dy"]).astype(np.float32)
        w = small_ints(5000 * seed + 3 * i + 2, sh["w"]).astype(np.float32)
        ws = torch.empty(max(pl.workspace_size(), 1), dtype=torch.uint8, device="cuda")
        run = DeviceRun(p, pl, to_device(dy, p), to_device(w, p), workspace=ws)()
        want = oracle.bf16_bits_to_f32(exact_expected_bits(p, oracle.bwd_data(p, dy, w)))
        got = run.result_f32()
        assert np.array_equal(got, want.reshape(got.shape)), (p, ksplit)
        assert run.guards_intact(), (p, ksplit)


# Split-K on the generic family: (problem, requested splits; clamped to the
# k tiles of the shortest class: c1 18, c2-14-3 36, c3a 8, c3b 8).
GENERIC_SPLIT = [("c1", 4), ("c1", 64), ("c2-14-3", 2), ("c3a", 3), ("c3b", 2), ("c3b", 8)]


@pytest.mark.parametrize("name,ksplit", GENERIC_SPLIT)
def test_generic_ksplit_vs_oracle(name, ksplit):
    """Generic family with split-K: random operands within the fp32
    tolerance, integer operands bit-exact, the same bits on a second call,
    guard bands intact."""
    p = by_name(name)
    pl = plan_for(p, cbd.KERNEL_GENERIC, ksplit=ksplit)
    info = pl.info()
    print(f"[ksplit-generic] {name} ksplit={ksplit}->{info.ksplit}", flush=True)
    assert info.kernel == cbd.KERNEL_GENERIC and 2 <= info.ksplit <= ksplit
    assert pl.workspace_size() == info.workspace_bytes > 0
    ws = torch.empty(pl.workspace_size(), dtype=torch.uint8, device="cuda")
    for kind in ("dist", "int"):
        dy, w = operands(p, kind)
        ref = oracle.bwd_data(p, dy, w)
        run = DeviceRun(p, pl, to_device(dy, p), to_device(w, p), workspace=ws)()
        if kind == "dist":
            ok, inf = check(p, run, ref)
            print(f"[ksplit-generic] {name}", inf, flush=True)
            assert ok, inf
        else:
            assert np.array_equal(run.result_bits().reshape(ref.shape), exact_expected_bits(p, ref))
        assert run.guards_intact()
        bits1 = run.result_bits().copy()
        run()
        assert np.array_equal(bits1, run.result_bits())


@pytest.mark.parametrize("seed,count", [(23, 60)])
def test_fuzz_generic_ksplit_integer_exact(seed, count):
    """Random problems (both layouts, both dtypes, groups, strides,
    dilations, padding) on the generic family with split-K: bit-exact."""
    rng = random.Random(seed + 11)
    for i, p in enumerate(fuzz_problems(seed, count)):
        ksplit = rng.choice([2, 3, 5, 16])
        pl = plan_for(p, cbd.KERNEL_GENERIC, ksplit=ksplit)
        print(f"[fuzz-ksplit-generic] i={i} ksplit={ksplit}->{pl.info().ksplit} {p}", flush=True)
        sh = oracle.shapes(p)
        dy = small_ints(7000 * seed + 3 * i + 1, sh["dy"]).astype(np.float32)
        w = small_ints(7000 * seed + 3 * i + 2, sh["w"]).astype(np.float32)
        ws = torch.empty(max(pl.workspace_size(), 1), dtype=torch.uint8, device="cuda")
        run = DeviceRun(p, pl, to_device(dy, p), to_device(w, p), workspace=ws)()
        ref = oracle.bwd_data(p, dy, w)
        assert np.array_equal(run.result_bits().reshape(ref.shape), exact_expected_bits(p, ref)), (p, ksplit)
        assert run.guards_intact(), (p, ksplit)


@pytest.mark.parametrize("name,n", [("c4", 1), ("c4", 2)])
def test_auto_split_runs_with_workspace(name, n):
    """The planner's split configuration: cbd_run (and cbd_run_ws with too
    small a workspace) runs the unsplit plan, cbd_run_ws with
    auto_workspace_bytes runs the split one (the same bits as an explicit
    ksplit plan); all within the tolerance of the oracle."""
    p = by_name(name) if n is None else by_name(name).with_(n=n)
    pl = plan_for(p)
    info = pl.info()
    print(f"[auto-split] {name} n={p.n} auto_ksplit={info.auto_ksplit}", flush=True)
    assert info.ksplit == 1 and info.workspace_bytes == 0
    assert info.auto_ksplit > 1 and pl.workspace_size() == info.auto_workspace_bytes > 0
    dy, w = operands(p)
    dyd, wd = to_device(dy, p), to_device(w, p)
    ws = torch.empty(info.auto_workspace_bytes, dtype=torch.uint8, device="cuda")
    small_ws = torch.empty(info.auto_workspace_bytes - 256, dtype=torch.uint8, device="cuda")
    plain = DeviceRun(p, pl, dyd, wd)().result_bits().copy()
    small = DeviceRun(p, pl, dyd, wd, workspace=small_ws)().result_bits().copy()
    split_run = DeviceRun(p, pl, dyd, wd, workspace=ws)()
    split = split_run.result_bits().copy()
    assert split_run.guards_intact()
    explicit = DeviceRun(p, plan_for(p, info.kernel, ksplit=info.auto_ksplit), dyd, wd, workspace=ws)()
    assert np.array_equal(plain, small)
    assert np.array_equal(split, explicit.result_bits())
    ref = oracle.bwd_data(p, dy, w)
    for bits in (plain, split):
        if p.dtype == "f32":
            ok, inf = check_f32(bits.view(np.float32).reshape(ref.shape), ref)
        else:
            ok, inf = check_bf16(bits.reshape(ref.shape), ref)
        assert ok, inf


@pytest.mark.parametrize("name", ["c1", "c3a", "c3b", "c4", "c5-s2", "c2-14-3"])
def test_per_class_launches_match_single_launch(name):
    """One launch per residue class gives the same bits as the single launch."""
    p = by_name(name)
    print(f"[per-class] {name}", flush=True)
    dy, w = operands(p)
    dy_d, w_d = to_device(dy, p), to_device(w, p)
    # the same family on both sides
    pl = plan_for(p, per_class=True)
    one = DeviceRun(p, plan_for(p, pl.info().kernel), dy_d, w_d)()
    assert pl.info().launches >= pl.info().num_subgemms
    many = DeviceRun(p, pl, dy_d, w_d)()
    assert np.array_equal(one.result_bits(), many.result_bits())
    assert many.guards_intact()


# Shape-specialised instances of the large-tile kernel: level 2 (the whole
# geometry compile-time: the headline problem at any batch and even width)
# and level 1 (k tiles per tap and taps per class compile-time).
STATIC_CASES = [
    ("c4", {}, 2), ("c4", {"n": 3}, 2), ("c4", {"n": 1, "wi": 100}, 2),
    ("c4", {"c": 1024}, 1), ("c4", {"n": 2, "hi": 3}, 1), ("c4", {"n": 2, "wi": 301}, 1),
]


@pytest.mark.parametrize("idx", range(len(STATIC_CASES)))
def test_static_shape_instance_matches_runtime(idx):
    """Each shape-specialised instance gives the same bits as the
    descriptor-driven kernel (which the oracle checks everywhere else), and
    matches the oracle at sampled outputs, including ragged batches/widths."""
    name, kw, level = STATIC_CASES[idx]
    p = by_name(name).with_(**kw)
    print(f"[static] {name} {kw} level={level}", flush=True)
    dy, w = operands(p)
    dy_d, w_d = to_device(dy, p), to_device(w, p)
    pa, pb = plan_for(p, static_shape=-1), plan_for(p)
    assert pa.info().static_shape == 0 and pb.info().static_shape == level
    a = DeviceRun(p, pa, dy_d, w_d)()
    b = DeviceRun(p, pb, dy_d, w_d)()
    bits = b.result_bits()
    assert np.array_equal(a.result_bits(), bits)
    assert b.guards_intact()
    rng = np.random.default_rng(100 + idx)
    cnt = 3000
    pts = np.stack([rng.integers(0, p.n, cnt), rng.integers(0, p.c, cnt),
                    rng.integers(0, p.hi, cnt), rng.integers(0, p.wi, cnt)], axis=1)
    pts[:4] = [[p.n - 1, p.c - 1, p.hi - 1, p.wi - 1], [0, 0, 0, 0],
               [p.n - 1, 0, p.hi - 1, p.wi - 2], [0, p.c - 1, 0, 1]]
    ref = oracle.bwd_data_at(p, dy, w, pts)
    got = bits.reshape(p.n, p.hi, p.wi, p.c)[pts[:, 0], pts[:, 2], pts[:, 3], pts[:, 1]]
    ok, info = check_bf16(got, ref)
    assert ok, info


GENERIC_STATIC = ("c1", "c2-14-1", "c2-14-3", "c2-15-1", "c2-15-3", "c2-16-1", "c2-16-3", "c3a", "c3b")


@pytest.mark.parametrize("name", GENERIC_STATIC)
def test_generic_static_instance_matches_runtime(name):
    """The generic family's shape-specialised instance of each workload
    problem gives the same bits as its descriptor-driven kernel, on random
    and integer operands; integer operands bit-exact against the oracle."""
    p = by_name(name)
    print(f"[static-generic] {name}", flush=True)
    pa, pb = plan_for(p, static_shape=-1), plan_for(p)
    assert pa.info().static_shape == 0 and pb.info().static_shape == 2
    for kind in ("dist", "int"):
        dy, w = operands(p, kind)
        dy_d, w_d = to_device(dy, p), to_device(w, p)
        a = DeviceRun(p, pa, dy_d, w_d)()
        b = DeviceRun(p, pb, dy_d, w_d)()
        assert np.array_equal(a.result_bits(), b.result_bits()), kind
        assert a.guards_intact() and b.guards_intact()
        if kind == "int":
            ref = oracle.bwd_data(p, dy, w)
            assert np.array_equal(b.result_bits().reshape(ref.shape), exact_expected_bits(p, ref))


@pytest.mark.parametrize("name", ["c5-s2", "c5-s1"])
def test_grouped_static_instance_matches_runtime(name):
    """The grouped 4x4x4-MFMA kernel's shape-specialised instance of each
    grouped workload problem gives the same bits as its descriptor-driven
    kernel, on random and integer operands; integer operands bit-exact
    against the oracle."""
    p = by_name(name)
    print(f"[static-grouped] {name}", flush=True)
    pa, pb = plan_for(p, static_shape=-1), plan_for(p)
    assert pa.info().static_shape == 0 and pb.info().static_shape == 2
    for kind in ("dist", "int"):
        dy, w = operands(p, kind)
        dy_d, w_d = to_device(dy, p), to_device(w, p)
        a = DeviceRun(p, pa, dy_d, w_d)()
        b = DeviceRun(p, pb, dy_d, w_d)()
        assert np.array_equal(a.result_bits(), b.result_bits()), kind
        assert a.guards_intact() and b.guards_intact()
        if kind == "int":
            ref = oracle.bwd_data(p, dy, w)
            assert np.array_equal(b.result_bits().reshape(ref.shape), exact_expected_bits(p, ref))


# One class at phase (0,0) over every stride block (1x1 filters at stride S):
# the epilogue writes each block whole, zeros included.  (name, N, G, C, K,
# Hi, Wi, stride, layout, dtype)
ZBLOCK_CASES = [
    ("nchw-f32-pairs", 3, 1, 20, 12, 28, 28, (2, 2), NCHW, "f32"),
    ("nchw-f32-oddw", 2, 1, 16, 8, 14, 27, (2, 2), NCHW, "f32"),
    ("nchw-bf16-pairs", 2, 1, 24, 40, 15, 30, (2, 2), NCHW, "bf16"),
    ("nhwc-f32", 2, 1, 20, 12, 28, 28, (2, 2), NHWC, "f32"),
    ("nhwc-bf16-s32", 2, 2, 16, 24, 13, 11, (3, 2), NHWC, "bf16"),
    ("nchw-f32-s21", 2, 1, 33, 17, 9, 10, (2, 1), NCHW, "f32"),
]


@pytest.mark.parametrize("idx", range(len(ZBLOCK_CASES)))
def test_whole_block_epilogue(idx):
    name, n, g, c, k, hi, wi, st, lay, dt = ZBLOCK_CASES[idx]
    p = Problem(name, n, g, c, k, hi, wi, 1, 1, st[0], st[1], 0, 0, 1, 1, lay, dt, "u", "u", 0, 0)
    print(f"[zblock] {p}", flush=True)
    pl = plan_for(p, cbd.KERNEL_GENERIC)
    info = pl.info()
    assert info.zero_in_epilogue == 1 and info.grid_zero == 0 and info.launches == 1
    sh = oracle.shapes(p)
    dy = small_ints(9100 + idx, sh["dy"]).astype(np.float32)
    w = small_ints(9200 + idx, sh["w"]).astype(np.float32)
    run = DeviceRun(p, pl, to_device(dy, p), to_device(w, p))()
    ref = oracle.bwd_data(p, dy, w)
    assert np.array_equal(run.result_bits().reshape(ref.shape), exact_expected_bits(p, ref))
    assert run.guards_intact()


def test_non_default_stream():
    p = by_name("c3a")
    dy, w = operands(p)
    ref = oracle.bwd_data(p, dy, w)
    pl = plan_for(p)
    s = torch.cuda.Stream()
    dy_d, w_d = to_device(dy, p), to_device(w, p)
    torch.cuda.synchronize()
    with torch.cuda.stream(s):
        run = DeviceRun(p, pl, dy_d, w_d)
        run(stream=s)
    s.synchronize()
    ok, info = check(p, run, ref)
    assert ok, info


def test_convenience_entry_matches_torch_layouts():
    """conv2d_bwd_data with torch-style arguments (NCHW and NHWC)."""
    p = by_name("c3a")
    dy, w = operands(p)
    ref = oracle.bwd_data(p, dy, w)
    dx = cbd.conv2d_bwd_data(to_device(dy, p), to_device(w, p), (p.n, p.c, p.hi, p.wi),
                             stride=2, padding=1, dilation=1, groups=1, layout="nchw")
    ok, info = check_f32(dx.cpu().numpy(), ref)
    assert ok, info


# ------------------------------------------------------------------- fuzz ---

def fuzz_problems(seed, count, *, layouts=(NCHW, NHWC), dtypes=("f32", "bf16"), family=None):
    rng = random.Random(seed)
    out = []
    while len(out) < count:
        layout = rng.choice(layouts)
        dtype = rng.choice(dtypes)
        if family == cbd.KERNEL_NHWC_BF16:
            g = rng.choice([1, 1, 2])
            cg = 8 * rng.randint(1, 40)
            kg = 32 * rng.randint(1, 6)
            layout, dtype = NHWC, "bf16"
        elif family == cbd.KERNEL_GROUPED:
            cg = rng.choice([1, 2, 4, 8])
            kg = cg
            g = rng.choice([1, 2, 4, 8, 16, 32, 64])
            layout = NHWC
        elif family == cbd.KERNEL_NCHW_ROWS:
            g = rng.randint(1, 4)
            cg, kg = rng.randint(1, 40), rng.randint(1, 40)
            layout = NCHW
        else:
            g = rng.randint(1, 4)
            cg, kg = rng.randint(1, 40), rng.randint(1, 40)
        p = Problem("fuzz", rng.randint(1, 3), g, g * cg, g * kg, rng.randint(1, 23),
                    rng.randint(1, 23), rng.randint(1, 5), rng.randint(1, 5), rng.randint(1, 4),
                    rng.randint(1, 4), rng.randint(0, 3), rng.randint(0, 3), rng.randint(1, 3),
                    rng.randint(1, 3), layout, dtype, "u", "u", 0, 0)
        if (p.hi + 2 * p.ph - p.dh * (p.y - 1) - 1 < 0
                or p.wi + 2 * p.pw - p.dw * (p.x - 1) - 1 < 0):
            continue
        if family in (cbd.KERNEL_GROUPED, cbd.KERNEL_NHWC_BF16, cbd.KERNEL_NCHW_ROWS):
            try:
                if plan_for(p, family).info().kernel != family:
                    continue
            except cbd.CbdError:
                continue
        out.append(p)
    return out


@pytest.mark.parametrize("family,seed,count", [
    (cbd.KERNEL_GENERIC, 11, 150),
    (cbd.KERNEL_NHWC_BF16, 12, 60),
    (cbd.KERNEL_GROUPED, 13, 80),
    (cbd.KERNEL_NCHW_ROWS, 14, 150),
])
def test_fuzz_integer_exact(family, seed, count):
    for i, p in enumerate(fuzz_problems(seed, count, family=family)):
        print(f"[fuzz] family={family} i={i} {p}", flush=True)
        sh = oracle.shapes(p)
        dy = small_ints(1000 * seed + 3 * i + 1, sh["dy"]).astype(np.float32)
        w = small_ints(1000 * seed + 3 * i + 2, sh["w"]).astype(np.float32)
        pl = plan_for(p, family)
        run = DeviceRun(p, pl, to_device(dy, p), to_device(w, p))()
        ref = oracle.bwd_data(p, dy, w)
        want = exact_expected_bits(p, ref)
        want = oracle.bf16_bits_to_f32(want) if p.dtype == "bf16" else want.view(np.float32)
        got = run.result_f32()
        assert np.array_equal(got, want.reshape(got.shape)), p
        assert run.guards_intact(), p


@pytest.mark.parametrize("family,seed,count", [
    (cbd.KERNEL_GENERIC, 21, 60),
    (cbd.KERNEL_NHWC_BF16, 22, 30),
    (cbd.KERNEL_GROUPED, 23, 40),
    (cbd.KERNEL_NCHW_ROWS, 24, 60),
])
def test_fuzz_random_values(family, seed, count):
    for i, p in enumerate(fuzz_problems(seed, count, family=family)):
        print(f"[fuzz-val] family={family} i={i} {p}", flush=True)
        sh = oracle.shapes(p)
        from cbd_inputs import to_dtype
        dy = to_dtype(uniform(2000 * seed + 3 * i + 1, sh["dy"]), p.dtype)
        w = to_dtype(uniform(2000 * seed + 3 * i + 2, sh["w"]), p.dtype)
        pl = plan_for(p, family)
        run = DeviceRun(p, pl, to_device(dy, p), to_device(w, p))()
        ok, info = check(p, run, oracle.bwd_data(p, dy, w))
        assert ok, (p, info)


def row_load_patterns(p):
    """Row-load patterns of the residue classes of an f32 NCHW problem on
    the generic family (host restatement of the kernel's choice, used only
    to show which K orders a fuzz set reaches): per class, 1/2 = one tap
    per filter row in 1/2 rows, 3/4 = two taps two apart in 1/2 rows,
    5 = 3x3 adjacent taps, 0 = another order."""
    import math

    def axis(f, s, d, pad):
        step = s // math.gcd(s, d)
        out = []
        for ph in range(s):
            taps = [j for j in range(f) if (ph + pad - j * d) % s == 0]
            if taps:
                out.append((len(taps), taps[0], step))
        return out
    pats = set()
    for th, _, _ in axis(p.y, p.sh, p.dh, p.ph):
        for tw, cw, stw in axis(p.x, p.sw, p.dw, p.pw):
            if tw == 1 and cw + 1 < p.x:
                pats.add({1: 1, 2: 2}.get(th, 0))
            elif tw == 2 and stw == 2:
                pats.add({1: 3, 2: 4}.get(th, 0))
            elif tw == 3 and stw == 1 and th == 3:
                pats.add(5)
            else:
                pats.add(0)
    return pats


@pytest.mark.parametrize("seed,count,ksplit", [(31, 120, 0), (32, 40, 3)])
def test_fuzz_generic_row_loads(seed, count, ksplit):
    """f32 NCHW problems on the generic family whose classes read W a
    filter row at a time (1-3 taps per load): filters 2, 3 and 5, strides
    1-3, dilation 1-2, groups, K/G not a multiple of 4 (k rows past K/G),
    ragged channel and position tiles, two- and four-wave workgroups, and
    split-K over the row-load k tiles; bit-exact on integer operands, every
    pattern reached."""
    rng = random.Random(seed)
    seen = set()
    waves = set()
    done = 0
    while done < count:
        g = rng.choice([1, 1, 2, 3])
        f = rng.choice([2, 3, 3, 5])
        s = rng.choice([1, 2, 2, 3])
        d = rng.choice([1, 1, 2])
        pad = rng.randint(0, 2)
        p = Problem("fuzz-rows", rng.randint(1, 3), g, g * rng.randint(1, 40), g * rng.randint(1, 40),
                    rng.randint(2, 20), rng.randint(2, 20), f, f, s, s, pad, pad, d, d, NCHW, "f32",
                    "u", "u", 0, 0)
        if p.hi + 2 * p.ph - p.dh * (p.y - 1) - 1 < 0 or p.wi + 2 * p.pw - p.dw * (p.x - 1) - 1 < 0:
            continue
        pats = row_load_patterns(p)
        seen |= pats
        opts = {"ksplit": ksplit} if ksplit else {}
        pl = plan_for(p, cbd.KERNEL_GENERIC, **opts)
        waves.add(pl.info().threads_main // 64)
        print(f"[fuzz-rows] i={done} pats={sorted(pats)} ksplit={pl.info().ksplit} "
              f"waves={pl.info().threads_main // 64} {p}", flush=True)
        sh = oracle.shapes(p)
        dy = small_ints(9000 * seed + 3 * done + 1, sh["dy"]).astype(np.float32)
        w = small_ints(9000 * seed + 3 * done + 2, sh["w"]).astype(np.float32)
        ws = torch.empty(max(pl.workspace_size(), 1), dtype=torch.uint8, device="cuda")
        run = DeviceRun(p, pl, to_device(dy, p), to_device(w, p), workspace=ws)()
        ref = oracle.bwd_data(p, dy, w)
        assert np.array_equal(run.result_bits().reshape(ref.shape), exact_expected_bits(p, ref)), p
        assert run.guards_intact(), p
        done += 1
    assert {1, 2, 3, 4, 5} <= seen, seen
    if not ksplit:  # two-wave workgroups (all classes one- to four-tap row loads) reached too
        assert 2 in waves and 4 in waves, waves


# Grouped family: the pipelined row kernel with several rows per workgroup
# (the automatic choice gives tiny problems one row each), and the one-row
# kernel it replaces (rows_per_wg = -1).
@pytest.mark.parametrize("seed,count", [(15, 80), (16, 40)])
def test_fuzz_grouped_rows_per_wg(seed, count):
    rng = random.Random(seed + 1000)
    for i, p in enumerate(fuzz_problems(seed, count, family=cbd.KERNEL_GROUPED)):
        rows = rng.choice([-1, 1, 2, 3, 5, 64])
        pl = plan_for(p, cbd.KERNEL_GROUPED, rows)
        inf = pl.info()
        print(f"[fuzz-rows] i={i} rows={rows} got={inf.rows_per_wg} lds={inf.lds_dynamic} {p}",
              flush=True)
        if rows == -1:
            assert inf.rows_per_wg == 0
        sh = oracle.shapes(p)
        dy = small_ints(3000 * seed + 3 * i + 1, sh["dy"]).astype(np.float32)
        w = small_ints(3000 * seed + 3 * i + 2, sh["w"]).astype(np.float32)
        run = DeviceRun(p, pl, to_device(dy, p), to_device(w, p))()
        want = exact_expected_bits(p, oracle.bwd_data(p, dy, w))
        want = oracle.bf16_bits_to_f32(want) if p.dtype == "bf16" else want.view(np.float32)
        got = run.result_f32()
        assert np.array_equal(got, want.reshape(got.shape)), (p, rows)
        assert run.guards_intact(), (p, rows)


@pytest.mark.parametrize("name", ["c5-s2", "c5-s1"])
@pytest.mark.parametrize("rows,dot,cols", [(-1, False, 0), (1, False, 0), (3, False, 0),
                                           (56, False, 0), (1, True, 0), (3, True, 0),
                                           (56, True, 0), (0, False, 8), (5, False, 12),
                                           (2, False, 56)])
def test_grouped_workload_rows_per_wg(name, rows, dot, cols):
    p = by_name(name)
    print(f"[rows] {name} rows={rows} dot={dot} cols={cols}", flush=True)
    dy, w = operands(p)
    pl = plan_for(p, cbd.KERNEL_AUTO, rows, dot, cols)
    inf = pl.info()
    assert inf.kernel == cbd.KERNEL_GROUPED
    assert inf.variant == (1 if rows == -1 else 2 if dot else 3)
    run = DeviceRun(p, pl, to_device(dy, p), to_device(w, p))()
    ok, info = check(p, run, oracle.bwd_data(p, dy, w))
    assert ok, info
    assert run.guards_intact()


# The 4x4x4-MFMA pipelined kernel: bf16, 4 channels per group, 32 or 64
# groups, random geometry and rows per workgroup; integer-exact.
@pytest.mark.parametrize("seed,count", [(17, 60)])
def test_fuzz_grouped_mfma(seed, count):
    rng = random.Random(seed)
    done = 0
    while done < count:
        g = rng.choice([32, 64])
        p = Problem("fuzz", rng.randint(1, 3), g, 4 * g, 4 * g, rng.randint(1, 40),
                    rng.randint(1, 40), rng.randint(1, 3), rng.randint(1, 3), rng.randint(1, 3),
                    rng.randint(1, 3), rng.randint(0, 2), rng.randint(0, 2), rng.randint(1, 2),
                    rng.randint(1, 2), NHWC, "bf16", "u", "u", 0, 0)
        if (p.hi + 2 * p.ph - p.dh * (p.y - 1) - 1 < 0
                or p.wi + 2 * p.pw - p.dw * (p.x - 1) - 1 < 0):
            continue
        rows = rng.choice([0, 1, 2, 5, 64])
        cols = rng.choice([0, 0, 4, 8, 13])
        merge = rng.choice([0, 1])
        try:
            pl = plan_for(p, cbd.KERNEL_GROUPED, rows, False, cols, merge_phases=merge)
        except cbd.CbdError:
            continue
        if pl.info().variant not in (3, 5):
            continue
        print(f"[fuzz-mfma] i={done} rows={rows} cols={cols} merge={merge} variant={pl.info().variant} {p}",
              flush=True)
        sh = oracle.shapes(p)
        dy = small_ints(4000 * seed + 3 * done + 1, sh["dy"]).astype(np.float32)
        w = small_ints(4000 * seed + 3 * done + 2, sh["w"]).astype(np.float32)
        run = DeviceRun(p, pl, to_device(dy, p), to_device(w, p))()
        want = oracle.bf16_bits_to_f32(exact_expected_bits(p, oracle.bwd_data(p, dy, w)))
        got = run.result_f32()
        assert np.array_equal(got, want.reshape(got.shape)), (p, rows, cols)
        assert run.guards_intact(), (p, rows, cols)
        done += 1


# The 4x4x4-MFMA kernel with the four phases of a 2 x 2 stride in one
# workgroup: random sizes (odd and even extents, so that phases differ in
# rows and columns), filters up to 4 x 4, padding, rows and column blocks;
# integer operands bit-exact against the oracle, and the same bits as one
# class per workgroup.
@pytest.mark.parametrize("seed,count", [(19, 50)])
def test_fuzz_grouped_mfma_merged(seed, count):
    rng = random.Random(seed)
    done = 0
    while done < count:
        g = rng.choice([32, 64])
        y, x = rng.randint(2, 4), rng.randint(2, 4)
        p = Problem("fuzz-merged", rng.randint(1, 3), g, 4 * g, 4 * g, rng.randint(2, 37),
                    rng.randint(2, 37), y, x, 2, 2, rng.randint(0, y - 1), rng.randint(0, x - 1), 1, 1,
                    NHWC, "bf16", "u", "u", 0, 0)
        if (p.hi + 2 * p.ph - (p.y - 1) - 1 < 0 or p.wi + 2 * p.pw - (p.x - 1) - 1 < 0):
            continue
        rows = rng.choice([0, 1, 2, 3, 64])
        cols = rng.choice([0, 0, 4, 8, 13])
        try:
            pm = plan_for(p, cbd.KERNEL_GROUPED, rows, False, cols, merge_phases=1)
        except cbd.CbdError:
            continue
        pu = plan_for(p, cbd.KERNEL_GROUPED, rows, False, cols, merge_phases=-1)
        assert pm.info().variant == 5 and pu.info().variant == 3
        print(f"[fuzz-merged] i={done} rows={rows} cols={cols} R={pm.info().rows_per_wg} "
              f"CB={pm.info().cols_per_wg} grid={pm.info().grid_main} {p}", flush=True)
        sh = oracle.shapes(p)
        dy = small_ints(5000 * seed + 3 * done + 1, sh["dy"]).astype(np.float32)
        w = small_ints(5000 * seed + 3 * done + 2, sh["w"]).astype(np.float32)
        dy_d, w_d = to_device(dy, p), to_device(w, p)
        rm = DeviceRun(p, pm, dy_d, w_d)()
        ru = DeviceRun(p, pu, dy_d, w_d)()
        want = oracle.bf16_bits_to_f32(exact_expected_bits(p, oracle.bwd_data(p, dy, w)))
        got = rm.result_f32()
        assert np.array_equal(got, want.reshape(got.shape)), (p, rows, cols)
        assert np.array_equal(rm.result_bits(), ru.result_bits()), (p, rows, cols)
        assert rm.guards_intact() and ru.guards_intact(), (p, rows, cols)
        done += 1


@pytest.mark.parametrize("name", ["c5-s2", "gs-c4-56-s2", "gs-c4-7-s2"])
def test_grouped_merged_matches_per_class(name):
    """The merged-phase plan (merge_phases = 1) of a stride-2 grouped
    workload gives the same bits as its default one-class-per-workgroup
    plan, on the workload's distributions; against the oracle within the
    bf16 tolerance."""
    p = by_name(name) if not name.startswith("gs-") else [q for q in GROUPED_SWEEP if q.name == name][0]
    print(f"[merged] {name}", flush=True)
    pm, pu = plan_for(p, merge_phases=1), plan_for(p)
    assert pm.info().variant == 5 and pu.info().variant == 3
    dy, w = operands(p)
    dy_d, w_d = to_device(dy, p), to_device(w, p)
    rm = DeviceRun(p, pm, dy_d, w_d)()
    ru = DeviceRun(p, pu, dy_d, w_d)()
    assert np.array_equal(rm.result_bits(), ru.result_bits())
    ok, info = check(p, rm, oracle.bwd_data(p, dy, w))
    assert ok, info
    assert rm.guards_intact() and ru.guards_intact()


# The grouped sweep (32 groups x 4..32 channels, 56..7 pixels, stride 1/2)
# at the batch the benchmark times (N = 32), so the launch configurations it
# times (rows and columns per workgroup, grid) are the ones checked: every
# output element against the oracle's loop nest, with the workload's
# distributions, then again with small-integer operands, bit for bit.
@pytest.mark.parametrize("name", [p.name for p in GROUPED_SWEEP])
def test_grouped_sweep_full(name):
    p = [q for q in GROUPED_SWEEP if q.name == name][0]
    assert p.n == 32
    pl = plan_for(p)
    inf = pl.info()
    print(f"[sweep] {name} n={p.n} variant={inf.variant} rows={inf.rows_per_wg} "
          f"cols={inf.cols_per_wg} grid={inf.grid_main}", flush=True)
    dy, w = operands(p)
    run = DeviceRun(p, pl, to_device(dy, p), to_device(w, p))()
    ok, info = check(p, run, oracle.bwd_data(p, dy, w))
    assert ok, (name, info)
    assert run.guards_intact()
    del dy, w
    dy, w = operands(p, "int")
    run = DeviceRun(p, pl, to_device(dy, p), to_device(w, p))()
    want = oracle.bf16_bits_to_f32(exact_expected_bits(p, oracle.bwd_data(p, dy, w)))
    got = run.result_f32()
    assert np.array_equal(got, want.reshape(got.shape)), name
    assert run.guards_intact()


# The 16x16x16-MFMA grouped kernel: bf16, 8 (as pairs), 16 or 32 channels
# per group, random geometry, rows and column blocks; integer-exact.
@pytest.mark.parametrize("seed,count", [(18, 60), (28, 40)])
def test_fuzz_grouped_wide(seed, count):
    rng = random.Random(seed)
    done = 0
    while done < count:
        cg = rng.choice([8, 16, 32])
        # group counts in slices of 256 bytes, including ones that do not
        # divide 256 and ones above 256 (the planner picks this kernel for them)
        g = rng.choice({8: [16, 32, 64, 48, 80, 512], 16: [8, 16, 32, 24, 40, 264],
                        32: [4, 8, 32, 12, 20, 260]}[cg])
        hmax = 40 if g <= 64 else 10
        p = Problem("fuzz", rng.randint(1, 2), g, cg * g, cg * g, rng.randint(1, hmax),
                    rng.randint(1, hmax), rng.randint(1, 3), rng.randint(1, 3), rng.randint(1, 3),
                    rng.randint(1, 3), rng.randint(0, 2), rng.randint(0, 2), rng.randint(1, 2),
                    rng.randint(1, 2), NHWC, "bf16", "u", "u", 0, 0)
        if (p.hi + 2 * p.ph - p.dh * (p.y - 1) - 1 < 0
                or p.wi + 2 * p.pw - p.dw * (p.x - 1) - 1 < 0):
            continue
        rows = rng.choice([0, 1, 3, 64])
        cols = rng.choice([0, 0, 16, 20])
        try:
            pl = plan_for(p, cbd.KERNEL_GROUPED, rows, False, cols)
        except cbd.CbdError:
            continue
        if pl.info().variant != 4 or pl.info().grid_main == 0:
            continue
        print(f"[fuzz-wide] i={done} rows={rows} cols={cols} {p}", flush=True)
        sh = oracle.shapes(p)
        dy = small_ints(6000 * seed + 3 * done + 1, sh["dy"]).astype(np.float32)
        w = small_ints(6000 * seed + 3 * done + 2, sh["w"]).astype(np.float32)
        run = DeviceRun(p, pl, to_device(dy, p), to_device(w, p))()
        want = oracle.bf16_bits_to_f32(exact_expected_bits(p, oracle.bwd_data(p, dy, w)))
        got = run.result_f32()
        assert np.array_equal(got, want.reshape(got.shape)), (p, rows, cols)
        assert run.guards_intact(), (p, rows, cols)
        done += 1


# ------------------------------------------------------------ graph capture ---

@pytest.mark.parametrize("name", ["c3b", "c4", "c5-s2"])
def test_graph_replay_matches_eager(name):
    """cbd_run is capturable (kernel launches only): every replay of a captured
    graph, with eager work and synchronisation between replays, reproduces the
    eager result bit for bit (c3b includes the zero-fill launch)."""
    p = by_name(name)
    print(f"[graph] {name}", flush=True)
    dy, w = operands(p)
    pl = plan_for(p)
    dy_d, w_d = to_device(dy, p), to_device(w, p)
    tdt = torch.float32 if p.dtype == "f32" else torch.bfloat16
    dx = torch.empty(pl.shapes()["dx"], dtype=tdt, device="cuda")
    cbd.run(pl, dy_d, w_d, dx)
    torch.cuda.synchronize()
    want = dx.clone()
    graph = torch.cuda.CUDAGraph()
    cap = torch.cuda.Stream()
    cap.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(cap):
        with torch.cuda.graph(graph, stream=cap):
            cbd.run(pl, dy_d, w_d, dx, stream=cap)
    torch.cuda.synchronize()
    for rep in range(4):
        dx.fill_(float("nan"))
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(dx.view(torch.int16 if p.dtype == "bf16" else torch.int32),
                           want.view(torch.int16 if p.dtype == "bf16" else torch.int32)), (name, rep)


# ------------------------------------------------- zero-insertion baseline ---

def plan_no_split(p, force=cbd.KERNEL_AUTO):
    dt = cbd.F32 if p.dtype == "f32" else cbd.BF16
    return cbd.plan(p.n, p.g, p.c, p.k, p.hi, p.wi, p.y, p.x, (p.sh, p.sw), (p.ph, p.pw),
                    (p.dh, p.dw), p.layout, dt, force_kernel=force, no_split=True)


@pytest.mark.parametrize("name", ["c1", "c2-14-3", "c3a", "c3b", "c5-s2"])
def test_no_split_vs_oracle(name):
    """The zero-insertion comparison mode computes the same dX."""
    p = by_name(name)
    print(f"[no-split] {name}", flush=True)
    dy, w = operands(p)
    run = DeviceRun(p, plan_no_split(p), to_device(dy, p), to_device(w, p))()
    ok, info = check(p, run, oracle.bwd_data(p, dy, w))
    assert ok, info
    assert run.guards_intact()


def test_no_split_c4_integer_exact():
    """Headline problem in the zero-insertion form on the large-tile kernel:
    bit-exact against the oracle on integer data."""
    p = by_name("c4")
    print("[no-split] c4", flush=True)
    dy, w = operands(p, "int")
    pl = plan_no_split(p)
    assert pl.info().kernel == cbd.KERNEL_NHWC_BF16
    run = DeviceRun(p, pl, to_device(dy, p), to_device(w, p))()
    got = run.result_f32()
    want = oracle.bf16_bits_to_f32(exact_expected_bits(p, oracle_full(p, "int")))
    assert np.array_equal(got, want.reshape(got.shape))
    assert run.guards_intact()


@pytest.mark.parametrize("family,seed,count", [
    (cbd.KERNEL_GENERIC, 31, 60),
    (cbd.KERNEL_NHWC_BF16, 32, 25),
])
def test_fuzz_no_split_integer_exact(family, seed, count):
    for i, p in enumerate(fuzz_problems(seed, count, family=family)):
        print(f"[fuzz-no-split] family={family} i={i} {p}", flush=True)
        sh = oracle.shapes(p)
        dy = small_ints(3000 * seed + 3 * i + 1, sh["dy"]).astype(np.float32)
        w = small_ints(3000 * seed + 3 * i + 2, sh["w"]).astype(np.float32)
        try:
            pl = plan_no_split(p, family)
        except cbd.CbdError:
            continue  # e.g. more than 16 taps for the large-tile kernel
        run = DeviceRun(p, pl, to_device(dy, p), to_device(w, p))()
        want = exact_expected_bits(p, oracle.bwd_data(p, dy, w))
        want = oracle.bf16_bits_to_f32(want) if p.dtype == "bf16" else want.view(np.float32)
        got = run.result_f32()
        assert np.array_equal(got, want.reshape(got.shape)), p
        assert run.guards_intact(), p


# ------------------------------------------------------------- alignment ---

@pytest.mark.parametrize("name,layout,dtype,elem_off", [
    ("c1", NCHW, "f32", 1), ("c2-14-3", NCHW, "f32", 3), ("c3b", NCHW, "f32", 1),
    ("c1", NHWC, "bf16", 1), ("c3a", NHWC, "bf16", 5)])
def test_generic_unaligned_views(name, layout, dtype, elem_off):
    """The generic family runs on tensor views that start a few elements into
    their storage (element-aligned, not 16-byte aligned) and gives the same
    bits as on aligned tensors, within the oracle's tolerance."""
    p = by_name(name).with_(layout=layout, dtype=dtype)
    print(f"[align] {name} layout={layout} {dtype} +{elem_off}", flush=True)
    dy, w = operands(p)
    pl = plan_for(p, cbd.KERNEL_GENERIC)
    inf = pl.info()
    es = 4 if dtype == "f32" else 2
    assert inf.align_dy == es and inf.align_w == es
    sh = pl.shapes()
    tdt = torch.float32 if dtype == "f32" else torch.bfloat16

    def view(a):
        flat = torch.zeros(a.size + elem_off, dtype=tdt, device="cuda")
        flat[elem_off:] = torch.from_numpy(np.ascontiguousarray(a).reshape(-1)).to(tdt).cuda()
        return flat[elem_off:].view(a.shape)
    dy_v, w_v = view(dy), view(w)
    assert (dy_v.data_ptr() % 16) != 0
    dx_off = elem_off if inf.align_dx == es else 16 // es
    buf = torch.full((int(np.prod(sh["dx"])) + dx_off + 64,), float("nan"), dtype=tdt, device="cuda")
    dx_v = buf[dx_off:dx_off + int(np.prod(sh["dx"]))].view(sh["dx"])
    cbd.run(pl, dy_v, w_v, dx_v)
    aligned = DeviceRun(p, pl, to_device(dy, p), to_device(w, p))()
    torch.cuda.synchronize()
    got = dx_v.cpu()
    want = aligned.dx.cpu()
    iv = torch.int32 if dtype == "f32" else torch.int16
    assert torch.equal(got.view(iv), want.view(iv))
    assert bool(torch.isnan(buf[:dx_off].float()).all()) and bool(torch.isnan(buf[dx_off + got.numel():].float()).all())
    ok, info = check(p, aligned, oracle.bwd_data(p, dy, w))
    assert ok, info


# ------------------------------------------------------------- concurrency ---

def test_concurrent_runs_on_two_streams():
    """Two host threads, each with its own stream, call cbd_run at the same
    time: each its own plan (generic family / grouped family) and both a
    third plan they share (plans are immutable).  Every result equals the
    single-threaded result bit for bit."""
    import threading
    names = ("c3a", "c5-s2", "c2-16-3")
    probs = {n: by_name(n) for n in names}
    plans = {n: plan_for(probs[n]) for n in names}
    ins = {}
    ref = {}
    for n in names:
        p = probs[n]
        dy, w = operands(p)
        ins[n] = (to_device(dy, p), to_device(w, p))
        ref[n] = DeviceRun(p, plans[n], *ins[n])().result_bits().copy()
    streams = [torch.cuda.Stream(), torch.cuda.Stream()]
    own = ["c3a", "c5-s2"]
    outs = [{n: DeviceRun(probs[n], plans[n], *ins[n]) for n in (own[t], "c2-16-3")} for t in range(2)]
    torch.cuda.synchronize()
    start = threading.Barrier(2)
    errors = []

    def worker(t):
        try:
            start.wait()
            for _ in range(40):
                for n, r in outs[t].items():
                    cbd.run(plans[n], r.dy_d, r.w_d, r.dx, stream=streams[t])
            streams[t].synchronize()
        except Exception as e:  # reported below
            errors.append(e)
    th = [threading.Thread(target=worker, args=(t,)) for t in range(2)]
    for x in th:
        x.start()
    for x in th:
        x.join(timeout=120)
    assert not errors, errors
    assert not any(x.is_alive() for x in th)
    torch.cuda.synchronize()
    for t in range(2):
        for n, r in outs[t].items():
            assert np.array_equal(r.result_bits(), ref[n]), (t, n)
            assert r.guards_intact()
