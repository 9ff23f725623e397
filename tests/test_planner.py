"""Host planner and C ABI tests (CPU only: cbd_plan needs no GPU).

* Residue classes: tap sets, phases, dY offsets and position counts checked
  against brute-force enumeration of the forward window.
* Coverage: every dX position is written by exactly one sub-GEMM or one
  zero region (the single-writer property the kernels rely on).
* CPU plan executor: a literal evaluation of the plan's descriptors must
  equal the oracle bit for bit on integer data, over random tiny problems
  (groups, strides, dilations with gcd(S, D) > 1, padding, both layouts).
* Boundary: invalid and unsupported problems, NULL / misaligned /
  overlapping pointers, exported symbols, plan accounting.
"""
import ctypes
import math
import os
import random
import subprocess
import sys

import numpy as np
import pytest

import dnn_conv2d_bwd_amd as cbd
import oracle
from cbd_inputs import PROBLEMS, small_ints
from cbd_inputs.problems import NCHW, NHWC, Problem

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def tiny(rng, layouts=(NCHW, NHWC)):
    while True:
        g = rng.randint(1, 4)
        p = Problem("t", rng.randint(1, 2), g, g * rng.randint(1, 3), g * rng.randint(1, 3),
                    rng.randint(1, 11), rng.randint(1, 11), rng.randint(1, 5), rng.randint(1, 5),
                    rng.randint(1, 4), rng.randint(1, 4), rng.randint(0, 3), rng.randint(0, 3),
                    rng.randint(1, 4), rng.randint(1, 4), rng.choice(layouts), "f32", "int", "int",
                    0, 0)
        if (p.hi + 2 * p.ph - p.dh * (p.y - 1) - 1 >= 0
                and p.wi + 2 * p.pw - p.dw * (p.x - 1) - 1 >= 0):
            return p


def plan_of(p, force=cbd.KERNEL_AUTO):
    dt = cbd.F32 if p.dtype == "f32" else cbd.BF16
    return cbd.plan(p.n, p.g, p.c, p.k, p.hi, p.wi, p.y, p.x, (p.sh, p.sw), (p.ph, p.pw),
                    (p.dh, p.dw), p.layout, dt, force_kernel=force)


def execute_plan(pl, p, dy, w):
    """Evaluate the plan's sub-GEMM descriptors and zero regions literally."""
    info = pl.info()
    ho_n, wo_n = info.ho, info.wo
    cg, kg = p.c // p.g, p.k // p.g
    if p.layout == NCHW:
        dy4, w4 = dy, w
    else:
        dy4, w4 = np.transpose(dy, (0, 3, 1, 2)), np.transpose(w, (0, 3, 1, 2))
    dx = np.full((p.n, p.c, p.hi, p.wi), np.nan)
    writes = np.zeros((p.hi, p.wi), dtype=np.int64)
    for s in pl.subgemms():
        for th in range(s.pos_h):
            for tw in range(s.pos_w):
                hi, wi = s.phase_h + p.sh * th, s.phase_w + p.sw * tw
                writes[hi, wi] += 1
                acc = np.zeros((p.n, p.c))
                for jh in range(s.taps_h):
                    for jw in range(s.taps_w):
                        ty, tx = s.class_h + s.tstep_h * jh, s.class_w + s.tstep_w * jw
                        ho = th + s.beta_h - s.delta_h * jh
                        wo = tw + s.beta_w - s.delta_w * jw
                        if not (0 <= ho < ho_n and 0 <= wo < wo_n):
                            continue
                        for g in range(p.g):
                            d = dy4[:, g * kg:(g + 1) * kg, ho, wo]          # (n, kg)
                            wt = w4[g * kg:(g + 1) * kg, :, ty, tx]          # (kg, cg)
                            acc[:, g * cg:(g + 1) * cg] += d @ wt
                dx[:, :, hi, wi] = acc
    for z in pl.zero_regions():
        for a in range(z.pos_h):
            for b in range(z.pos_w):
                hi, wi = z.phase_h + p.sh * a, z.phase_w + p.sw * b
                writes[hi, wi] += 1
                dx[:, :, hi, wi] = 0.0
    return (dx if p.layout == NCHW else np.transpose(dx, (0, 2, 3, 1))), writes


def test_axis_classes_match_enumeration():
    """For every class: its taps are exactly those reaching its phase, and
    tap j at position t reads dY row t + beta - delta*j."""
    rng = random.Random(1)
    for _ in range(400):
        p = tiny(rng)
        pl = plan_of(p)
        ho_n, wo_n = pl.info().ho, pl.info().wo
        for s in pl.subgemms():
            for axis in ("h", "w"):
                S, D, P, F, L, O = ((p.sh, p.dh, p.ph, p.y, p.hi, ho_n) if axis == "h"
                                    else (p.sw, p.dw, p.pw, p.x, p.wi, wo_n))
                phase, cls = getattr(s, "phase_" + axis), getattr(s, "class_" + axis)
                taps, T = getattr(s, "taps_" + axis), getattr(s, "tstep_" + axis)
                beta, delta = getattr(s, "beta_" + axis), getattr(s, "delta_" + axis)
                pos = getattr(s, "pos_" + axis)
                assert T == S // math.gcd(S, D) and delta == D // math.gcd(S, D)
                assert pos == len(range(phase, L, S))
                want = {f for f in range(F) if (phase + P - f * D) % S == 0}
                assert want == {cls + T * j for j in range(taps)}
                for t in range(pos):
                    h = phase + S * t
                    for j in range(taps):
                        f = cls + T * j
                        assert (h + P - f * D) == S * (t + beta - delta * j)


def test_plan_executor_matches_oracle_bitwise():
    rng = random.Random(2)
    for i in range(600):
        p = tiny(rng)
        sh = oracle.shapes(p)
        dy, w = small_ints(10 * i + 1, sh["dy"]), small_ints(10 * i + 2, sh["w"])
        pl = plan_of(p)
        got, writes = execute_plan(pl, p, dy, w)
        assert np.all(writes == 1), (p, writes)
        assert np.array_equal(got, oracle.bwd_data(p, dy, w)), p


def test_workload_plans():
    expect = {  # (sub-GEMMs, zero regions, kernel)
        "c1": (1, 0, cbd.KERNEL_GENERIC), "c3a": (4, 0, cbd.KERNEL_GENERIC),
        "c3b": (1, 3, cbd.KERNEL_GENERIC), "c4": (2, 0, cbd.KERNEL_NHWC_BF16),
        "c5-s2": (4, 0, cbd.KERNEL_GROUPED), "c5-s1": (1, 0, cbd.KERNEL_GROUPED),
    }
    for p in PROBLEMS:
        forces = (cbd.KERNEL_AUTO, cbd.KERNEL_GENERIC) + ((cbd.KERNEL_NCHW_ROWS,) if p.layout == NCHW else ())
        for force in forces:
            pl = plan_of(p, force)
            info = pl.info()
            ho, wo = oracle.out_hw(p)
            assert (info.ho, info.wo) == (ho, wo)
            assert info.useful_flops == 2 * p.n * p.c * (p.k // p.g) * ho * wo * p.y * p.x
            subs = pl.subgemms()
            assert [s.id for s in subs] == list(range(len(subs)))
            assert all(subs[i].k >= subs[i + 1].k for i in range(len(subs) - 1))  # LPT
            assert info.launches == 1 + (info.grid_zero > 0)
            if info.kernel == cbd.KERNEL_NCHW_ROWS:
                # workgroups = images x groups x 16-channel blocks x row blocks;
                # unreached phases written by the same launch
                assert all(s.tiles == 0 and s.tile_begin == 0 for s in subs)
                assert info.grid_main == (p.n * p.g * -(-(p.c // p.g) // 16)
                                          * -(-p.hi // info.rows_per_wg))
                assert info.grid_zero == 0 and 0 < info.lds_dynamic <= 160 * 1024
                continue
            tiles = 0
            for s in subs:
                assert s.tile_begin == tiles
                tiles += s.tiles
            # the generic family folds the zero-fill workgroups into its launch,
            # or writes the unreached positions in its epilogue
            fused = info.num_zero_regions > 0 and info.grid_zero == 0 and not info.zero_in_epilogue
            zero_wgs = -(-info.zero_elems // (256 * 2)) if fused and p.layout == NCHW else 0
            assert tiles + zero_wgs == info.grid_main
        if p.name in expect:
            info = plan_of(p).info()
            assert (info.num_subgemms, info.num_zero_regions, info.kernel) == expect[p.name]
    c4 = plan_of([q for q in PROBLEMS if q.name == "c4"][0])
    assert [(s.m, s.n, s.k) for s in c4.subgemms()] == [(2048, 4096, 2048)] * 2
    assert c4.info().grid_main == 256 and c4.info().executed_macs * 2 == c4.info().useful_flops
    c3b_p = [q for q in PROBLEMS if q.name == "c3b"][0]
    for force in (cbd.KERNEL_AUTO, cbd.KERNEL_GENERIC):
        c3b = plan_of(c3b_p, force)
        assert c3b.info().zero_elems == 32 * 64 * 28 * 28 * 3 // 4
        assert c3b.info().launches == 1 and c3b.info().grid_zero == 0  # zeros in the main launch
        assert c3b.info().zero_in_epilogue == 1 and c3b.info().grid_main == 392  # written by its epilogue
    # the row-block family (forced only): one workgroup per CU, balanced row blocks
    rows = {q.name: plan_of(q, cbd.KERNEL_NCHW_ROWS).info() for q in PROBLEMS if q.layout == NCHW}
    assert {n: (i.grid_main, i.rows_per_wg) for n, i in rows.items() if n in ("c1", "c2-14-3", "c3a", "c3b")} \
        == {"c1": (8, 4), "c2-14-3": (256, 4), "c3a": (256, 14), "c3b": (256, 14)}


def test_forced_kernels():
    c4 = [q for q in PROBLEMS if q.name == "c4"][0]
    assert plan_of(c4, cbd.KERNEL_GENERIC).info().kernel == cbd.KERNEL_GENERIC
    c1 = [q for q in PROBLEMS if q.name == "c1"][0]
    with pytest.raises(cbd.CbdError) as e:
        plan_of(c1, cbd.KERNEL_NHWC_BF16)
    assert e.value.status == 2
    with pytest.raises(cbd.CbdError) as e:
        plan_of(c1, cbd.KERNEL_GROUPED)
    assert e.value.status == 2


def test_no_split_plans():
    """Zero-insertion comparison mode: one sub-GEMM over all dX positions and
    all taps, no zero regions, MACs = N*C*(K/G)*Hi*Wi*Y*X."""
    for q in PROBLEMS:
        dt = cbd.F32 if q.dtype == "f32" else cbd.BF16
        pl = cbd.plan(q.n, q.g, q.c, q.k, q.hi, q.wi, q.y, q.x, (q.sh, q.sw), (q.ph, q.pw),
                      (q.dh, q.dw), q.layout, dt, no_split=True)
        inf = pl.info()
        assert inf.num_subgemms == 1 and inf.num_zero_regions == 0 and inf.launches == 1
        assert inf.kernel != cbd.KERNEL_GROUPED
        assert inf.executed_macs == q.n * q.c * (q.k // q.g) * q.hi * q.wi * q.y * q.x
        (s,) = pl.subgemms()
        assert (s.pos_h, s.pos_w, s.taps_h, s.taps_w) == (q.hi, q.wi, q.y, q.x)
        assert s.tile_begin == 0 and s.tiles == inf.grid_main
    c4 = [q for q in PROBLEMS if q.name == "c4"][0]
    split = plan_of(c4).info().executed_macs
    assert cbd.plan(problem=cbd.make_problem(c4.n, 1, c4.c, c4.k, c4.hi, c4.wi, c4.y, c4.x,
                                             (c4.sh, c4.sw), 0, 1, "nhwc", "bf16"),
                    no_split=True).info().executed_macs == 2 * split
    c5 = [q for q in PROBLEMS if q.name == "c5-s1"][0]
    with pytest.raises(cbd.CbdError) as e:
        cbd.plan(c5.n, c5.g, c5.c, c5.k, c5.hi, c5.wi, c5.y, c5.x, 1, 1, 1, "nhwc", "bf16",
                 force_kernel=cbd.KERNEL_GROUPED, no_split=True)
    assert e.value.status == 2
    bad = cbd.PlanOptions(cbd.KERNEL_AUTO, 2)
    h = ctypes.c_void_p()
    prob = cbd.make_problem(2, 1, 8, 8, 8, 8, 3, 3, 2, 1, 1, "nchw", "f32")
    assert cbd._lib.cbd_plan_ex(ctypes.byref(prob), ctypes.byref(bad), ctypes.byref(h)) == 1


@pytest.mark.parametrize("field,value,status", [
    ("n", 0, 1), ("g", 3, 1), ("c", -1, 1), ("stride_h", 0, 1), ("pad_w", -1, 1),
    ("dil_w", 0, 1), ("layout", 7, 1), ("dtype", 9, 1), ("y", 40, 1),
    ("stride_h", 9, 2), ("dil_h", 65, 2), ("n", 1 << 40, 2),
])
def test_invalid_and_unsupported(field, value, status):
    prob = cbd.make_problem(2, 2, 8, 8, 16, 16, 3, 3, 2, 1, 1, "nchw", "f32")
    setattr(prob, field, value)
    if field == "stride_h" and value == 9:
        prob.stride_w = 8  # 72 > 64 classes
    with pytest.raises(cbd.CbdError) as e:
        cbd.Plan(prob)
    assert e.value.status == status
    assert cbd._lib.cbd_last_error().decode() != ""


def test_tensor_size_limit():
    prob = cbd.make_problem(1024, 1, 1024, 8, 64, 64, 1, 1, 1, 0, 1, "nhwc", "f32")  # dX 16 GiB
    with pytest.raises(cbd.CbdError) as e:
        cbd.Plan(prob)
    assert e.value.status == 2


def test_exports_and_null_handling():
    L = ctypes.CDLL(cbd.LIB_PATH)
    header = open(os.path.join(ROOT, "include", "cbd.h")).read()
    for name in cbd.EXPORTS:
        assert hasattr(L, name), name
        assert name + "(" in header, name
    # every function declared in the header is exported
    import re
    declared = set(re.findall(r"\b(cbd_[a-z_]+)\s*\(", header))
    assert declared == set(cbd.EXPORTS)
    assert cbd._lib.cbd_status_string(0) == b"CBD_OK"
    assert cbd._lib.cbd_status_string(3) == b"CBD_ERR_HIP"
    cbd._lib.cbd_plan_destroy(None)
    assert cbd._lib.cbd_plan(None, None) == 1
    pl = cbd.plan(2, 1, 16, 16, 14, 14, 3, 3, 1, 1, 1, "nchw", "f32")
    assert cbd._lib.cbd_plan_info(pl.handle, None) == 1
    assert cbd._lib.cbd_plan_subgemm(pl.handle, 5, ctypes.byref(cbd.SubGemm())) == 1
    assert cbd._lib.cbd_plan_zero_region(pl.handle, 0, ctypes.byref(cbd.ZeroRegion())) == 1
    # run-time argument checks happen before any HIP call
    base = 1 << 40
    assert cbd.run_raw(pl, 0, base, base + (1 << 30)) == 1                   # NULL dy
    assert cbd.run_raw(pl, base + 2, base + (1 << 28), base + (1 << 30)) == 2  # misaligned (f32: 4 bytes)
    assert cbd.run_raw(pl, base, base + (1 << 28), base + 64) == 1           # dx overlaps dy


def test_ksplit_plans():
    """Split-K accounting: S workgroups per tile (clamped to the shortest
    class's k tiles), a 256x256 f32 workspace block per workgroup, one more
    launch, cbd_run refusing such a plan before any HIP call."""
    c4 = [p for p in PROBLEMS if p.name == "c4"][0]
    base = cbd.plan(problem=cbd.make_problem(c4.n, c4.g, c4.c, c4.k, c4.hi, c4.wi, c4.y, c4.x,
                                             (c4.sh, c4.sw), (c4.ph, c4.pw), (c4.dh, c4.dw),
                                             c4.layout, cbd.BF16))
    b = base.info()
    assert b.ksplit == 1 and b.workspace_bytes == 0 and base.workspace_size() == 0
    for s in (2, 3, 8, 64):
        pl = cbd.plan(c4.n, c4.g, c4.c, c4.k, c4.hi, c4.wi, c4.y, c4.x, (c4.sh, c4.sw),
                      (c4.ph, c4.pw), (c4.dh, c4.dw), c4.layout, cbd.BF16, ksplit=s)
        i = pl.info()
        # c4: K/G = 2048 and one tap per class: 64 k tiles, so 64 splits at most
        assert i.ksplit == min(s, 64)
        assert i.grid_main == b.grid_main * i.ksplit
        assert i.workspace_bytes == i.grid_main * 256 * 256 * 4 == pl.workspace_size()
        assert i.launches == b.launches + 1
        assert i.executed_macs == b.executed_macs
        for sg in pl.subgemms():
            assert sg.tiles % i.ksplit == 0 and sg.tile_begin % i.ksplit == 0
        big = 1 << 40
        assert cbd.run_raw(pl, big, big + (1 << 30), big + (1 << 31)) == 1  # no workspace
        ws = big + (1 << 33)
        L = cbd._lib
        P = ctypes.c_void_p
        assert L.cbd_run_ws(pl.handle, P(big), P(big + (1 << 30)), P(big + (1 << 31)), P(ws),
                            ctypes.c_uint64(i.workspace_bytes - 1), P(0)) == 1  # too small
        assert L.cbd_run_ws(pl.handle, P(big), P(big + (1 << 30)), P(big + (1 << 31)), P(ws + 16),
                            ctypes.c_uint64(i.workspace_bytes), P(0)) == 2      # misaligned
        assert L.cbd_run_ws(pl.handle, P(big), P(big + (1 << 30)), P(big + (1 << 31)), P(big),
                            ctypes.c_uint64(i.workspace_bytes), P(0)) == 1      # overlaps dy
    # a short class clamps S: 3x3 stride 2 has a one-tap class (K/G = 64: 2 k tiles)
    pl = cbd.plan(2, 1, 256, 64, 9, 9, 3, 3, 2, 1, 1, "nhwc", "bf16", ksplit=8)
    assert pl.info().kernel == cbd.KERNEL_NHWC_BF16 and pl.info().ksplit == 2
    # the grouped and row-block families refuse it
    with pytest.raises(cbd.CbdError):
        cbd.plan(2, 32, 128, 128, 12, 12, 3, 3, 2, 1, 1, "nhwc", "bf16", ksplit=2)
    with pytest.raises(cbd.CbdError):
        cbd.plan(2, 1, 16, 16, 14, 14, 3, 3, 1, 1, 1, "nchw", "f32", ksplit=2,
                 force_kernel=cbd.KERNEL_NCHW_ROWS)
    with pytest.raises(cbd.CbdError):
        cbd.plan(2, 1, 16, 16, 14, 14, 3, 3, 1, 1, 1, "nchw", "f32", ksplit=65)


def test_static_shape_plans():
    c4 = [p for p in PROBLEMS if p.name == "c4"][0]
    args = (c4.n, c4.g, c4.c, c4.k, c4.hi, c4.wi, c4.y, c4.x, (c4.sh, c4.sw), (c4.ph, c4.pw),
            (c4.dh, c4.dw), c4.layout, cbd.BF16)
    a, b = cbd.plan(*args, static_shape=-1).info(), cbd.plan(*args).info()
    assert (a.grid_main, a.launches, a.executed_macs) == (b.grid_main, b.launches, b.executed_macs)
    # the headline geometry gets the fully specialised instance (level 2)
    assert a.static_shape == 0 and b.static_shape == 2
    assert cbd.plan(*args, static_shape=1).info().static_shape == 2
    assert cbd.plan(*args, ksplit=2).info().static_shape == 0
    assert cbd.plan(*args, per_class=True).info().static_shape == 1
    # any batch or (even) width keeps level 2; other geometry with K/G = 2048
    # and one tap per class gets level 1
    for n, wi in ((3, 512), (1, 64), (16, 1000)):
        assert cbd.plan(n, 1, 2048, 2048, 1, wi, 1, 2, (1, 2), 0, 1, "nhwc", "bf16").info().static_shape == 2
    lvl1 = [(16, 1, 1024, 2048, 1, 512, 1, 2, (1, 2), 0, 1),   # C = 1024
            (4, 1, 2048, 2048, 3, 64, 1, 2, (1, 2), 0, 1),     # Hi = 3
            (4, 1, 2048, 2048, 1, 63, 1, 2, (1, 2), 0, 1),     # odd width
            (4, 1, 2048, 2048, 1, 64, 1, 2, (1, 2), (0, 1), 1),  # padding
            (2, 2, 4096, 4096, 1, 64, 1, 2, (1, 2), 0, 1)]     # two groups
    for q in lvl1:
        assert cbd.plan(*q, "nhwc", "bf16").info().static_shape == 1, q
    other = (2, 1, 256, 1024, 1, 64, 1, 2, (1, 2), 0, 1, "nhwc", "bf16")
    assert cbd.plan(*other).info().static_shape == 0
    with pytest.raises(cbd.CbdError):   # K/G = 1024: no instance
        cbd.plan(*other, static_shape=1)
    with pytest.raises(cbd.CbdError):   # split-K: no instance
        cbd.plan(*args, static_shape=1, ksplit=2)


GENERIC_STATIC = ("c1", "c2-14-1", "c2-14-3", "c2-15-1", "c2-15-3", "c2-16-1", "c2-16-3", "c3a", "c3b")


def test_generic_static_shapes():
    """Every workload problem on the generic family finds its
    shape-specialised instance (the compiled table is current), with the
    same launch as the descriptor-driven plan; other shapes, split-K,
    per-class, no-split and static_shape=-1 plans do not, and requiring one
    where none exists is refused."""
    by = {q.name: q for q in PROBLEMS}
    for name in GENERIC_STATIC:
        p = by[name]
        a, b = plan_of(p).info(), plan_of(p, cbd.KERNEL_GENERIC).info()
        assert (a.kernel, a.static_shape, b.static_shape) == (cbd.KERNEL_GENERIC, 2, 2), name
        dt = cbd.F32 if p.dtype == "f32" else cbd.BF16
        args = (p.n, p.g, p.c, p.k, p.hi, p.wi, p.y, p.x, (p.sh, p.sw), (p.ph, p.pw), (p.dh, p.dw), p.layout, dt)
        d = cbd.plan(*args, static_shape=-1).info()
        assert d.static_shape == 0
        assert (d.grid_main, d.grid_zero, d.launches, d.tile_m, d.tile_n, d.threads_main) == \
            (a.grid_main, a.grid_zero, a.launches, a.tile_m, a.tile_n, a.threads_main)
        assert cbd.plan(*args, static_shape=1).info().static_shape == 2
        for kw in ({"ksplit": 2}, {"per_class": True}, {"no_split": True}):
            assert cbd.plan(*args, **kw).info().static_shape == 0, (name, kw)
    # a batch the table does not hold: the descriptor-driven kernel
    c3a = by["c3a"]
    assert plan_of(c3a.with_(n=31)).info().static_shape == 0
    with pytest.raises(cbd.CbdError):
        cbd.plan(31, 1, 64, 64, 28, 28, 3, 3, 2, 1, 1, "nchw", "f32", static_shape=1)


GROUPED_STATIC = ("c5-s2", "c5-s1")


def test_grouped_static_shapes():
    """The grouped workload problems find their shape-specialised instance of
    the 4x4x4-MFMA kernel with the descriptor-driven plan's launch; forced
    row kernels, per-class plans, other batches and static_shape=-1 plans do
    not, and requiring one where none exists is refused."""
    by = {q.name: q for q in PROBLEMS}
    for name in GROUPED_STATIC:
        p = by[name]
        a = plan_of(p).info()
        assert (a.kernel, a.variant, a.static_shape) == (cbd.KERNEL_GROUPED, 3, 2), name
        dt = cbd.F32 if p.dtype == "f32" else cbd.BF16
        args = (p.n, p.g, p.c, p.k, p.hi, p.wi, p.y, p.x, (p.sh, p.sw), (p.ph, p.pw), (p.dh, p.dw), p.layout, dt)
        d = cbd.plan(*args, static_shape=-1).info()
        assert (d.static_shape, d.variant) == (0, 3)
        assert (d.grid_main, d.grid_zero, d.launches, d.rows_per_wg, d.cols_per_wg, d.threads_main) == \
            (a.grid_main, a.grid_zero, a.launches, a.rows_per_wg, a.cols_per_wg, a.threads_main)
        assert cbd.plan(*args, static_shape=1).info().static_shape == 2
        assert cbd.plan(*args, per_class=True).info().static_shape == 0
    c5 = by["c5-s2"]
    assert plan_of(c5.with_(n=63)).info().static_shape == 0
    with pytest.raises(cbd.CbdError):
        cbd.plan(63, 32, 128, 128, 56, 56, 3, 3, 2, 1, 1, "nhwc", "bf16", static_shape=1)


def test_merge_phases_option():
    """merge_phases = 1 runs the stride-2 grouped workload with the four
    phases in one workgroup (variant 5, whole-image grid, no class tile
    ranges); the default keeps one class per workgroup; a problem the merged
    form does not serve is refused, and out-of-range values are invalid."""
    by = {q.name: q for q in PROBLEMS}
    p = by["c5-s2"]
    args = (p.n, p.g, p.c, p.k, p.hi, p.wi, p.y, p.x, (p.sh, p.sw), (p.ph, p.pw), (p.dh, p.dw), p.layout, cbd.BF16)
    d = cbd.plan(*args).info()
    assert d.variant == 3
    pm = cbd.plan(*args, merge_phases=1)
    m = pm.info()
    assert (m.variant, m.static_shape, m.num_zero_regions, m.launches) == (5, 0, 0, 1)
    subs = pm.subgemms()
    assert len(subs) == 4 and all(s.tiles == 0 and s.tile_begin == 0 for s in subs)
    assert {(s.phase_h, s.phase_w) for s in subs} == {(0, 0), (0, 1), (1, 0), (1, 1)}
    ph = max(s.pos_h for s in subs)
    pw = max(s.pos_w for s in subs)
    assert m.grid_main == p.n * -(-ph // m.rows_per_wg) * -(-pw // m.cols_per_wg)
    assert m.cols_per_wg % 4 == 0 and 0 < m.lds_dynamic <= 160 * 1024
    assert m.useful_flops == d.useful_flops and m.executed_macs == d.executed_macs
    assert cbd.plan(*args, merge_phases=-1).info().variant == 3
    s1 = by["c5-s1"]
    with pytest.raises(cbd.CbdError):  # stride 1: one class
        cbd.plan(s1.n, s1.g, s1.c, s1.k, s1.hi, s1.wi, s1.y, s1.x, (s1.sh, s1.sw), (s1.ph, s1.pw),
                 (s1.dh, s1.dw), s1.layout, cbd.BF16, merge_phases=1)
    with pytest.raises(cbd.CbdError):  # per_class
        cbd.plan(*args, merge_phases=1, per_class=True)
    with pytest.raises(cbd.CbdError):
        cbd.plan(*args, merge_phases=2)


@pytest.mark.skipif(os.path.exists("/dev/kfd"),
                    reason="passes made-up device addresses to a real launch: only on a machine "
                           "with no GPU driver at all, where the launch itself must fail")
def test_run_without_device_returns_hip_error():
    """On a machine with no GPU, cbd_run reports CBD_ERR_HIP instead of
    aborting (run in a child process to keep this one clean).  The addresses
    are never dereferenced here: with no device the launch fails before any
    kernel runs; where a GPU driver exists the test is skipped."""
    code = (
        "import dnn_conv2d_bwd_amd as cbd\n"
        "pl = cbd.plan(2, 1, 16, 16, 14, 14, 3, 3, 1, 1, 1, 'nchw', 'f32')\n"
        "b = 1 << 40\n"
        "st = cbd.run_raw(pl, b, b + (1 << 28), b + (1 << 30))\n"
        "print('STATUS', st)\n"
    )
    r = subprocess.run([sys.executable, "-c", code], cwd=ROOT, capture_output=True, text=True,
                       timeout=120, env={**os.environ, "HIP_VISIBLE_DEVICES": "-1"})
    assert r.returncode == 0, r.stderr
    assert "STATUS 3" in r.stdout, r.stdout + r.stderr


def test_generic_tile_choice():
    """Generic family: 64x64 tiles only when that grid has at least 1024
    tiles (four per CU), 32x32 otherwise, 16 rows for at most 16 channels per
    group (16 wide too on small grids); k tiles 8 wide up to 32x32."""
    from cbd_inputs.problems import Problem as P_
    small = [q for q in PROBLEMS if q.name in ("c2-14-3", "c3a", "c3b")]
    for q in small:
        inf = plan_of(q, cbd.KERNEL_GENERIC).info()
        assert (inf.tile_m, inf.tile_n, inf.tile_k) == (32, 32, 8), q.name
    c1 = plan_of([q for q in PROBLEMS if q.name == "c1"][0], cbd.KERNEL_GENERIC).info()
    assert (c1.tile_m, c1.tile_n, c1.tile_k) == (16, 16, 8)
    # eight waves per workgroup only for long K (>= 32 k tiles) on small grids;
    # f32 KCYX classes that read W a filter row at a time count k tiles of 4 k
    # rows over all taps (8 for the 3x3 32-channel problems: four waves)
    waves = {q.name: plan_of(q, cbd.KERNEL_GENERIC).info().threads_main // 64 for q in PROBLEMS[:9]}
    assert waves == {"c1": 4, "c2-14-1": 4, "c2-14-3": 4, "c2-15-1": 4, "c2-15-3": 4,
                     "c2-16-1": 4, "c2-16-3": 4, "c3a": 2, "c3b": 4}
    # the same 3x3 stride-1 32-channel problem in NHWC (no row loads): eight
    nhwc = [q for q in PROBLEMS if q.name == "c2-14-3"][0].with_(layout=NHWC)
    assert plan_of(nhwc, cbd.KERNEL_GENERIC).info().threads_main == 8 * 64
    big = P_("g64", 16, 1, 64, 64, 64, 64, 1, 1, 1, 1, 0, 0, 1, 1, NCHW, "f32", "u", "u", 0, 0)
    inf = plan_of(big, cbd.KERNEL_GENERIC).info()
    assert (inf.tile_m, inf.tile_n, inf.tile_k, inf.grid_main) == (64, 64, 16, 1024)
    just_below = big.with_(hi=62, wi=64)  # 16*62*64 / 64 = 992 tiles of 64x64
    inf = plan_of(just_below, cbd.KERNEL_GENERIC).info()
    assert (inf.tile_m, inf.tile_n) == (32, 32)


def test_grouped_beyond_256_groups_no_crash():
    """Grouped problems the 16x16x16-MFMA kernel accepts with G > 256 (or G
    not dividing 256): a problem with no sub-GEMM plans as zero-fill only,
    and asking for the row / direct kernels (rows_per_wg = -1) is refused,
    never a crash (these once divided by zero in the planner)."""
    # 1x1 filter, stride 2, pad 1, 1x1 input: the one position is padding, no class has positions
    for g in (512, 1024):
        pl = cbd.plan(1, g, 8 * g, 8 * g, 1, 1, 1, 1, 2, 1, 1, "nhwc", "bf16")
        inf = pl.info()
        assert inf.num_subgemms == 0 and inf.grid_main == 0 and inf.grid_zero > 0
    for g, hw in ((512, 8), (1024, 4), (48, 8)):
        with pytest.raises(cbd.CbdError) as e:
            cbd.plan(2, g, 8 * g, 8 * g, hw, hw, 3, 3, 1, 1, 1, "nhwc", "bf16", rows_per_wg=-1)
        assert e.value.status == 2
        # without the option the 16x16x16-MFMA kernel takes them
        inf = cbd.plan(2, g, 8 * g, 8 * g, hw, hw, 3, 3, 1, 1, 1, "nhwc", "bf16").info()
        assert inf.kernel == cbd.KERNEL_GROUPED and inf.variant == 4


def test_alignment_requirements():
    """Generic family: element alignment (16 bytes for dx when a zero-fill
    writes 16-byte NHWC chunks); other families 16 bytes.  A misaligned
    pointer is refused before anything is launched."""
    f32 = cbd.plan(2, 1, 16, 16, 14, 14, 3, 3, 1, 1, 1, "nchw", "f32", force_kernel=cbd.KERNEL_GENERIC).info()
    assert (f32.kernel, f32.align_dy, f32.align_w, f32.align_dx) == (cbd.KERNEL_GENERIC, 4, 4, 4)
    # row-block family (forced): element loads of dY, 16-byte loads of W when its
    # 16-channel blocks are whole (f32), dx stores as wide as a dX row allows
    for wi, vb in ((14, 8), (15, 4), (16, 16)):
        r = cbd.plan(2, 1, 16, 16, 14, wi, 3, 3, 1, 1, 1, "nchw", "f32", force_kernel=cbd.KERNEL_NCHW_ROWS).info()
        assert (r.kernel, r.align_dy, r.align_w, r.align_dx) == (cbd.KERNEL_NCHW_ROWS, 4, 16, vb)
    r = cbd.plan(2, 1, 12, 16, 14, 14, 3, 3, 1, 1, 1, "nchw", "f32", force_kernel=cbd.KERNEL_NCHW_ROWS).info()
    assert (r.kernel, r.align_dy, r.align_w, r.align_dx) == (cbd.KERNEL_NCHW_ROWS, 4, 4, 8)
    r = cbd.plan(2, 1, 16, 16, 14, 15, 3, 3, 1, 1, 1, "nchw", "bf16", force_kernel=cbd.KERNEL_NCHW_ROWS).info()
    assert (r.kernel, r.align_dy, r.align_dx) == (cbd.KERNEL_NCHW_ROWS, 2, 2)
    bf = cbd.plan(2, 1, 12, 12, 9, 9, 3, 3, 1, 1, 1, "nchw", "bf16", force_kernel=cbd.KERNEL_GENERIC).info()
    assert (bf.align_dy, bf.align_w, bf.align_dx) == (2, 2, 2)
    # NCHW zero-fill writes elements; NHWC rows of 64 f32 channels in 16-byte
    # chunks (1x1 stride 2 with padding 1: the reached phase is (1,1))
    z_nchw = cbd.plan(2, 1, 64, 64, 28, 28, 1, 1, 2, 1, 1, "nchw", "f32", force_kernel=cbd.KERNEL_GENERIC).info()
    assert z_nchw.num_zero_regions == 3 and z_nchw.align_dx == 4 and not z_nchw.zero_in_epilogue
    z_nhwc = cbd.plan(2, 1, 64, 64, 28, 28, 1, 1, 2, 1, 1, "nhwc", "f32",
                      force_kernel=cbd.KERNEL_GENERIC).info()
    assert z_nhwc.num_zero_regions == 3 and (z_nhwc.align_dy, z_nhwc.align_dx) == (4, 16)
    # without padding the one class is phase (0,0): its epilogue writes whole
    # 2x2 blocks, in (value, 0) pairs for NCHW with an even width
    for lay, wi, ax in (("nchw", 28, 8), ("nchw", 27, 4), ("nhwc", 28, 4)):
        zb = cbd.plan(2, 1, 64, 64, 28, wi, 1, 1, 2, 0, 1, lay, "f32", force_kernel=cbd.KERNEL_GENERIC).info()
        assert (zb.zero_in_epilogue, zb.grid_zero, zb.launches, zb.align_dx) == (1, 0, 1, ax), (lay, wi)
    zb16 = cbd.plan(2, 1, 64, 64, 28, 28, 1, 1, 2, 0, 1, "nchw", "bf16", force_kernel=cbd.KERNEL_GENERIC).info()
    assert zb16.align_dx == 4
    c4 = cbd.plan(16, 1, 2048, 2048, 1, 512, 1, 2, (1, 2), 0, 1, "nhwc", "bf16").info()
    assert (c4.align_dy, c4.align_w, c4.align_dx) == (16, 16, 16)
    pl = cbd.plan(2, 1, 16, 16, 14, 14, 3, 3, 1, 1, 1, "nchw", "f32", force_kernel=cbd.KERNEL_GENERIC)
    big = 1 << 40
    for off in ((2, 0, 0), (0, 1, 0), (0, 0, 3)):   # refused before any launch
        assert cbd.run_raw(pl, big + off[0], big + (1 << 28) + off[1], big + (1 << 30) + off[2]) == 2
    assert "aligned" in cbd._lib.cbd_last_error().decode()


def test_cbd_log_plan_dump():
    """CBD_LOG=1 describes every plan on stderr; unset or 0 prints nothing."""
    code = ("import dnn_conv2d_bwd_amd as cbd\n"
            "cbd.plan(32, 1, 64, 64, 28, 28, 1, 1, 2, 0, 1, 'nchw', 'f32')\n")
    for val, expect in (("1", True), ("0", False), ("", False)):
        r = subprocess.run([sys.executable, "-c", code], cwd=ROOT, capture_output=True, text=True,
                           timeout=120, env={**os.environ, "CBD_LOG": val})
        assert r.returncode == 0, r.stderr
        assert ("[cbd] plan:" in r.stderr) == expect, (val, r.stderr)
        if expect:
            assert "kernel generic" in r.stderr and "sub-GEMM 0:" in r.stderr
            assert r.stderr.count("zero region:") == 3


def test_split_k_plans():
    """Split-K: explicit splits on the large-tile and generic families
    (clamped to the shortest class's k tiles, one f32 partial tile per
    (tile, split) in the workspace, a finalising launch), and the planner's
    own split configuration (large-tile kernel, below 64 tiles)."""
    by = {q.name: q for q in PROBLEMS}

    def mk(p, **kw):
        dt = cbd.F32 if p.dtype == "f32" else cbd.BF16
        return cbd.plan(p.n, p.g, p.c, p.k, p.hi, p.wi, p.y, p.x, (p.sh, p.sw), (p.ph, p.pw),
                        (p.dh, p.dw), p.layout, dt, **kw)

    # explicit splits on the generic family, clamped: c3b has one 1x1 class,
    # 64/8 = 8 k tiles; c3a's shortest class has one tap, 8 k tiles; c1 has
    # 9 taps x 16/8
    for name, req, want in (("c3b", 64, 8), ("c3a", 5, 5), ("c1", 64, 18), ("c2-14-3", 3, 3)):
        pl = mk(by[name], force_kernel=cbd.KERNEL_GENERIC, ksplit=req)
        i = pl.info()
        assert (i.kernel, i.ksplit) == (cbd.KERNEL_GENERIC, want), name
        gemm_tiles = sum(s.tiles for s in pl.subgemms())
        assert gemm_tiles % want == 0
        assert i.workspace_bytes == gemm_tiles * i.tile_m * i.tile_n * 4
        assert pl.workspace_size() == i.workspace_bytes
        assert i.launches == 2 + (i.grid_zero > 0)
        assert (i.auto_ksplit, i.auto_workspace_bytes) == (1, 0)
    # the planner's split configuration: below 64 tiles, splits up to 128
    # workgroups (a power of two, each split at least 4 k tiles)
    c4 = by["c4"]
    for n, s in ((1, 8), (2, 4), (4, 1), (8, 1), (16, 1)):
        i = mk(c4.with_(n=n)).info()
        assert (i.ksplit, i.auto_ksplit) == (1, s), n
        assert (i.auto_workspace_bytes > 0) == (s > 1)
        assert i.auto_workspace_bytes == (i.grid_main * s * 256 * 256 * 4 if s > 1 else 0)
    # the generic family splits only when asked (c1: 25 tiles, still unsplit)
    for name in by:
        i = mk(by[name]).info()
        assert (i.auto_ksplit, i.auto_workspace_bytes) == (1, 0), name
    c4_1 = c4.with_(n=1)
    assert mk(c4_1).workspace_size() == mk(c4_1).info().auto_workspace_bytes > 0
    # ksplit 1: never split; per_class: no split configuration
    for kw in ({"ksplit": 1}, {"per_class": True}):
        i = mk(c4_1, **kw).info()
        assert (i.ksplit, i.auto_ksplit, i.auto_workspace_bytes, i.workspace_bytes) == (1, 1, 0, 0)
    # families without split-K refuse an explicit split
    with pytest.raises(cbd.CbdError) as e:
        mk(by["c5-s2"], ksplit=2)
    assert e.value.status == 2


def test_grouped_wide_rows_per_workgroup():
    """The 16x16x16-MFMA grouped kernel's row blocks: up to four workgroups
    per compute unit, half as many (twice the rows) where blocks would have
    four rows or fewer and again below three, rows split evenly over a
    column's blocks; the grid is images x row blocks x 256-byte group slices
    x column blocks."""
    from cbd_inputs import GROUPED_SWEEP
    want = {"gs-c8-14-s1": 4, "gs-c8-7-s1": 2, "gs-c16-7-s1": 4, "gs-c32-7-s1": 4, "gs-c32-14-s1": 7,
            "gs-c32-56-s1": 28, "gs-c16-56-s2": 14, "gs-c8-56-s1": 10, "gs-c32-28-s2": 14}
    seen = set()
    for p in GROUPED_SWEEP:
        if p.c // p.g < 8:
            continue
        pl = cbd.plan(p.n, p.g, p.c, p.k, p.hi, p.wi, p.y, p.x, (p.sh, p.sw), (p.ph, p.pw), (p.dh, p.dw),
                      p.layout, cbd.BF16)
        i = pl.info()
        subs = pl.subgemms()
        ph = max(s.pos_h for s in subs)
        pw = max(s.pos_w for s in subs)
        r = i.rows_per_wg
        blocks = -(-ph // r)
        assert -(-ph // blocks) == r, (p.name, r, ph)  # even blocks
        slices = p.c * 2 // 256
        assert i.grid_main == sum(p.n * -(-s.pos_h // r) * slices * -(-s.pos_w // i.cols_per_wg) for s in subs)
        if p.name in want:
            assert r == want[p.name], (p.name, r)
            seen.add(p.name)
    assert seen == set(want)
