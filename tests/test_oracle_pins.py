"""Pins for the CPU oracle: checks against things other than the oracle itself.

Each test fixes the oracle to something the pages or mathematics determine:
  * a library routine: torch's CPU float64 convolution backward
    (aten.convolution_backward, the call in the torch-IR listing of fusilli
    issue #101) and forward (conv2d);
  * the adjoint identity <conv_fwd(x, W), dY> = <x, conv_bwd_data(dY, W)>;
  * impulse responses and a pure-Python scatter form on tiny inputs;
  * finite differences of L(x) = <conv_fwd(x, W), dY>;
  * the zero-insertion + flipped-filter form and its printed geometry
    (16x1x513x2048 zero tensor, insert offset 1, stride 2 in the BOO listing);
  * exact zeros at positions no tap reaches (3/4 of dX for 1x1 stride 2);
  * GEMM special cases, group block-diagonality, layout invariance,
    linearity;
  * a negative control: the unflipped contraction of the Fusilli listing
    must fail the pins;
  * the rounding helpers against torch / numpy conversions.
"""
import json
import os
import random

import numpy as np
import pytest
import torch

import oracle
from cbd_inputs import PROBLEMS, draw, problem_by_name, small_ints, uniform
from cbd_inputs.problems import NCHW, NHWC, Problem

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def mk(n=1, g=1, c=2, k=2, hi=5, wi=5, y=3, x=3, sh=1, sw=1, ph=0, pw=0, dh=1, dw=1,
       layout=NCHW, dtype="f32"):
    return Problem("tiny", n, g, c, k, hi, wi, y, x, sh, sw, ph, pw, dh, dw, layout,
                   dtype, "u", "u", 0, 0)


def out_size(i, p, d, t, s):
    # written independently of the oracle: count window starts
    return len([o for o in range(i + 2 * p) if o * s + d * (t - 1) < i + 2 * p])


def random_problems(count, seed, max_hw=9, layouts=(NCHW, NHWC)):
    rng = random.Random(seed)
    out = []
    while len(out) < count:
        g = rng.randint(1, 3)
        p = mk(n=rng.randint(1, 2), g=g, c=g * rng.randint(1, 3), k=g * rng.randint(1, 3),
               hi=rng.randint(1, max_hw), wi=rng.randint(1, max_hw), y=rng.randint(1, 4),
               x=rng.randint(1, 4), sh=rng.randint(1, 3), sw=rng.randint(1, 3),
               ph=rng.randint(0, 2), pw=rng.randint(0, 2), dh=rng.randint(1, 3),
               dw=rng.randint(1, 3), layout=rng.choice(layouts))
        if out_size(p.hi, p.ph, p.dh, p.y, p.sh) < 1 or out_size(p.wi, p.pw, p.dw, p.x, p.sw) < 1:
            continue
        out.append(p)
    return out


def operands(p, kind, seed):
    sh = oracle.shapes(p)
    f = small_ints if kind == "int" else uniform
    return f(seed + 1, sh["dy"]), f(seed + 2, sh["w"]), f(seed + 3, sh["dx"])


def to_nchw(p, a, which):
    """Logical NCHW / KCYX view of a layout-ordered array (for torch)."""
    if p.layout == NCHW:
        return a
    return np.transpose(a, (0, 3, 1, 2)) if which != "w" else np.transpose(a, (0, 3, 1, 2))


def from_nchw(p, a):
    return a if p.layout == NCHW else np.transpose(a, (0, 2, 3, 1))


def torch_bwd(p, dy, w):
    dy_t = torch.from_numpy(np.ascontiguousarray(to_nchw(p, dy, "dy")))
    w_t = torch.from_numpy(np.ascontiguousarray(to_nchw(p, w, "w")))
    x_shape = [p.n, p.c, p.hi, p.wi]
    dx, _, _ = torch.ops.aten.convolution_backward(
        dy_t, torch.zeros(x_shape, dtype=torch.float64), w_t, None, [p.sh, p.sw],
        [p.ph, p.pw], [p.dh, p.dw], False, [0, 0], p.g, [True, False, False])
    return from_nchw(p, dx.numpy())


def torch_fwd(p, x, w):
    x_t = torch.from_numpy(np.ascontiguousarray(to_nchw(p, x, "x")))
    w_t = torch.from_numpy(np.ascontiguousarray(to_nchw(p, w, "w")))
    y = torch.nn.functional.conv2d(x_t, w_t, None, (p.sh, p.sw), (p.ph, p.pw),
                                   (p.dh, p.dw), p.g)
    return from_nchw(p, y.numpy())


def scatter_bwd(p, dy, w):
    """Pure-Python scatter form: every dY element, through every tap, adds to
    the input position the forward convolution read it from."""
    cg, kg = p.c // p.g, p.k // p.g
    dy4 = to_nchw(p, dy, "dy")
    w4 = to_nchw(p, w, "w")
    dx = np.zeros((p.n, p.c, p.hi, p.wi))
    _, _, ho_n, wo_n = dy4.shape
    for n in range(p.n):
        for gk in range(p.k):
            g = gk // kg
            for ho in range(ho_n):
                for wo in range(wo_n):
                    d = dy4[n, gk, ho, wo]
                    for c in range(cg):
                        for ty in range(p.y):
                            h = ho * p.sh + ty * p.dh - p.ph
                            if not 0 <= h < p.hi:
                                continue
                            for tx in range(p.x):
                                ww = wo * p.sw + tx * p.dw - p.pw
                                if 0 <= ww < p.wi:
                                    dx[n, g * cg + c, h, ww] += d * w4[gk, c, ty, tx]
    return from_nchw(p, dx)


# ----------------------------------------------------------------- shapes ---

def test_output_size_matches_independent_count():
    for p in random_problems(200, 7):
        assert oracle.out_hw(p) == (out_size(p.hi, p.ph, p.dh, p.y, p.sh),
                                    out_size(p.wi, p.pw, p.dw, p.x, p.sw))


def test_boo_listing_geometry():
    """Printed shapes of fusilli #101: dY 16x1x256x2048 from dX 16x1x512x2048
    with a 1x2 filter at stride (1,2); zero-inserted operand 513 wide with
    dY at offset 1, stride 2."""
    gold = json.load(open(os.path.join(GOLDEN, "fusilli101_boo_geometry.json")))
    n, hi, wi, c = gold["dx_shape"]
    k, y, x, cw = gold["w_shape"]
    assert cw == c
    p = mk(n=n, c=c, k=k, hi=hi, wi=wi, y=y, x=x, sh=gold["stride"][0], sw=gold["stride"][1],
           ph=gold["padding"][0], pw=gold["padding"][1], dh=gold["dilation"][0],
           dw=gold["dilation"][1], g=gold["groups"], layout=NHWC)
    ho, wo = oracle.out_hw(p)
    assert [n, ho, wo, k] == gold["dy_shape"]
    # The zero-insertion geometry is independent of channel counts: shrink them.
    small = p.with_(n=1, c=4, k=4)
    dy = uniform(11, oracle.shapes(small)["dy"])
    w = uniform(12, oracle.shapes(small)["w"])
    dx_zi, (hz, wz, lh, lw) = oracle.bwd_data_zero_insert(small, dy, w)
    zshape = gold["zero_inserted_shape"]
    assert (hz, wz) == (zshape[1], zshape[2])
    assert (lh, lw) == (gold["insert_offsets"][1], gold["insert_offsets"][2])
    assert (small.sh, small.sw) == (gold["insert_strides"][1], gold["insert_strides"][2])
    np.testing.assert_allclose(dx_zi, oracle.bwd_data(small, dy, w), rtol=1e-13, atol=1e-13)


def test_driver_configs_are_the_stride1_workload():
    """The six tested driver lines map onto valid problems whose dY extents
    follow the padded-window count (1x1 pad 1 grows the image by 2)."""
    gold = json.load(open(os.path.join(GOLDEN, "rocmlir246_driver_configs.json")))
    for cfg in gold["configs"]:
        p = mk(n=cfg["batchsize"], c=cfg["in_channels"], k=cfg["out_channels"],
               hi=cfg["in_h"], wi=cfg["in_w"], y=cfg["fil_h"], x=cfg["fil_w"],
               sh=cfg["conv_stride"][0], sw=cfg["conv_stride"][1], ph=cfg["padding"][0],
               pw=cfg["padding"][1], dh=cfg["dilation"][0], dw=cfg["dilation"][1],
               g=cfg["groupsize"])
        ho, wo = oracle.out_hw(p)
        assert ho == cfg["in_h"] + 2 - cfg["fil_h"] + 1
        assert wo == cfg["in_w"] + 2 - cfg["fil_w"] + 1
    names = {q.name for q in PROBLEMS if q.config == 2}
    for cfg in gold["configs"][:4]:
        assert f"c2-{cfg['in_h']}-{cfg['fil_h']}" in names


# --------------------------------------------- library routine (torch f64) ---

@pytest.mark.parametrize("kind", ["int", "float"])
def test_matches_torch_convolution_backward(kind):
    for i, p in enumerate(random_problems(60, 101 if kind == "int" else 202)):
        dy, w, _ = operands(p, kind, 1000 * i)
        got = oracle.bwd_data(p, dy, w)
        ref = torch_bwd(p, dy, w)
        if kind == "int":
            assert np.array_equal(got, ref), p
        else:
            np.testing.assert_allclose(got, ref, rtol=1e-12, atol=1e-12, err_msg=str(p))


def test_forward_matches_torch_conv2d():
    for i, p in enumerate(random_problems(60, 303)):
        _, w, x = operands(p, "int", 77 * i)
        assert np.array_equal(oracle.conv_fwd(p, x, w), torch_fwd(p, x, w)), p


@pytest.mark.parametrize("name", [q.name for q in PROBLEMS if q.config in (1, 2, 3)])
def test_workload_matches_torch(name):
    p = problem_by_name(name)
    sh = oracle.shapes(p)
    dy = draw(p.dist_dy, 1 + 17 * p.variant, sh["dy"], p.dtype)
    w = draw(p.dist_w, 2 + 17 * p.variant, sh["w"], p.dtype)
    np.testing.assert_allclose(oracle.bwd_data(p, dy, w), torch_bwd(p, dy.astype(np.float64),
                               w.astype(np.float64)), rtol=1e-11, atol=1e-11)


# ------------------------------------------------------------- adjoint -------

def test_adjoint_identity_exact_on_integers():
    for i, p in enumerate(random_problems(150, 404)):
        dy, w, x = operands(p, "int", 31 * i)
        lhs = np.dot(oracle.conv_fwd(p, x, w).ravel(), dy.ravel())
        rhs = np.dot(x.ravel(), oracle.bwd_data(p, dy, w).ravel())
        assert lhs == rhs, p


def test_adjoint_identity_random():
    for i, p in enumerate(random_problems(60, 505)):
        dy, w, x = operands(p, "float", 37 * i)
        fx = oracle.conv_fwd(p, x, w)
        bx = oracle.bwd_data(p, dy, w)
        scale = np.abs(fx).ravel() @ np.abs(dy).ravel() + np.abs(x).ravel() @ np.abs(bx).ravel()
        assert abs(fx.ravel() @ dy.ravel() - x.ravel() @ bx.ravel()) <= 1e-12 * max(scale, 1), p


@pytest.mark.parametrize("name", ["c3a", "c3b", "c5-s2"])
def test_adjoint_identity_on_workload_shapes(name):
    p = problem_by_name(name).with_(n=2)
    dy, w, x = operands(p, "int", 9000 + p.config)
    lhs = np.dot(oracle.conv_fwd(p, x, w).ravel(), dy.ravel())
    rhs = np.dot(x.ravel(), oracle.bwd_data(p, dy, w).ravel())
    assert lhs == rhs


# ---------------------------------------------- impulses and brute force ----

def test_dy_impulse_scatters_the_filter():
    rng = random.Random(5)
    for p in random_problems(40, 606):
        sh = oracle.shapes(p)
        _, w, _ = operands(p, "int", 3)
        dy = np.zeros(sh["dy"])
        n = rng.randrange(p.n)
        kk = rng.randrange(p.k)
        ho_n, wo_n = oracle.out_hw(p)
        ho, wo = rng.randrange(ho_n), rng.randrange(wo_n)
        idx = (n, kk, ho, wo) if p.layout == NCHW else (n, ho, wo, kk)
        dy[idx] = 1.0
        got = to_nchw(p, oracle.bwd_data(p, dy, w), "dx")
        exp = np.zeros((p.n, p.c, p.hi, p.wi))
        w4 = to_nchw(p, w, "w")
        cg, kg = p.c // p.g, p.k // p.g
        g = kk // kg
        for c in range(cg):
            for ty in range(p.y):
                for tx in range(p.x):
                    h, ww = ho * p.sh + ty * p.dh - p.ph, wo * p.sw + tx * p.dw - p.pw
                    if 0 <= h < p.hi and 0 <= ww < p.wi:
                        exp[n, g * cg + c, h, ww] += w4[kk, c, ty, tx]
        assert np.array_equal(got, exp), p


def test_matches_pure_python_scatter():
    for i, p in enumerate(random_problems(30, 707)):
        dy, w, _ = operands(p, "int", 13 * i)
        assert np.array_equal(oracle.bwd_data(p, dy, w), scatter_bwd(p, dy, w)), p


def test_sampled_entry_point_matches_full():
    for i, p in enumerate(random_problems(30, 808)):
        dy, w, _ = operands(p, "float", 19 * i)
        full = oracle.bwd_data(p, dy, w)
        full4 = to_nchw(p, full, "dx")
        rng = np.random.default_rng(i)
        pts = np.stack([rng.integers(0, p.n, 50), rng.integers(0, p.c, 50),
                        rng.integers(0, p.hi, 50), rng.integers(0, p.wi, 50)], axis=1)
        got = oracle.bwd_data_at(p, dy, w, pts)
        exp = full4[pts[:, 0], pts[:, 1], pts[:, 2], pts[:, 3]]
        np.testing.assert_allclose(got, exp, rtol=1e-14, atol=1e-14)


# --------------------------------------------------- finite differences ------

def test_finite_differences_exact():
    """L(x) = <fwd(x, W), dY> is linear in x, so the central difference with
    unit step equals dL/dx_i = dX_i exactly on integer data."""
    for i, p in enumerate(random_problems(12, 909, max_hw=6)):
        dy, w, x = operands(p, "int", 23 * i)
        dx = oracle.bwd_data(p, dy, w).ravel()
        xf = x.ravel().copy()
        for j in range(xf.size):
            e = np.zeros_like(xf)
            e[j] = 1.0
            lp = oracle.conv_fwd(p, (xf + e).reshape(x.shape), w).ravel() @ dy.ravel()
            lm = oracle.conv_fwd(p, (xf - e).reshape(x.shape), w).ravel() @ dy.ravel()
            assert (lp - lm) / 2 == dx[j], (p, j)


# --------------------------------------------------- zero-insertion form ----

def test_zero_insertion_cross_form_exact():
    for i, p in enumerate(random_problems(80, 1001)):
        dy, w, _ = operands(p, "int", 29 * i)
        zi, _ = oracle.bwd_data_zero_insert(p, dy, w)
        assert np.array_equal(zi, oracle.bwd_data(p, dy, w)), p


def test_stride1_is_full_correlation_with_flipped_transposed_filter():
    """At stride 1 the result is a full correlation of dY against the filter
    flipped in both spatial axes with the C and K roles exchanged (scipy)."""
    from scipy.signal import correlate2d

    for i, p in enumerate(random_problems(40, 1102, layouts=(NCHW,))):
        p = p.with_(sh=1, sw=1, dh=1, dw=1)
        if p.hi + 2 * p.ph < p.y or p.wi + 2 * p.pw < p.x:
            continue
        dy, w, _ = operands(p, "int", 41 * i)
        cg, kg = p.c // p.g, p.k // p.g
        exp = np.zeros((p.n, p.c, p.hi, p.wi))
        for n in range(p.n):
            for g in range(p.g):
                for c in range(cg):
                    acc = 0
                    for k in range(kg):
                        flipped = w[g * kg + k, c, ::-1, ::-1]
                        full = correlate2d(dy[n, g * kg + k], flipped, mode="full")
                        acc = acc + full
                    # the full correlation has Ho+Y-1 = Hi+2P rows; row hi+P is dX row hi
                    oy, ox = p.ph, p.pw
                    exp[n, g * cg + c] = acc[oy:oy + p.hi, ox:ox + p.wi]
        assert np.array_equal(oracle.bwd_data(p, dy, w), exp), p


def unflipped_form(p, dy, w):
    """Negative control: the contraction of the Fusilli listing in fusilli
    issue #101 -- the zero-inserted dY correlated with the filter *without*
    the spatial flip (questioned in that thread).  Not the oracle."""
    assert p.layout == NCHW and p.g == 1 and p.dh == 1 and p.dw == 1
    ho_n, wo_n = oracle.out_hw(p)
    lh, lw = p.y - 1 - p.ph, p.x - 1 - p.pw
    z = np.zeros((p.n, p.k, p.hi + p.y - 1, p.wi + p.x - 1))
    for ho in range(ho_n):
        for wo in range(wo_n):
            hz, wz = lh + ho * p.sh, lw + wo * p.sw
            if 0 <= hz < z.shape[2] and 0 <= wz < z.shape[3]:
                z[:, :, hz, wz] = dy[:, :, ho, wo]
    dx = np.zeros((p.n, p.c, p.hi, p.wi))
    for ty in range(p.y):
        for tx in range(p.x):
            dx += np.einsum("nkhw,kc->nchw", z[:, :, ty:ty + p.hi, tx:tx + p.wi], w[:, :, ty, tx])
    return dx


def test_negative_control_unflipped_filter_is_caught():
    p = mk(n=2, c=3, k=4, hi=8, wi=9, y=2, x=3, sh=1, sw=2, ph=0, pw=1)
    dy, w, x = operands(p, "int", 4242)
    bad = unflipped_form(p, dy, w)
    good = oracle.bwd_data(p, dy, w)
    assert not np.array_equal(bad, good)
    # ... and the adjoint identity exposes it
    lhs = np.dot(oracle.conv_fwd(p, x, w).ravel(), dy.ravel())
    assert lhs == np.dot(x.ravel(), good.ravel())
    assert lhs != np.dot(x.ravel(), bad.ravel())
    # with a filter symmetric under the flip the two coincide (sanity of the control)
    wsym = w + w[:, :, ::-1, ::-1]
    assert np.array_equal(unflipped_form(p, dy, wsym), oracle.bwd_data(p, dy, wsym))


# -------------------------------------------------------------- zeros -------

def reachable(i, pad, dil, taps, stride, out_n):
    return any(0 <= (i + pad - t * dil) // stride < out_n and (i + pad - t * dil) % stride == 0
               and i + pad - t * dil >= 0 for t in range(taps))


def test_exact_zeros_where_no_tap_reaches():
    for i, p in enumerate(random_problems(80, 1203)):
        dy, w, _ = operands(p, "float", 53 * i)
        dx = to_nchw(p, oracle.bwd_data(p, dy, w), "dx")
        ho_n, wo_n = oracle.out_hw(p)
        for h in range(p.hi):
            for ww in range(p.wi):
                if not (reachable(h, p.ph, p.dh, p.y, p.sh, ho_n)
                        and reachable(ww, p.pw, p.dw, p.x, p.sw, wo_n)):
                    assert np.all(dx[:, :, h, ww] == 0.0), (p, h, ww)


def test_c3b_three_quarters_zero():
    p = problem_by_name("c3b")
    sh = oracle.shapes(p)
    dx = oracle.bwd_data(p, uniform(1, sh["dy"]), uniform(2, sh["w"]))
    assert np.all(dx[:, :, 1::2, :] == 0) and np.all(dx[:, :, :, 1::2] == 0)
    assert np.count_nonzero(dx[:, :, 0::2, 0::2] == 0) == 0
    assert np.count_nonzero(dx == 0) == dx.size * 3 // 4


# ------------------------------------------------------- GEMM reductions ----

def test_c4_shape_is_two_gemms():
    """1x2 filter at stride (1,2), pad 0 (the fusilli #101 problem, channels
    reduced): dX[:, 0, r::2, :] = dY[:, 0, :, :] @ W[:, 0, r, :] for r = 0, 1."""
    p = problem_by_name("c4").with_(n=2, wi=32, c=96, k=80)
    sh = oracle.shapes(p)
    dy, w = uniform(1, sh["dy"]), uniform(2, sh["w"])
    dx = oracle.bwd_data(p, dy, w)
    for r in range(2):
        exp = dy[:, 0].reshape(-1, p.k) @ w[:, 0, r, :]
        np.testing.assert_allclose(dx[:, 0, r::2, :].reshape(-1, p.c), exp, rtol=1e-13, atol=1e-13)


def test_c3b_is_one_gemm_on_even_phases():
    p = problem_by_name("c3b").with_(n=3)
    sh = oracle.shapes(p)
    dy, w = small_ints(1, sh["dy"]), small_ints(2, sh["w"])
    dx = oracle.bwd_data(p, dy, w)
    exp = np.einsum("nkhw,kc->nchw", dy, w[:, :, 0, 0])
    assert np.array_equal(dx[:, :, 0::2, 0::2], exp)


def test_c2_1x1_pad1_is_gemm_on_cropped_dy():
    p = problem_by_name("c2-15-1").with_(n=3)
    sh = oracle.shapes(p)
    dy, w = small_ints(1, sh["dy"]), small_ints(2, sh["w"])
    exp = np.einsum("nkhw,kc->nchw", dy[:, :, 1:-1, 1:-1], w[:, :, 0, 0])
    assert np.array_equal(oracle.bwd_data(p, dy, w), exp)


# -------------------------------------------- groups, layout, linearity -----

def test_groups_are_block_diagonal():
    for i, p in enumerate(random_problems(40, 1304, layouts=(NCHW,))):
        if p.g == 1:
            continue
        dy, w, _ = operands(p, "int", 61 * i)
        dx = oracle.bwd_data(p, dy, w)
        cg, kg = p.c // p.g, p.k // p.g
        for g in range(p.g):
            q = p.with_(g=1, c=cg, k=kg)
            sub = oracle.bwd_data(q, dy[:, g * kg:(g + 1) * kg], w[g * kg:(g + 1) * kg])
            assert np.array_equal(dx[:, g * cg:(g + 1) * cg], sub), p


def test_layout_invariance():
    for i, p in enumerate(random_problems(40, 1405, layouts=(NCHW,))):
        dy, w, _ = operands(p, "float", 67 * i)
        q = p.with_(layout=NHWC)
        dx_a = oracle.bwd_data(p, dy, w)
        dx_b = oracle.bwd_data(q, np.transpose(dy, (0, 2, 3, 1)), np.transpose(w, (0, 2, 3, 1)))
        assert np.array_equal(np.transpose(dx_b, (0, 3, 1, 2)), dx_a), p


def test_linearity_exact():
    for i, p in enumerate(random_problems(40, 1506)):
        dy1, w, _ = operands(p, "int", 71 * i)
        dy2, _, _ = operands(p, "int", 71 * i + 5)
        lhs = oracle.bwd_data(p, 3 * dy1 - 2 * dy2, w)
        rhs = 3 * oracle.bwd_data(p, dy1, w) - 2 * oracle.bwd_data(p, dy2, w)
        assert np.array_equal(lhs, rhs), p


# ------------------------------------------------------------- rounding -----

def test_round_bf16_matches_torch():
    rng = np.random.default_rng(3)
    bits = rng.integers(0, 2 ** 32, 200000, dtype=np.uint64).astype(np.uint32)
    vals = bits.view(np.float32)
    vals = vals[np.isfinite(vals)]
    # explicit halfway and near-halfway patterns, both parities
    base = rng.integers(0, 2 ** 16, 5000, dtype=np.uint64).astype(np.uint32) << np.uint32(16)
    for low in (0x8000, 0x7FFF, 0x8001, 0x0001, 0xFFFF):
        extra = (base | np.uint32(low)).view(np.float32)
        vals = np.concatenate([vals, extra[np.isfinite(extra)]])
    vals = np.concatenate([vals, np.array([0.0, -0.0, 1.0, -1.0, 3.4e38, 1e-40, -1e-45],
                                          dtype=np.float32)])
    want = torch.from_numpy(vals).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(oracle.round_bf16_bits(vals), want)


def test_round_f32_matches_numpy():
    rng = np.random.default_rng(4)
    v = rng.standard_normal(100000) * 10.0 ** rng.integers(-30, 30, 100000)
    assert np.array_equal(oracle.round_f32(v), v.astype(np.float32))
