"""The benchmark's sampled parity check (bench.sample_parity), on the CPU:
the oracle's own result, rounded to the output dtype, passes; a result off by
more than the stated tolerance, or nonzero where the oracle is exactly zero,
fails."""
import numpy as np

import bench
import oracle
from cbd_inputs import draw, seed_for
from cbd_inputs.problems import Problem, NCHW, NHWC


def _case(layout, dtype, stride):
    p = Problem("t", 2, 1, 8, 8, 9, 10, 1, 1, stride, stride, 0, 0, 1, 1, layout, dtype, "n1", "n0.5", 0, 0)
    sh = oracle.shapes(p)
    dy = draw(p.dist_dy, seed_for(p, "dy"), sh["dy"], dtype)
    w = draw(p.dist_w, seed_for(p, "w"), sh["w"], dtype)
    ref = oracle.reference(p, dy, w)
    out = ref["ref_f32"] if dtype == "f32" else oracle.bf16_bits_to_f32(ref["ref_bf16_bits"]).reshape(sh["dx"])
    rng = np.random.default_rng(3)
    pts = np.stack([rng.integers(0, p.n, 400), rng.integers(0, p.c, 400),
                    rng.integers(0, p.hi, 400), rng.integers(0, p.wi, 400)], axis=1)
    return p, pts, oracle.bwd_data_at(p, dy, w, pts), np.array(out, dtype=np.float32)


def _at(p, a, pt):
    n, c, h, w = pt
    return (n, c, h, w) if p.layout == NCHW else (n, h, w, c)


def test_exact_result_passes():
    for layout in (NCHW, NHWC):
        for dtype in ("f32", "bf16"):
            p, pts, ref, out = _case(layout, dtype, 2)
            r = bench.sample_parity(p, pts, ref, out)
            assert r["pass"] and r["zeros_ok"], (layout, dtype, r)
            if dtype == "bf16":
                assert r["ulp_max"] <= 0.5 + 1e-9 and r["ulp_viol_floored"] == 0


def test_bf16_off_by_four_ulps_fails():
    p, pts, ref, out = _case(NHWC, "bf16", 1)
    i = int(np.argmax(np.abs(ref)))
    idx = _at(p, out, pts[i])
    v = np.float32(out[idx])
    bits = np.array([v], dtype=np.float32).view(np.uint32)
    bits += np.uint32(4 << 16)  # four bf16 ulps further from zero
    out[idx] = bits.view(np.float32)[0]
    r = bench.sample_parity(p, pts, ref, out)
    assert not r["pass"] and r["ulp_viol_floored"] >= 1


def test_nonzero_at_unreached_position_fails():
    # 1x1 filter, stride 2: odd rows and columns of dX are never reached.
    p, pts, ref, out = _case(NCHW, "f32", 2)
    zero = [i for i in range(len(ref)) if ref[i] == 0.0]
    assert zero
    out[_at(p, out, pts[zero[0]])] = 1e-30
    r = bench.sample_parity(p, pts, ref, out)
    assert not r["zeros_ok"] and not r["pass"]
