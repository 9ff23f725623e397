"""The benchmark's whole-tensor parity check (bench.parity_of), on the CPU:
the oracle's own result, rounded to the output dtype, passes; a result off by
more than the stated tolerance, or nonzero where the oracle is exactly zero,
fails.  And the CPU baseline (bench.cpu_baseline) times one oracle call on the
whole problem and reports its thread count."""
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
    return p, dy, w, ref["dx64"].ravel(), np.array(out, dtype=np.float32).ravel()


def test_exact_result_passes():
    for layout in (NCHW, NHWC):
        for dtype in ("f32", "bf16"):
            p, _, _, ref, out = _case(layout, dtype, 2)
            r = bench.parity_of(p, out, ref)
            assert r["pass"] and r["zeros_ok"] and r["elements"] == ref.size, (layout, dtype, r)
            if dtype == "bf16":
                assert r["ulp_max"] <= 0.5 + 1e-9 and r["ulp_viol_floored"] == 0


def test_bf16_off_by_four_ulps_fails():
    p, _, _, ref, out = _case(NHWC, "bf16", 1)
    i = int(np.argmax(np.abs(ref)))
    bits = np.array([out[i]], dtype=np.float32).view(np.uint32)
    bits += np.uint32(4 << 16)  # four bf16 ulps further from zero
    out[i] = bits.view(np.float32)[0]
    r = bench.parity_of(p, out, ref)
    assert not r["pass"] and r["ulp_viol_floored"] >= 1


def test_nonzero_at_unreached_position_fails():
    # 1x1 filter, stride 2: odd rows and columns of dX are never reached.
    p, _, _, ref, out = _case(NCHW, "f32", 2)
    zero = np.flatnonzero(ref == 0.0)
    assert zero.size
    out[zero[0]] = 1e-30
    r = bench.parity_of(p, out, ref)
    assert not r["zeros_ok"] and not r["pass"]


def test_cpu_baseline_whole_problem():
    p, dy, w, ref, out = _case(NHWC, "bf16", 2)

    class Info:
        useful_flops = 2 * p.n * p.c * p.k * 5 * 5  # any positive count
    r = bench.cpu_baseline(p, dy, w, Info, dx_gpu=out.reshape(oracle.shapes(p)["dx"]))
    assert r["kind"] == "oracle" and r["cores"] == r["oracle_threads"] == oracle.num_threads() >= 1
    assert r["value"] > 0 and r["oracle_s"] >= 0 and "whole problem" in r["sample"]
    assert r["parity"]["pass"] and r["parity"]["elements"] == ref.size
