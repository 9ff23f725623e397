"""Shared helpers for the GPU parity tests: seeded operands, one GPU run
through the C ABI (with NaN sentinel and guard bands), and the acceptance
criteria.

Acceptance (per element, against the fp64 oracle on the same inputs):
  * fp32 output: relative L2 <= 1e-5 and max abs error <= 1e-4 * max |ref|.
  * bf16 output: relative L2 <= 8e-3 and every element within 2 bf16 ulps of
    the oracle rounded to fp32 and then to bf16.  Ulps are counted in the
    bf16 spacing at magnitude max(|ref|, 2^-10 * rms(ref)): below that floor
    the f32 accumulation error of a long dot product, not the kernel, sets
    the last bf16 bit.  The strict (unfloored) count is reported as well.
  * integer-valued inputs: bit-exact (every partial sum is an integer below
    2^24, exact in f32).
"""
from __future__ import annotations

import numpy as np
import torch

import dnn_conv2d_bwd_amd as cbd
import oracle
from cbd_inputs import draw, seed_for, small_ints

GUARD = 64  # elements of sentinel before and after dX


def operands(p, kind="dist"):
    """Seeded dY, W as float32 arrays holding dtype-representable values."""
    sh = oracle.shapes(p)
    if kind == "int":
        dy = small_ints(seed_for(p, "dy"), sh["dy"]).astype(np.float32)
        w = small_ints(seed_for(p, "w"), sh["w"]).astype(np.float32)
    else:
        dy = draw(p.dist_dy, seed_for(p, "dy"), sh["dy"], p.dtype)
        w = draw(p.dist_w, seed_for(p, "w"), sh["w"], p.dtype)
    return dy, w


def plan_for(p, force=cbd.KERNEL_AUTO, rows_per_wg=0, grouped_dot=False, cols_per_wg=0, ksplit=0,
             per_class=False, static_shape=0, merge_phases=0):
    dt = cbd.F32 if p.dtype == "f32" else cbd.BF16
    return cbd.plan(p.n, p.g, p.c, p.k, p.hi, p.wi, p.y, p.x, (p.sh, p.sw), (p.ph, p.pw),
                    (p.dh, p.dw), p.layout, dt, force_kernel=force, rows_per_wg=rows_per_wg,
                    grouped_dot=grouped_dot, cols_per_wg=cols_per_wg, ksplit=ksplit,
                    per_class=per_class, static_shape=static_shape, merge_phases=merge_phases)


def torch_dtype(p):
    return torch.float32 if p.dtype == "f32" else torch.bfloat16


def to_device(a, p):
    return torch.from_numpy(np.ascontiguousarray(a)).to(torch_dtype(p)).cuda()


class DeviceRun:
    """Allocates a sentinel-filled dX with guard bands and runs a plan."""

    def __init__(self, p, pl, dy_d, w_d, workspace=None):
        self.p, self.pl = p, pl
        self.ws = workspace
        self.shape = pl.shapes()["dx"]
        self.numel = int(np.prod(self.shape))
        self.buf = torch.full((self.numel + 2 * GUARD,), float("nan"), dtype=torch_dtype(p),
                              device="cuda")
        self.dx = self.buf[GUARD:GUARD + self.numel].view(self.shape)
        self.dy_d, self.w_d = dy_d, w_d

    def __call__(self, stream=None):
        cbd.run(self.pl, self.dy_d, self.w_d, self.dx, stream=stream, workspace=self.ws)
        return self

    def result_f32(self):
        torch.cuda.synchronize()
        return self.dx.float().cpu().numpy()

    def result_bits(self):
        torch.cuda.synchronize()
        if self.p.dtype == "f32":
            return self.dx.cpu().view(torch.int32).numpy().view(np.uint32)
        return self.dx.cpu().view(torch.int16).numpy().view(np.uint16)

    def guards_intact(self):
        torch.cuda.synchronize()
        g = torch.cat([self.buf[:GUARD], self.buf[-GUARD:]]).float()
        return bool(torch.isnan(g).all())


def bf16_order(bits):
    """Map bf16 bit patterns to integers that are monotonic in value (+0 = -0 = 0)."""
    b = bits.astype(np.int64)
    mag = b & 0x7FFF
    return np.where(b & 0x8000, -mag, mag)


def bf16_ulp(mag):
    """Spacing of bf16 numbers at magnitude mag (> 0, normal range)."""
    e = np.floor(np.log2(np.maximum(mag, 2.0 ** -126)))
    return np.exp2(e - 7)


def check_f32(got, ref64):
    err = got.astype(np.float64) - ref64
    ref_norm = np.linalg.norm(ref64)
    rel_l2 = np.linalg.norm(err) / max(ref_norm, 1e-300)
    max_abs = float(np.max(np.abs(err))) if err.size else 0.0
    scale = float(np.max(np.abs(ref64))) if ref64.size else 0.0
    ok = rel_l2 <= 1e-5 and max_abs <= 1e-4 * scale
    return ok, dict(rel_l2=float(rel_l2), max_abs=max_abs, max_ref=scale)


def check_bf16(got_bits, ref64):
    """got_bits: uint16 bf16 patterns; ref64: the fp64 oracle."""
    ref_bits = oracle.round_bf16_bits(oracle.round_f32(ref64))
    got = oracle.bf16_bits_to_f32(got_bits).astype(np.float64)
    ref_b = oracle.bf16_bits_to_f32(ref_bits).astype(np.float64)
    err = got - ref64
    rel_l2 = np.linalg.norm(err) / max(np.linalg.norm(ref64), 1e-300)
    strict = np.abs(bf16_order(got_bits.ravel()) - bf16_order(ref_bits.ravel()))
    rms = float(np.sqrt(np.mean(ref64 ** 2))) if ref64.size else 0.0
    floor = 2.0 ** -10 * rms
    mag = np.maximum(np.abs(ref_b.ravel()), floor)
    floored = np.abs(got.ravel() - ref_b.ravel()) > 2 * bf16_ulp(mag) * (1 + 1e-12)
    floored &= mag > 0
    info = dict(rel_l2=float(rel_l2), ulp_max=int(strict.max()) if strict.size else 0,
                ulp_viol_strict=int(np.count_nonzero(strict > 2)),
                ulp_viol_floored=int(np.count_nonzero(floored)))
    ok = rel_l2 <= 8e-3 and info["ulp_viol_floored"] == 0
    return ok, info


def check(p, gpu: DeviceRun, ref64):
    if p.dtype == "f32":
        return check_f32(gpu.result_f32().reshape(ref64.shape), ref64)
    return check_bf16(gpu.result_bits().reshape(ref64.shape), ref64)


def exact_expected_bits(p, ref64):
    """Bit patterns the GPU must produce when every partial sum is exact."""
    r32 = oracle.round_f32(ref64)
    if p.dtype == "f32":
        return r32.view(np.uint32).reshape(ref64.shape)
    return oracle.round_bf16_bits(r32).reshape(ref64.shape)
