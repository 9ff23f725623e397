"""The workloads: twelve concrete backward-data problems.

Shapes and distributions:
  * fp32 stride-1 padding cases (N=32, C=K=32, Hi=Wi in {14, 15, 16},
    1x1 and 3x3, pad 1): rocMLIR PR #246 "Backward data", the driver command
    lines listed for the padding issue (gkcyx / ngchw / ngkhw, groupsize 1).
  * bf16 NHWC stride-(1,2) case (dY 16x1x256x2048, W 2048x1x2x2048 KYXC,
    dX 16x1x512x2048): fusilli issue #101, the BOO listing's import shapes.
  * A small fp32 case, an fp32 stride-2 pair (one with three of four dX
    phases unreached), and a ResNeXt-style grouped bf16 pair (32 groups of 4
    channels) standing in for the resnext configurations that MIOpen PR #272
    asks about but does not list.

Seeds: 1000*config + 10*variant + {1: dY, 2: W, 3: forward input x}.

No convolution arithmetic lives here; output sizes are derived by whoever
consumes a problem (the oracle and the planner each have their own).
"""
from __future__ import annotations

from dataclasses import dataclass, asdict, replace

NCHW = 0  # ngchw dX / ngkhw dY / gkcyx W (identical to NCHW/KCYX when G=1)
NHWC = 1  # NHWC dX / NHWK dY / KYXC W


@dataclass(frozen=True)
class Problem:
    name: str
    n: int
    g: int
    c: int  # total input (dX) channels
    k: int  # total output (dY) channels
    hi: int
    wi: int
    y: int
    x: int
    sh: int
    sw: int
    ph: int
    pw: int
    dh: int
    dw: int
    layout: int
    dtype: str  # 'f32' or 'bf16'
    dist_dy: str  # 'u', 'n<sigma>' or 'int'
    dist_w: str
    config: int
    variant: int

    def as_dict(self):
        return asdict(self)

    def with_(self, **kw) -> "Problem":
        return replace(self, **kw)

    def vector(self):
        """The 15-entry int64 problem vector used by both C ABIs' callers."""
        return [self.n, self.g, self.c, self.k, self.hi, self.wi, self.y, self.x,
                self.sh, self.sw, self.ph, self.pw, self.dh, self.dw, self.layout]


def seed_for(p: Problem, tensor: str) -> int:
    return 1000 * p.config + 10 * p.variant + {"dy": 1, "w": 2, "x": 3}[tensor]


def _mk(name, config, variant, n, g, c, k, hi, wi, y, x, s, pad, layout, dtype,
        ddy, dw_, dil=(1, 1)):
    sh, sw = s
    ph, pw = pad
    return Problem(name, n, g, c, k, hi, wi, y, x, sh, sw, ph, pw, dil[0], dil[1],
                   layout, dtype, ddy, dw_, config, variant)


PROBLEMS = [
    _mk("c1", 1, 0, 2, 1, 16, 16, 14, 14, 3, 3, (1, 1), (1, 1), NCHW, "f32", "u", "u"),
]
_v = 1
for _hw in (14, 15, 16):
    for _f in (1, 3):
        PROBLEMS.append(_mk(f"c2-{_hw}-{_f}", 2, _v, 32, 1, 32, 32, _hw, _hw, _f, _f,
                            (1, 1), (1, 1), NCHW, "f32", "u", "u"))
        _v += 1
PROBLEMS += [
    _mk("c3a", 3, 1, 32, 1, 64, 64, 28, 28, 3, 3, (2, 2), (1, 1), NCHW, "f32", "u", "u"),
    _mk("c3b", 3, 2, 32, 1, 64, 64, 28, 28, 1, 1, (2, 2), (0, 0), NCHW, "f32", "u", "u"),
    _mk("c4", 4, 0, 16, 1, 2048, 2048, 1, 512, 1, 2, (1, 2), (0, 0), NHWC, "bf16",
        "n1", "n0.02"),
    _mk("c5-s2", 5, 1, 64, 32, 128, 128, 56, 56, 3, 3, (2, 2), (1, 1), NHWC, "bf16",
        "n1", "n0.05"),
    _mk("c5-s1", 5, 2, 64, 32, 128, 128, 56, 56, 3, 3, (1, 1), (1, 1), NHWC, "bf16",
        "n1", "n0.05"),
]


# A ResNeXt-style grouped sweep (32 groups; 4, 8, 16 or 32 channels per
# group; 56, 28, 14 or 7 pixels square; 3x3, pad 1, stride 1 or 2; bf16
# NHWC, N=32): a synthetic second workload standing in for the resnext
# configurations that MIOpen PR #272 asks about without listing them.
# Config 6, variant = running index (seeds as above).
GROUPED_SWEEP = []
for _cg in (4, 8, 16, 32):
    for _hw in (56, 28, 14, 7):
        for _s in (1, 2):
            GROUPED_SWEEP.append(_mk(f"gs-c{_cg}-{_hw}-s{_s}", 6, len(GROUPED_SWEEP), 32, 32,
                                     32 * _cg, 32 * _cg, _hw, _hw, 3, 3, (_s, _s), (1, 1), NHWC,
                                     "bf16", "n1", "n0.05"))


def problem_by_name(name: str) -> Problem:
    for p in PROBLEMS + GROUPED_SWEEP:
        if p.name == name:
            return p
    raise KeyError(name)
