"""CPU oracle for 2-D convolution backward-data -- TEST INFRASTRUCTURE ONLY.

Only the test suite, `__graft_entry__.smoke()` and the `cpu_baseline` leg of
`bench.py` may import this package.  The HIP library never includes, links
or calls it, and this package never touches the HIP library.

Thin ctypes wrapper over `cbd_oracle.c` (plain C, fp64 accumulation).  A
problem is anything with the attributes n, g, c, k, hi, wi, y, x, sh, sw,
ph, pw, dh, dw, layout (the workload dataclass in `cbd_inputs.problems`
qualifies).  Operands are flat or shaped numpy arrays in the memory order of
the layout; they are widened to float64 before the call.

Every function is pinned in tests/test_oracle_pins.py against a library
routine (torch's CPU float64 convolution), the adjoint identity, impulse
responses, finite differences, the zero-insertion form of fusilli issue
#101's BOO listing, exact zeros, and GEMM special cases; none is
"parity unpinned".
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "cbd_oracle.c")
_SO = os.path.join(_HERE, "libcbd_oracle.so")
_lib = None

_I64P = ctypes.POINTER(ctypes.c_int64)
_F64P = ctypes.POINTER(ctypes.c_double)


def build() -> str:
    """Compile the oracle with gcc (no fast-math, no FMA contraction)."""
    tmp = _SO + ".tmp"
    subprocess.check_call(["gcc", "-O3", "-std=c11", "-fopenmp", "-fPIC", "-shared",
                           "-ffp-contract=off", "-fno-fast-math", "-Wall",
                           "-o", tmp, _SRC])
    os.replace(tmp, _SO)
    return _SO


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(_SO):
            build()
        L = ctypes.CDLL(_SO)
        for name in ("cbd_oracle_conv_fwd", "cbd_oracle_bwd_data"):
            getattr(L, name).argtypes = [_I64P, _F64P, _F64P, _F64P]
            getattr(L, name).restype = ctypes.c_int
        L.cbd_oracle_bwd_data_at.argtypes = [_I64P, _F64P, _F64P, ctypes.c_int64,
                                             _I64P, _F64P]
        L.cbd_oracle_bwd_data_at.restype = ctypes.c_int
        L.cbd_oracle_bwd_data_zero_insert.argtypes = [_I64P, _F64P, _F64P, _F64P, _I64P]
        L.cbd_oracle_bwd_data_zero_insert.restype = ctypes.c_int
        L.cbd_oracle_out_hw.argtypes = [_I64P, _I64P]
        L.cbd_oracle_out_hw.restype = ctypes.c_int
        L.cbd_oracle_round_f32.argtypes = [ctypes.c_int64, _F64P, ctypes.c_void_p]
        L.cbd_oracle_round_f32.restype = None
        L.cbd_oracle_round_bf16.argtypes = [ctypes.c_int64, ctypes.c_void_p, ctypes.c_void_p]
        L.cbd_oracle_round_bf16.restype = None
        L.cbd_oracle_num_threads.restype = ctypes.c_int
        _lib = L
    return _lib


def _pvec(p) -> np.ndarray:
    return np.array([p.n, p.g, p.c, p.k, p.hi, p.wi, p.y, p.x, p.sh, p.sw, p.ph,
                     p.pw, p.dh, p.dw, p.layout], dtype=np.int64)


def _ptr(a, t):
    return a.ctypes.data_as(t)


def _f64(a) -> np.ndarray:
    return np.ascontiguousarray(a, dtype=np.float64).reshape(-1)


def out_hw(p):
    """(Ho, Wo) of the forward convolution that the problem describes."""
    hw = np.zeros(2, dtype=np.int64)
    if lib().cbd_oracle_out_hw(_ptr(_pvec(p), _I64P), _ptr(hw, _I64P)):
        raise ValueError("invalid problem")
    return int(hw[0]), int(hw[1])


def shapes(p):
    """Memory-order shapes of dX (= forward x), dY and W for the layout."""
    ho, wo = out_hw(p)
    cg = p.c // p.g
    if p.layout == 0:
        return dict(dx=(p.n, p.c, p.hi, p.wi), dy=(p.n, p.k, ho, wo),
                    w=(p.k, cg, p.y, p.x))
    return dict(dx=(p.n, p.hi, p.wi, p.c), dy=(p.n, ho, wo, p.k),
                w=(p.k, p.y, p.x, cg))


def conv_fwd(p, x, w) -> np.ndarray:
    sh = shapes(p)
    out = np.zeros(int(np.prod(sh["dy"])), dtype=np.float64)
    xd, wd = _f64(x), _f64(w)
    if lib().cbd_oracle_conv_fwd(_ptr(_pvec(p), _I64P), _ptr(xd, _F64P), _ptr(wd, _F64P),
                                 _ptr(out, _F64P)):
        raise ValueError("invalid problem")
    return out.reshape(sh["dy"])


def bwd_data(p, dy, w) -> np.ndarray:
    """dX in float64 (memory order of the layout)."""
    sh = shapes(p)
    out = np.zeros(int(np.prod(sh["dx"])), dtype=np.float64)
    dyd, wd = _f64(dy), _f64(w)
    if lib().cbd_oracle_bwd_data(_ptr(_pvec(p), _I64P), _ptr(dyd, _F64P), _ptr(wd, _F64P),
                                 _ptr(out, _F64P)):
        raise ValueError("invalid problem")
    return out.reshape(sh["dx"])


def bwd_data_at(p, dy, w, pts) -> np.ndarray:
    """dX at positions pts = int array (npts, 4) of (n, channel, hi, wi)."""
    pts = np.ascontiguousarray(pts, dtype=np.int64).reshape(-1, 4)
    out = np.zeros(pts.shape[0], dtype=np.float64)
    dyd, wd = _f64(dy), _f64(w)
    if lib().cbd_oracle_bwd_data_at(_ptr(_pvec(p), _I64P), _ptr(dyd, _F64P),
                                    _ptr(wd, _F64P), pts.shape[0], _ptr(pts, _I64P),
                                    _ptr(out, _F64P)):
        raise ValueError("invalid problem")
    return out


def bwd_data_zero_insert(p, dy, w):
    """Cross form (zero-inserted dY, flipped filter).  Returns (dX, geometry)
    with geometry = (Hz, Wz, Lh, Lw): the zero-inserted extent and the
    offset of the first dY row / column in it."""
    sh = shapes(p)
    out = np.zeros(int(np.prod(sh["dx"])), dtype=np.float64)
    geom = np.zeros(4, dtype=np.int64)
    dyd, wd = _f64(dy), _f64(w)
    rc = lib().cbd_oracle_bwd_data_zero_insert(_ptr(_pvec(p), _I64P), _ptr(dyd, _F64P),
                                               _ptr(wd, _F64P), _ptr(out, _F64P),
                                               _ptr(geom, _I64P))
    if rc:
        raise ValueError("invalid problem" if rc == -1 else "out of memory")
    return out.reshape(sh["dx"]), tuple(int(v) for v in geom)


def round_f32(a) -> np.ndarray:
    a = _f64(a)
    out = np.empty(a.size, dtype=np.float32)
    lib().cbd_oracle_round_f32(a.size, _ptr(a, _F64P), out.ctypes.data)
    return out


def round_bf16_bits(a32) -> np.ndarray:
    a32 = np.ascontiguousarray(a32, dtype=np.float32).reshape(-1)
    out = np.empty(a32.size, dtype=np.uint16)
    lib().cbd_oracle_round_bf16(a32.size, a32.ctypes.data, out.ctypes.data)
    return out


def bf16_bits_to_f32(bits) -> np.ndarray:
    b = np.ascontiguousarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    return b.view(np.float32)


def reference(p, dy, w):
    """dict(dx64, ref_f32, ref_bf16_bits): the fp64 result, rounded once to
    fp32, and that fp32 value rounded to bf16 (the fp32-accumulated result
    rounded to bf16)."""
    dx64 = bwd_data(p, dy, w)
    r32 = round_f32(dx64).reshape(dx64.shape)
    return dict(dx64=dx64, ref_f32=r32, ref_bf16_bits=round_bf16_bits(r32).reshape(dx64.shape))


def num_threads() -> int:
    return int(lib().cbd_oracle_num_threads())
