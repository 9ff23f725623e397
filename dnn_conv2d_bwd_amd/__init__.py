"""dnn_conv2d_bwd_amd -- 2-D convolution backward-data for MI355X (gfx950).

Thin Python binding over the C ABI in include/cbd.h (libcbd.so, built
in-tree by `python -m dnn_conv2d_bwd_amd.build`).  This module only
marshals arguments; every step of the computation runs in the library's HIP
kernels.  torch supplies device memory and streams.

    import dnn_conv2d_bwd_amd as cbd
    p = cbd.plan(n=16, g=1, c=2048, k=2048, hi=1, wi=512, y=1, x=2,
                 stride=(1, 2), pad=(0, 0), dil=(1, 1), layout="nhwc", dtype="bf16")
    cbd.run(p, dy, w, dx)                 # torch tensors on the GPU, dx overwritten

`conv2d_bwd_data(dy, w, input_size, stride, padding, dilation, groups,
layout)` mirrors torch's convolution_backward with output_mask
[True, False, False] (the call in the torch-IR listing of fusilli issue #101)
and allocates dX.

If libcbd.so is missing, importing this module raises ImportError: there is
no fallback path.
"""
from __future__ import annotations

import ctypes
import os

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libcbd.so")

NCHW, NHWC = 0, 1
F32, BF16 = 0, 1
KERNEL_AUTO, KERNEL_GENERIC, KERNEL_NHWC_BF16, KERNEL_GROUPED, KERNEL_NCHW_ROWS = -1, 0, 1, 2, 3
KERNEL_NAMES = {0: "generic", 1: "nhwc_bf16", 2: "grouped", 3: "nchw_rows"}

STATUS = {0: "CBD_OK", 1: "CBD_ERR_INVALID_ARG", 2: "CBD_ERR_UNSUPPORTED", 3: "CBD_ERR_HIP",
          4: "CBD_ERR_NO_MEMORY"}

# Every symbol include/cbd.h declares.
EXPORTS = ("cbd_plan", "cbd_plan_ex", "cbd_run", "cbd_run_ws", "cbd_run_noalloc", "cbd_plan_workspace_size",
           "cbd_plan_destroy", "cbd_status_string", "cbd_last_error", "cbd_plan_info",
           "cbd_plan_subgemm", "cbd_plan_zero_region")


class Problem(ctypes.Structure):
    _fields_ = [("n", ctypes.c_int64), ("g", ctypes.c_int64), ("c", ctypes.c_int64),
                ("k", ctypes.c_int64), ("hi", ctypes.c_int64), ("wi", ctypes.c_int64),
                ("y", ctypes.c_int64), ("x", ctypes.c_int64),
                ("stride_h", ctypes.c_int32), ("stride_w", ctypes.c_int32),
                ("pad_h", ctypes.c_int32), ("pad_w", ctypes.c_int32),
                ("dil_h", ctypes.c_int32), ("dil_w", ctypes.c_int32),
                ("layout", ctypes.c_int32), ("dtype", ctypes.c_int32)]


class PlanOptions(ctypes.Structure):
    _fields_ = [("force_kernel", ctypes.c_int32), ("no_split", ctypes.c_int32),
                ("rows_per_wg", ctypes.c_int32), ("grouped_dot", ctypes.c_int32),
                ("cols_per_wg", ctypes.c_int32), ("ksplit", ctypes.c_int32),
                ("per_class", ctypes.c_int32), ("static_shape", ctypes.c_int32),
                ("merge_phases", ctypes.c_int32), ("reserved", ctypes.c_int32 * 3)]


class PlanInfo(ctypes.Structure):
    _fields_ = [("ho", ctypes.c_int64), ("wo", ctypes.c_int64),
                ("num_subgemms", ctypes.c_int32), ("num_zero_regions", ctypes.c_int32),
                ("kernel", ctypes.c_int32), ("tile_m", ctypes.c_int32),
                ("tile_n", ctypes.c_int32), ("tile_k", ctypes.c_int32),
                ("threads_main", ctypes.c_int32), ("launches", ctypes.c_int32),
                ("grid_main", ctypes.c_int64), ("grid_zero", ctypes.c_int64),
                ("useful_flops", ctypes.c_int64), ("executed_macs", ctypes.c_int64),
                ("zero_elems", ctypes.c_int64), ("lds_dynamic", ctypes.c_int64),
                ("rows_per_wg", ctypes.c_int64), ("cols_per_wg", ctypes.c_int64),
                ("ksplit", ctypes.c_int64), ("static_shape", ctypes.c_int64),
                ("workspace_bytes", ctypes.c_int64),
                ("variant", ctypes.c_int64),
                ("align_dy", ctypes.c_int32), ("align_w", ctypes.c_int32),
                ("align_dx", ctypes.c_int32),
                ("auto_ksplit", ctypes.c_int64), ("auto_workspace_bytes", ctypes.c_int64),
                ("zero_in_epilogue", ctypes.c_int32), ("reserved_", ctypes.c_int32)]


class SubGemm(ctypes.Structure):
    _fields_ = [("id", ctypes.c_int32), ("class_h", ctypes.c_int32), ("class_w", ctypes.c_int32),
                ("phase_h", ctypes.c_int32), ("phase_w", ctypes.c_int32),
                ("beta_h", ctypes.c_int32), ("beta_w", ctypes.c_int32),
                ("taps_h", ctypes.c_int32), ("taps_w", ctypes.c_int32),
                ("tstep_h", ctypes.c_int32), ("tstep_w", ctypes.c_int32),
                ("delta_h", ctypes.c_int32), ("delta_w", ctypes.c_int32),
                ("pos_h", ctypes.c_int64), ("pos_w", ctypes.c_int64),
                ("m", ctypes.c_int64), ("n", ctypes.c_int64), ("k", ctypes.c_int64),
                ("tile_begin", ctypes.c_int64), ("tiles", ctypes.c_int64)]


class ZeroRegion(ctypes.Structure):
    _fields_ = [("phase_h", ctypes.c_int32), ("phase_w", ctypes.c_int32),
                ("pos_h", ctypes.c_int64), ("pos_w", ctypes.c_int64)]


def _load():
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is not built; run `python dnn_conv2d_bwd_amd/build.py`")
    L = ctypes.CDLL(LIB_PATH)
    P = ctypes.POINTER
    L.cbd_plan.argtypes = [P(Problem), P(ctypes.c_void_p)]
    L.cbd_plan_ex.argtypes = [P(Problem), P(PlanOptions), P(ctypes.c_void_p)]
    L.cbd_run.argtypes = [ctypes.c_void_p] * 5
    L.cbd_run_ws.argtypes = [ctypes.c_void_p] * 5 + [ctypes.c_uint64, ctypes.c_void_p]
    L.cbd_run_noalloc.argtypes = [ctypes.c_void_p] * 5
    L.cbd_plan_workspace_size.argtypes = [ctypes.c_void_p, P(ctypes.c_uint64)]
    L.cbd_plan_destroy.argtypes = [ctypes.c_void_p]
    L.cbd_plan_destroy.restype = None
    L.cbd_status_string.argtypes = [ctypes.c_int]
    L.cbd_status_string.restype = ctypes.c_char_p
    L.cbd_last_error.restype = ctypes.c_char_p
    L.cbd_plan_info.argtypes = [ctypes.c_void_p, P(PlanInfo)]
    L.cbd_plan_subgemm.argtypes = [ctypes.c_void_p, ctypes.c_int32, P(SubGemm)]
    L.cbd_plan_zero_region.argtypes = [ctypes.c_void_p, ctypes.c_int32, P(ZeroRegion)]
    for f in ("cbd_plan", "cbd_plan_ex", "cbd_run", "cbd_run_ws", "cbd_run_noalloc", "cbd_plan_workspace_size",
              "cbd_plan_info", "cbd_plan_subgemm",
              "cbd_plan_zero_region"):
        getattr(L, f).restype = ctypes.c_int
    return L


_lib = _load()


class CbdError(RuntimeError):
    def __init__(self, status, where):
        self.status = status
        detail = _lib.cbd_last_error().decode()
        super().__init__(f"{where}: {STATUS.get(status, status)}: {detail}")


def _check(st, where):
    if st != 0:
        raise CbdError(st, where)


def _pair(v):
    return (v, v) if isinstance(v, int) else (int(v[0]), int(v[1]))


def _layout(v):
    if isinstance(v, str):
        return {"nchw": NCHW, "gkcyx": NCHW, "ngchw": NCHW, "nhwc": NHWC, "kyxc": NHWC}[v.lower()]
    return int(v)


def _dtype(v):
    if isinstance(v, str):
        return {"f32": F32, "fp32": F32, "float32": F32, "bf16": BF16, "bfloat16": BF16}[v.lower()]
    return int(v)


def make_problem(n, g, c, k, hi, wi, y, x, stride=1, pad=0, dil=1, layout="nchw", dtype="f32"):
    sh, sw = _pair(stride)
    ph, pw = _pair(pad)
    dh, dw = _pair(dil)
    return Problem(n, g, c, k, hi, wi, y, x, sh, sw, ph, pw, dh, dw, _layout(layout), _dtype(dtype))


class Plan:
    """Owns a cbd_plan_t; immutable; safe to run from several streams."""

    def __init__(self, problem: Problem, force_kernel: int = KERNEL_AUTO, no_split: bool = False,
                 rows_per_wg: int = 0, grouped_dot: bool = False, cols_per_wg: int = 0,
                 ksplit: int = 0, per_class: bool = False, static_shape: int = 0, merge_phases: int = 0):
        self.problem = problem
        h = ctypes.c_void_p()
        opts = PlanOptions(force_kernel, 1 if no_split else 0, rows_per_wg, 1 if grouped_dot else 0,
                           cols_per_wg, ksplit, 1 if per_class else 0, int(static_shape), int(merge_phases))
        _check(_lib.cbd_plan_ex(ctypes.byref(problem), ctypes.byref(opts), ctypes.byref(h)),
               "cbd_plan")
        self._h = h

    @property
    def handle(self):
        return self._h

    def workspace_size(self) -> int:
        """Device workspace bytes for the plan's fastest configuration
        (required for an explicit ksplit >= 2; otherwise enables the
        planner's split configuration; 0: none)."""
        out = ctypes.c_uint64()
        _check(_lib.cbd_plan_workspace_size(self._h, ctypes.byref(out)), "cbd_plan_workspace_size")
        return int(out.value)

    def info(self) -> PlanInfo:
        out = PlanInfo()
        _check(_lib.cbd_plan_info(self._h, ctypes.byref(out)), "cbd_plan_info")
        return out

    def subgemms(self):
        out = []
        for i in range(self.info().num_subgemms):
            s = SubGemm()
            _check(_lib.cbd_plan_subgemm(self._h, i, ctypes.byref(s)), "cbd_plan_subgemm")
            out.append(s)
        return out

    def zero_regions(self):
        out = []
        for i in range(self.info().num_zero_regions):
            z = ZeroRegion()
            _check(_lib.cbd_plan_zero_region(self._h, i, ctypes.byref(z)), "cbd_plan_zero_region")
            out.append(z)
        return out

    def shapes(self):
        """Memory-order shapes of dx, dy and w."""
        p, inf = self.problem, self.info()
        cg = p.c // p.g
        if p.layout == NCHW:
            return dict(dx=(p.n, p.c, p.hi, p.wi), dy=(p.n, p.k, inf.ho, inf.wo),
                        w=(p.k, cg, p.y, p.x))
        return dict(dx=(p.n, p.hi, p.wi, p.c), dy=(p.n, inf.ho, inf.wo, p.k),
                    w=(p.k, p.y, p.x, cg))

    def __del__(self):
        h = getattr(self, "_h", None)
        lib = _lib  # None during interpreter shutdown
        if lib is not None and h is not None and h.value:
            lib.cbd_plan_destroy(h)
            self._h = None


def plan(n=None, g=1, c=None, k=None, hi=None, wi=None, y=None, x=None, stride=1, pad=0, dil=1,
         layout="nchw", dtype="f32", force_kernel=KERNEL_AUTO, problem=None,
         no_split=False, rows_per_wg=0, grouped_dot=False, cols_per_wg=0, ksplit=0,
         per_class=False, static_shape=0, merge_phases=0) -> Plan:
    if problem is None:
        problem = make_problem(n, g, c, k, hi, wi, y, x, stride, pad, dil, layout, dtype)
    return Plan(problem, force_kernel, no_split, rows_per_wg, grouped_dot, cols_per_wg, ksplit,
                per_class, static_shape, merge_phases)


def _torch_dtype(dt):
    import torch

    return torch.float32 if dt == F32 else torch.bfloat16


def _check_tensor(t, shape, dt, name):
    import torch

    if not isinstance(t, torch.Tensor) or t.device.type != "cuda":
        raise ValueError(f"{name} must be a GPU torch tensor")
    if t.dtype != _torch_dtype(dt):
        raise ValueError(f"{name} has dtype {t.dtype}, plan wants {_torch_dtype(dt)}")
    if not t.is_contiguous() or tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must be contiguous with shape {tuple(shape)}, got {tuple(t.shape)}")


def run(p: Plan, dy, w, dx, stream=None, workspace=None) -> None:
    """dx <- conv_bwd_data(dy, w) on `stream` (default: torch's current stream).
    workspace: a device tensor for cbd_run_ws -- required (at least
    p.workspace_size() bytes) for a plan with an explicit ksplit >= 2;
    otherwise optional, and with at least p.workspace_size() bytes the plan
    runs the planner's split-K configuration; None: cbd_run."""
    import torch

    sh = p.shapes()
    dt = p.problem.dtype
    _check_tensor(dy, sh["dy"], dt, "dy")
    _check_tensor(w, sh["w"], dt, "w")
    _check_tensor(dx, sh["dx"], dt, "dx")
    if stream is None:
        stream = torch.cuda.current_stream(dx.device)
    handle = stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream)
    if workspace is None:
        _check(_lib.cbd_run(p.handle, ctypes.c_void_p(dy.data_ptr()), ctypes.c_void_p(w.data_ptr()),
                            ctypes.c_void_p(dx.data_ptr()), ctypes.c_void_p(handle)), "cbd_run")
    else:
        if not workspace.is_cuda or not workspace.is_contiguous():
            raise ValueError("workspace must be a contiguous device tensor")
        _check(_lib.cbd_run_ws(p.handle, ctypes.c_void_p(dy.data_ptr()),
                               ctypes.c_void_p(w.data_ptr()), ctypes.c_void_p(dx.data_ptr()),
                               ctypes.c_void_p(workspace.data_ptr()),
                               ctypes.c_uint64(workspace.numel() * workspace.element_size()),
                               ctypes.c_void_p(handle)), "cbd_run_ws")


NOALLOC_SCRATCH_BYTES = 32 << 20  # CBD_NOALLOC_SCRATCH_BYTES


def run_noalloc(p: Plan, dy, w, dx, stream=None) -> None:
    """dx <- conv_bwd_data(dy, w) through cbd_run_noalloc: the library's own
    static device workspace instead of a caller's (no allocation)."""
    import torch

    sh = p.shapes()
    dt = p.problem.dtype
    _check_tensor(dy, sh["dy"], dt, "dy")
    _check_tensor(w, sh["w"], dt, "w")
    _check_tensor(dx, sh["dx"], dt, "dx")
    if stream is None:
        stream = torch.cuda.current_stream(dx.device)
    handle = stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream)
    _check(_lib.cbd_run_noalloc(p.handle, ctypes.c_void_p(dy.data_ptr()), ctypes.c_void_p(w.data_ptr()),
                                ctypes.c_void_p(dx.data_ptr()), ctypes.c_void_p(handle)), "cbd_run_noalloc")


def run_raw(p: Plan, dy_ptr: int, w_ptr: int, dx_ptr: int, stream_handle: int = 0) -> int:
    """cbd_run on raw device addresses; returns the status code."""
    return _lib.cbd_run(p.handle, ctypes.c_void_p(dy_ptr), ctypes.c_void_p(w_ptr),
                        ctypes.c_void_p(dx_ptr), ctypes.c_void_p(stream_handle))


_plan_cache = {}


def conv2d_bwd_data(dy, w, input_size, stride=1, padding=0, dilation=1, groups=1, layout="nchw"):
    """dX for torch tensors.  input_size is dX's logical (N, C, H, W); layout
    'nchw' takes dy as (N, K, Ho, Wo) and w as (K, C/G, Y, X), 'nhwc' takes dy
    as (N, Ho, Wo, K) and w as (K, Y, X, C/G) and returns dX as (N, H, W, C)."""
    import torch

    lay = _layout(layout)
    n, c, hi, wi = (int(v) for v in input_size)
    if lay == NCHW:
        k, _, y, x = w.shape
    else:
        k, y, x, _ = w.shape
    dt = F32 if dy.dtype == torch.float32 else BF16
    key = (n, groups, c, k, hi, wi, y, x, _pair(stride), _pair(padding), _pair(dilation), lay, dt)
    p = _plan_cache.get(key)
    if p is None:
        p = plan(n, groups, c, k, hi, wi, y, x, stride, padding, dilation, lay, dt)
        _plan_cache[key] = p
    dx = torch.empty(p.shapes()["dx"], dtype=dy.dtype, device=dy.device)
    run(p, dy, w, dx)
    return dx
