"""cbd_run_noalloc (the library's own static device workspace, for callers
that cannot allocate) against cbd_run_ws with a caller workspace: the same
bits, on two calls in a row with the second problem smaller, for split-K
plans of both families and the planner's split configuration; plans whose
workspace exceeds the static array are refused before any launch."""
from __future__ import annotations

import numpy as np
import pytest
import torch

import dnn_conv2d_bwd_amd as cbd
import oracle
from cbd_inputs import PROBLEMS
from parity import DeviceRun, check, exact_expected_bits, operands, plan_for, to_device

pytestmark = pytest.mark.gpu


def by_name(name):
    return [p for p in PROBLEMS if p.name == name][0]


class NoAllocRun(DeviceRun):
    def __call__(self, stream=None):
        cbd.run_noalloc(self.pl, self.dy_d, self.w_d, self.dx, stream=stream)
        return self


# (problem, batch override, forced kernel, ksplit): pairs run in order, the
# second smaller than the first.
SEQUENCES = [
    # the planner's split configuration of the headline problem's batch
    # shards: 4 and 8 splits, each exactly 32 MiB of partial tiles
    [("c4", 2, cbd.KERNEL_AUTO, 0), ("c4", 1, cbd.KERNEL_AUTO, 0)],
    # explicit split-K on the generic family (fp32 NCHW)
    [("c3b", None, cbd.KERNEL_GENERIC, 4), ("c1", None, cbd.KERNEL_GENERIC, 3)],
    # explicit split-K on the large-tile kernel
    [("c4", 4, cbd.KERNEL_NHWC_BF16, 2), ("c4", 1, cbd.KERNEL_NHWC_BF16, 3)],
    # plans without a workspace
    [("c3a", None, cbd.KERNEL_AUTO, 0), ("c2-14-3", None, cbd.KERNEL_AUTO, 0)],
]


@pytest.mark.parametrize("seq", range(len(SEQUENCES)))
def test_noalloc_matches_run_ws(seq):
    for name, n, force, ksplit in SEQUENCES[seq]:
        p = by_name(name) if n is None else by_name(name).with_(n=n)
        pl = plan_for(p, force, ksplit=ksplit)
        info = pl.info()
        print(f"[noalloc] {name} n={p.n} ksplit={info.ksplit} auto={info.auto_ksplit} "
              f"ws={pl.workspace_size()}", flush=True)
        assert pl.workspace_size() <= cbd.NOALLOC_SCRATCH_BYTES
        dy, w = operands(p)
        dyd, wd = to_device(dy, p), to_device(w, p)
        ws = (torch.empty(pl.workspace_size(), dtype=torch.uint8, device="cuda")
              if pl.workspace_size() else None)
        want = DeviceRun(p, pl, dyd, wd, workspace=ws)()
        got = NoAllocRun(p, pl, dyd, wd)()
        assert np.array_equal(got.result_bits(), want.result_bits()), (name, p.n)
        assert got.guards_intact()
        ok, inf = check(p, got, oracle.bwd_data(p, dy, w))
        assert ok, inf
        # the same bits again (the array keeps the last call's partials)
        bits = got.result_bits().copy()
        got()
        assert np.array_equal(bits, got.result_bits())


def test_noalloc_integer_exact():
    """Split configurations through the static workspace, integer operands:
    bit-exact against the oracle."""
    for name, n, force, ksplit in (("c4", 1, cbd.KERNEL_AUTO, 0), ("c3a", None, cbd.KERNEL_GENERIC, 5)):
        p = by_name(name) if n is None else by_name(name).with_(n=n)
        pl = plan_for(p, force, ksplit=ksplit)
        dy, w = operands(p, "int")
        run = NoAllocRun(p, pl, to_device(dy, p), to_device(w, p))()
        ref = oracle.bwd_data(p, dy, w)
        assert np.array_equal(run.result_bits().reshape(ref.shape), exact_expected_bits(p, ref)), name
        assert run.guards_intact()


def test_noalloc_refuses_large_workspace():
    """A split plan whose partial tiles exceed the static array: UNSUPPORTED,
    nothing launched (dX keeps its sentinel)."""
    p = by_name("c4")
    pl = plan_for(p, cbd.KERNEL_NHWC_BF16, ksplit=2)  # 512 tiles x 256 KiB
    assert pl.workspace_size() > cbd.NOALLOC_SCRATCH_BYTES
    dy, w = operands(p)
    run = NoAllocRun(p, pl, to_device(dy, p), to_device(w, p))
    with pytest.raises(cbd.CbdError) as e:
        run()
    assert e.value.status == 2
    assert "cbd_run_noalloc holds" in cbd._lib.cbd_last_error().decode()
    torch.cuda.synchronize()
    assert torch.isnan(run.buf.float()).all()
