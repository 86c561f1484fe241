"""Error reporting around launches (host-forced conditions only; every
kernel that runs exits normally)."""
from __future__ import annotations

import ctypes

import numpy as np
import pytest

import synth

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
import gguf_quant_dequant_amd as q  # noqa: E402
from gpu_util import DeviceBytes, dev  # noqa: E402


def _hip():
    # the HIP runtime the library and torch share (one soname, already loaded)
    return ctypes.CDLL("libamdhip64.so.7", mode=ctypes.RTLD_GLOBAL)


def test_an_earlier_runtime_error_is_reported_as_such_and_cleared():
    case = synth.GEMV_CASES["q8_0_256x1024"]
    W, X = synth.gemv_inputs(case, 1)
    Wd = DeviceBytes(W)
    xd = torch.from_numpy(X[0]).to(dev())
    y = torch.full((case.rows,), float("nan"), device=dev())
    torch.cuda.synchronize()
    hip = _hip()
    lib = q.load_library()
    # a failing host call leaves an error on this thread (an invalid device)
    assert hip.hipSetDevice(ctypes.c_int(1 << 20)) != 0
    if hip.hipPeekAtLastError() == 0:
        pytest.skip("this HIP runtime does not keep the failed call's error")
    # straight through the C ABI, so that no other runtime call comes between
    rc = lib.qgemv(case.fmt, ctypes.c_void_p(Wd.ptr), case.rows, case.cols,
                   ctypes.c_void_p(xd.data_ptr()), ctypes.c_void_p(y.data_ptr()), 1, None)
    assert rc == q.QG_ELAUNCH
    assert "earlier" in q.qg_last_error()
    assert hip.hipPeekAtLastError() == 0  # reported, and cleared
    torch.cuda.synchronize()
    assert torch.isnan(y).all()  # nothing was launched
    # the error was cleared: the next call runs
    q.qgemv(case.fmt, Wd.ptr, case.rows, case.cols, xd, y, 1)
    torch.cuda.synchronize()
    assert np.isfinite(y.cpu().numpy()).all()
