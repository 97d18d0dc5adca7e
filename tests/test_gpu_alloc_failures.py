"""Error injection: every device and pinned-host allocation the library makes
can be made to fail from the host (spectra_test_fail_allocations).  Each
allocating entry point must then report SPECTRA_E_NOMEM, release what it had
allocated (the device's free memory returns to its value) and work normally
once the hook is off.  No kernel is made to fail: the hook acts before the
allocation, on the host."""
import os
import tempfile

import numpy as np
import pytest

from dequant_gemv_spectra_amd import synth

pytestmark = pytest.mark.gpu


def _sp():
    from dequant_gemv_spectra_amd import spectra
    return spectra


def _torch():
    import torch
    return torch


def _free_bytes():
    torch = _torch()
    torch.cuda.synchronize()
    return torch.cuda.mem_get_info()[0]


def _expect_nomem(sp, fn):
    with pytest.raises(sp.SpectraError) as e:
        fn()
    assert e.value.status == sp.SPECTRA_E_NOMEM, (e.value.status, str(e.value))


@pytest.fixture
def hook_off():
    yield
    _sp().spectra_test_fail_allocations(0, 0)


def test_pack_fails_cleanly_at_each_allocation(hook_off):
    """Host pack allocates W and gamma staging, the kurtosis scratch, the
    status words and the container: failing each one in turn."""
    sp = _sp()
    W, g, x = synth.random_case(200, 300, 4, 70)
    ref = sp.spectra_export(sp.spectra_pack(W, g))
    free0 = _free_bytes()
    for skip in range(5):
        sp.spectra_test_fail_allocations(skip, 1)
        _expect_nomem(sp, lambda: sp.spectra_pack(W, g))
        sp.spectra_test_fail_allocations(0, 0)
    assert _free_bytes() == free0
    c = sp.spectra_pack(W, g)  # and the next pack is whole
    assert sp.spectra_export(c) == ref
    c.close()


def test_workspace_kv_step_and_load_fail_cleanly(hook_off):
    sp, torch = _sp(), _torch()
    W, g, x = synth.random_case(96, 512, 4, 71, M=24)
    c = sp.spectra_pack(W, g)
    xd = torch.from_numpy(x).cuda()
    want = sp.spectra_gemm(c, xd, kernel="mfma")
    path = os.path.join(tempfile.mkdtemp(), "c.spc")
    sp.spectra_save(c, path)
    s = torch.cuda.Stream()  # device objects the checks below use, made before the reference point
    y = torch.empty(96, dtype=torch.float16, device="cuda")
    x0 = xd[0].contiguous()
    ym = torch.empty((24, 96), dtype=torch.float16, device="cuda")
    # warm each path once (the runtime loads a kernel's code object on its
    # first use, which takes device memory for good)
    plan = sp.StepPlan([{"containers": [c], "ys": [y], "input": -1, "x": x0}])
    plan.run()
    plan.close()
    kv = sp.KvCache(64, 2, 64)
    kv.close()
    sp.spectra_load(path).close()
    torch.cuda.synchronize()
    free0 = _free_bytes()
    def failing(label, skip, fn):
        sp.spectra_test_fail_allocations(skip, 1)
        _expect_nomem(sp, fn)
        sp.spectra_test_fail_allocations(0, 0)
        now = _free_bytes()
        assert now == free0, f"{label} (allocation {skip + 1}): device free memory {now - free0:+d} bytes"

    failing("MFMA workspace of a new stream", 0, lambda: sp.spectra_gemm(c, xd, ym, stream=s, kernel="mfma"))
    failing("KV cache", 0, lambda: sp.KvCache(64, 2, 64))
    failing("step plan", 0, lambda: sp.StepPlan([{"containers": [c], "ys": [y], "input": -1, "x": x0}]))
    for skip in range(3):  # a file load: the container, then each pinned staging buffer
        failing("file load", skip, lambda: sp.spectra_load(path))
    # everything works again
    sp.spectra_gemm(c, xd, ym, stream=s, kernel="mfma")
    torch.cuda.synchronize()
    assert torch.equal(ym, want)
    c2 = sp.spectra_load(path)
    assert sp.spectra_export(c2) == sp.spectra_export(c)
    kv = sp.KvCache(64, 2, 64)
    kv.close()
    c2.close()
    c.close()


def test_hook_rejects_negative_arguments():
    sp = _sp()
    with pytest.raises(sp.SpectraError) as e:
        sp.spectra_test_fail_allocations(-1, 1)
    assert e.value.status == sp.SPECTRA_E_INVAL
