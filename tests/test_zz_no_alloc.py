"""The product entry point that allocates nothing (spectra_gemm_noalloc),
through the C ABI: its outputs equal spectra_gemm_ex's bit for bit and meet
the oracle bound, on two calls in a row (the second with a smaller input),
and a workspace larger than its static scratch is refused (or, for the
split-K kernel's partial sums, the kernel it replaces runs)."""
import numpy as np
import pytest

from dequant_gemv_spectra_amd import synth
from oracle import spectra_oracle as O

pytestmark = pytest.mark.gpu


def test_noalloc_matches_gemm_ex_on_consecutive_calls():
    import torch
    from dequant_gemv_spectra_amd import spectra as sp
    W, g, _ = synth.random_case(700, 2600, 30, 123)
    c = sp.spectra_pack(W, g)
    W_hat = O.unpack(sp.spectra_export(c))["W_hat"]
    rng = np.random.default_rng(123)
    for M, kernel in ((64, "mfma"), (9, "mfma"), (5, "auto"), (1, "auto")):  # larger, then smaller inputs
        x = rng.standard_normal((M, 2600)).astype(np.float16)
        xd = torch.from_numpy(x).cuda()
        y_ref = sp.spectra_gemm(c, xd, kernel=kernel)
        y = torch.full((M, 700), 3.0, dtype=torch.float16, device="cuda")
        sp.spectra_gemm_noalloc(c, xd, y, kernel=kernel)
        torch.cuda.synchronize()
        assert torch.equal(y, y_ref), f"M={M} ({kernel}): differs from spectra_gemm_ex"
        err = np.abs(y.cpu().numpy().astype(np.float64) - O.matmul_ref(W_hat, x))
        assert (err <= O.tolerance(W_hat, x)).all(), f"M={M}: outside the oracle bound"
    c.close()


def test_noalloc_refuses_a_workspace_past_its_scratch():
    import torch
    from dequant_gemv_spectra_amd import spectra as sp
    W, g, _ = synth.random_case(64, 8192, 0, 124)
    c = sp.spectra_pack(W, g)
    M = 600  # 600 * 8192 * 2 bytes > 8 MiB
    x = torch.zeros((M, 8192), dtype=torch.float16, device="cuda")
    y = torch.zeros((M, 64), dtype=torch.float16, device="cuda")
    with pytest.raises(sp.SpectraError) as e:
        sp.spectra_gemm_noalloc(c, x, y, kernel="mfma")
    assert e.value.status == sp.SPECTRA_E_UNSUPPORTED
    assert "8 MiB" in str(e.value)
    c.close()


def test_noalloc_runs_split_k_and_falls_back_past_its_scratch():
    """The split-K kernel under the no-allocation entry point: bit-equal to
    spectra_gemm_ex while its fp32 partial sums fit the 8 MiB scratch; past
    that (here 3 K-ranges x 16 rows x 48000 outputs x 4 bytes, on a shape the
    tiled kernel declines) the entry point runs the strip kernel instead,
    within the oracle bound on sampled rows, and refuses split-K when it is
    forced."""
    import torch
    from dequant_gemv_spectra_amd import spectra as sp
    W, g, _ = synth.random_case(3000, 2048, 20, 125)
    c = sp.spectra_pack(W, g)
    W_hat = O.unpack(sp.spectra_export(c))["W_hat"]
    rng = np.random.default_rng(125)
    for M in (8, 3):
        x = rng.standard_normal((M, 2048)).astype(np.float16)
        xd = torch.from_numpy(x).cuda()
        y_ref = sp.spectra_gemm(c, xd, kernel="mfma_splitk")
        y = torch.full((M, 3000), 3.0, dtype=torch.float16, device="cuda")
        sp.spectra_gemm_noalloc(c, xd, y, kernel="mfma_splitk")
        torch.cuda.synchronize()
        assert torch.equal(y, y_ref), f"M={M}: differs from spectra_gemm_ex"
        err = np.abs(y.cpu().numpy().astype(np.float64) - O.matmul_ref(W_hat, x))
        assert (err <= O.tolerance(W_hat, x)).all()
    c.close()
    W, g, _ = synth.random_case(48000, 12000, 100, 126)
    c = sp.spectra_pack(W, g)
    del W
    img = sp.spectra_export(c)
    M = 16
    assert sp.spectra_gemm_plan(c, M) == "k_mfma_sk"
    x = rng.standard_normal((M, 12000)).astype(np.float16)
    y = torch.full((M, 48000), 3.0, dtype=torch.float16, device="cuda")
    sp.spectra_gemm_noalloc(c, torch.from_numpy(x).cuda(), y)
    torch.cuda.synchronize()
    rows = np.unique(np.concatenate([np.arange(512), rng.integers(0, 48000, 1500), np.arange(47700, 48000)]))
    W_hat = O.reconstruct_rows(img, rows)
    err = np.abs(y.cpu().numpy()[:, rows].astype(np.float64) - O.matmul_ref(W_hat, x))
    assert (err <= O.tolerance(W_hat, x)).all()
    with pytest.raises(sp.SpectraError) as e:  # forced, the split-K kernel is refused rather than replaced
        sp.spectra_gemm_noalloc(c, torch.from_numpy(x).cuda(), y, kernel="mfma_splitk")
    assert e.value.status == sp.SPECTRA_E_UNSUPPORTED
    c.close()
