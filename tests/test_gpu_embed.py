"""GPU parity of the fused embedding gather (spectra_embed) against the oracle.

Every gathered row must equal the oracle's row of W_hat rounded once to fp16,
bit for bit; ids outside [0, N) give zero rows.
"""
import numpy as np
import pytest

from dequant_gemv_spectra_amd import synth
from oracle import spectra_oracle as O

pytestmark = pytest.mark.gpu


def _sp():
    from dequant_gemv_spectra_amd import spectra
    return spectra


def _torch():
    import torch
    return torch


def _pack(W, g):
    sp = _sp()
    c = sp.spectra_pack(W, g)
    return c, sp.spectra_export(c)


def _gather(c, ids, out=None):
    sp, torch = _sp(), _torch()
    t = torch.from_numpy(np.asarray(ids, np.int32)).cuda()
    y = sp.spectra_embed(c, t, out=out)
    torch.cuda.synchronize()
    return y


def _check(c, img, ids):
    y = _gather(c, ids).cpu().numpy()
    ref = O.embed_ref(img, ids)
    diff = np.nonzero(y.view(np.uint16) != ref.view(np.uint16))
    assert diff[0].size == 0, f"{diff[0].size} entries differ, first at {diff[0][0]}, {diff[1][0]}"


EMBED_CASES = [  # (N, K, planted heavy-tailed channels, seed, T)
    (1, 1, 0, 0, 3),
    (9, 5, 0, 1, 17),
    (300, 1000, 10, 2, 64),      # K % 8 == 0: whole-chunk stores
    (257, 97, 5, 3, 200),        # K % 8 != 0: per-channel stores
    (64, 8192, 82, 4, 150),
    (2049, 3072, 31, 5, 1000),
    (100, 130, 129, 6, 40),      # more heavy-tailed channels than bulk ones
    (50, 16384, 160, 7, 33),     # a long row: fewer waves per block fit the LDS
]


@pytest.mark.parametrize("N,K,n_out,seed,T", EMBED_CASES)
def test_embed_matches_oracle(N, K, n_out, seed, T):
    W, g, _ = synth.random_case(N, K, n_out, seed)
    c, img = _pack(W, g)
    rng = np.random.default_rng(seed + 100)
    ids = rng.integers(0, N, T)
    ids[: min(T, 3)] = [0, N - 1, 0][: min(T, 3)]  # first and last rows, a repeat
    _check(c, img, ids)


def test_embed_out_of_range_ids_give_zero_rows():
    W, g, _ = synth.random_case(40, 256, 4, 8)
    c, img = _pack(W, g)
    ids = np.array([-1, 0, 40, 39, 2**31 - 1, -(2**31), 7], np.int64)
    y = _gather(c, ids).cpu().numpy()
    assert not y[[0, 2, 4, 5]].any()
    _check(c, img, ids)


def test_embed_grid_table_gathers_back_exactly():
    # the oracle pin's construction: grid-valued bulk groups and one spike channel
    rng = np.random.default_rng(9)
    N, K, spike, e = 48, 97, 40, -8
    bulk = [k for k in range(K) if k != spike]
    W = np.zeros((N, K), np.float64)
    for n in range(N):
        for g0 in range(0, len(bulk), 32):
            ch = bulk[g0:g0 + 32]
            z = int(rng.integers(0, 16))
            q = rng.integers(0, 16, len(ch))
            q[rng.choice(len(ch), 2, replace=False)] = [0, 15]
            W[n, ch] = (q - z) * 2.0 ** e
    W[5, spike] = -2.25
    W16 = W.astype(np.float16)
    c, img = _pack(W16, np.ones(K, np.float16))
    ids = np.arange(N)[::-1].copy()
    y = _gather(c, ids).cpu().numpy()
    assert np.array_equal(y.view(np.uint16), W16[ids].view(np.uint16))


def test_embed_unaligned_output_and_empty():
    sp, torch = _sp(), _torch()
    W, g, _ = synth.random_case(70, 512, 5, 10)
    c, img = _pack(W, g)
    ids = np.arange(0, 70, 3)
    buf = torch.zeros(len(ids) * 512 + 2, dtype=torch.float16, device="cuda")
    out = buf[2:].view(len(ids), 512)  # 4-byte but not 16-byte aligned
    y = _gather(c, ids, out=out).cpu().numpy()
    ref = O.embed_ref(img, ids)
    assert np.array_equal(y.view(np.uint16), ref.view(np.uint16))
    assert buf[:2].abs().sum().item() == 0  # nothing written before out
    empty = _gather(c, np.zeros(0, np.int64))
    assert tuple(empty.shape) == (0, 512)


def test_embed_error_paths():
    sp, torch = _sp(), _torch()
    W, g, _ = synth.random_case(20, 64, 2, 11)
    c, _ = _pack(W, g)
    ids = torch.zeros(4, dtype=torch.int32, device="cuda")
    out = torch.empty((4, 64), dtype=torch.float16, device="cuda")
    L = sp.lib()
    import ctypes
    assert L.spectra_embed(c.handle, None, 4, ctypes.c_void_p(out.data_ptr()), None) == sp.SPECTRA_E_INVAL
    assert L.spectra_embed(c.handle, ctypes.c_void_p(ids.data_ptr()), -1,
                           ctypes.c_void_p(out.data_ptr()), None) == sp.SPECTRA_E_INVAL
    assert L.spectra_embed(c.handle, ctypes.c_void_p(ids.data_ptr() + 2), 1,
                           ctypes.c_void_p(out.data_ptr()), None) == sp.SPECTRA_E_INVAL
    assert L.spectra_embed(None, ctypes.c_void_p(ids.data_ptr()), 1,
                           ctypes.c_void_p(out.data_ptr()), None) == sp.SPECTRA_E_INVAL


@pytest.mark.timeout(900)
def test_embed_lm_head_table_sampled():
    """The 131072 x 3072 table (the LM-head shape read as a tied embedding),
    4096 random ids, every gathered row checked."""
    wl = synth.workload(4)
    lin = wl.linears[0]
    W, g = synth.weights(lin, 4), synth.gamma(lin, 4)
    c, img = _pack(W, g)
    del W
    ids = np.random.default_rng(12).integers(0, lin.N, 4096)
    _check(c, img, ids)
