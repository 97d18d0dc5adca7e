"""GPU parity of the Group-32 4-bit KV cache: the quantized data written on
append must equal the oracle's bit for bit; decode attention over the cache
must meet |out - ref| <= 1e-3 * (sum_t p_t |V_hat[t]|) + 1e-6 per element."""
import numpy as np
import pytest

from oracle import spectra_oracle as O

pytestmark = pytest.mark.gpu


def _sp():
    from dequant_gemv_spectra_amd import spectra
    return spectra


def _torch():
    import torch
    return torch


def _split_export(buf, L, H, G):
    n = L * H * G
    parts, pos = [], 0
    for _ in range(2):
        rec = np.frombuffer(buf, "<u4", 4 * n, pos).reshape(L, H, G, 4)
        pos += 16 * n
        sc = np.frombuffer(buf, "<f2", n, pos).reshape(L, H, G)
        pos += 2 * n
        zb = np.frombuffer(buf, np.uint8, n // 2, pos).reshape(L, H, G // 2)
        pos += n // 2
        z = np.empty((L, H, G), np.uint8)
        z[..., 0::2] = zb & 0xF
        z[..., 1::2] = zb >> 4
        q = O.decode_codes(rec.reshape(L * H, G, 4)).reshape(L, H, G, 32)
        parts.append((q, z, sc))
    return parts


def _vectors(rng, T, H, D, scale=1.0):
    return (rng.standard_normal((T, H, D)) * scale).astype(np.float16)


@pytest.mark.parametrize("H,D,chunks,seed", [(1, 64, [1], 0), (8, 128, [5, 1, 30], 1), (2, 256, [17, 3], 2),
                                             (4, 128, [64], 3)])
def test_append_is_bit_exact(H, D, chunks, seed):
    sp, torch = _sp(), _torch()
    rng = np.random.default_rng(seed)
    L = sum(chunks)
    kv = sp.KvCache(L + 7, H, D)
    ks, vs = [], []
    for T in chunks:
        k, v = _vectors(rng, T, H, D), _vectors(rng, T, H, D, 0.3)
        ks.append(k)
        vs.append(v)
        kv.append(torch.from_numpy(k).cuda(), torch.from_numpy(v).cuda())
    torch.cuda.synchronize()
    assert kv.length == L
    (kq, kz, ks16), (vq, vz, vs16) = _split_export(kv.export(), L, H, D // 32)
    for (q, z, s), x in [((kq, kz, ks16), np.concatenate(ks)), ((vq, vz, vs16), np.concatenate(vs))]:
        rq, rz, rs = O.kv_quantize(x)
        assert np.array_equal(q, rq) and np.array_equal(z, rz)
        assert np.array_equal(s.view(np.uint16), rs.view(np.uint16))


def _attend_case(H, rep, D, L, seed, k_scale=1.0):
    sp, torch = _sp(), _torch()
    rng = np.random.default_rng(seed)
    k, v = _vectors(rng, L, H, D, k_scale), _vectors(rng, L, H, D, 0.5)
    kv = sp.KvCache(L, H, D)
    kv.append(torch.from_numpy(k).cuda(), torch.from_numpy(v).cuda())
    q16 = rng.standard_normal((H * rep, D)).astype(np.float16)
    out = kv.attend(torch.from_numpy(q16).cuda()).cpu().numpy().astype(np.float64)
    Kh = O.kv_dequantize(*O.kv_quantize(k))
    Vh = O.kv_dequantize(*O.kv_quantize(v))
    ref = O.kv_attend_ref(q16, Kh, Vh)
    tol = O.kv_attend_tolerance(q16, Kh, Vh)
    err = np.abs(out - ref)
    assert np.all(err <= tol), f"worst ratio {(err / tol).max():.3g}"
    return kv


@pytest.mark.parametrize("H,rep,D,L,seed", [(1, 1, 64, 1, 10), (2, 4, 128, 37, 11), (8, 4, 128, 513, 12),
                                            (1, 16, 256, 1000, 13), (4, 2, 64, 2049, 14)])
def test_attend_within_bound(H, rep, D, L, seed):
    _attend_case(H, rep, D, L, seed)


# One split exactly and one token past it (128 tokens per split), then more
# splits than the combine requests in its first round of loads (32 * 256 / D:
# 64 at D = 128, 32 at D = 256, 128 at D = 64), which walks the remaining
# splits in a second loop.
@pytest.mark.parametrize("H,rep,D,L,seed", [(1, 2, 128, 128, 20), (1, 2, 128, 129, 21), (1, 4, 128, 8325, 22),
                                            (2, 2, 256, 4500, 23), (1, 2, 64, 16600, 24)])
def test_attend_split_boundaries(H, rep, D, L, seed):
    _attend_case(H, rep, D, L, seed)


# Every build of the split kernel (rep rounded up to 1, 2, 4, 8, 16) at every
# head size, at a short cache and one past a split boundary.
@pytest.mark.parametrize("rep", [1, 2, 4, 8, 16])
@pytest.mark.parametrize("D", [64, 128, 256])
@pytest.mark.parametrize("L", [300, 129])
def test_attend_every_build(rep, D, L):
    _attend_case(2 if rep < 16 else 1, rep, D, L, 1000 + 10 * rep + D + L)


# Ratios that are not powers of two run on the next build with the extra
# query heads masked: the 1.5B-class layer's 12 query heads over 2 cache heads
# (6 per cache head), and the other odd ratios.
@pytest.mark.parametrize("H,rep,D,L", [(2, 6, 128, 700), (1, 3, 64, 200), (3, 5, 128, 129), (2, 7, 256, 300),
                                       (1, 9, 128, 260), (1, 12, 64, 131), (1, 15, 128, 400)])
def test_attend_odd_ratios(H, rep, D, L):
    _attend_case(H, rep, D, L, 2000 + rep)


def test_attend_peaked_scores():
    # large keys make the softmax nearly one-hot: the max subtraction matters
    _attend_case(2, 2, 128, 300, 15, k_scale=8.0)


def test_attend_4b_decoder_shape_long_context():
    """32 query heads on 8 cache heads of 128, 8192 cached tokens."""
    _attend_case(8, 4, 128, 8192, 16)


def test_capacity_reset_and_errors():
    sp, torch = _sp(), _torch()
    kv = sp.KvCache(10, 2, 64)
    x = torch.zeros((6, 2, 64), dtype=torch.float16, device="cuda")
    kv.append(x, x)
    with pytest.raises(sp.SpectraError):
        kv.append(x, x)  # 12 > 10
    assert kv.length == 6
    kv.reset()
    assert kv.length == 0
    q = torch.zeros((2, 64), dtype=torch.float16, device="cuda")
    with pytest.raises(sp.SpectraError):
        kv.attend(q)  # empty cache
    kv.append(x, x)
    with pytest.raises(sp.SpectraError):
        kv.attend(torch.zeros((3, 64), dtype=torch.float16, device="cuda"))  # 3 not a multiple of 2
    out = kv.attend(q)
    assert not out.cpu().numpy().any()  # zero values -> zero output
    with pytest.raises(sp.SpectraError):
        sp.KvCache(10, 2, 96)  # head_dim not 64/128/256
    kv.close()
    assert sp.lib().spectra_kv_length(None) == -1
