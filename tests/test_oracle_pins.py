"""Pins of the CPU oracle against facts that do not come from the oracle itself:
closed forms, library routines on special cases, hand-derived byte fixtures,
brute force on tiny inputs and invariants of the method.  CPU only."""
import os

import numpy as np
import pytest
import scipy.stats

from oracle import spectra_oracle as O
from dequant_gemv_spectra_amd import synth

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _col(values, K=1, gamma=1.0):
    W = np.zeros((len(values), K), dtype=np.float16)
    W[:, 0] = np.asarray(values, dtype=np.float16)
    g = np.full(K, gamma, dtype=np.float16)
    return W, g


# --------------------------------------------------------------------------
# kurtosis: closed forms
# --------------------------------------------------------------------------
@pytest.mark.parametrize("N", list(range(2, 41)) + [64, 256, 1000])
def test_single_spike_excess_kurtosis_closed_form(N):
    # One nonzero value among N is Bernoulli(1/N): excess kurtosis (N^2-6N+6)/(N-1).
    for pos, a in ((0, 1.0), (N - 1, -3.5), (N // 2, 0.0625)):
        vals = np.zeros(N)
        vals[pos] = a
        W, g = _col(vals, gamma=0.75)
        kap, m2 = O.channel_kurtosis(W, g)
        exact = (N * N - 6 * N + 6) / (N - 1)
        assert kap[0] == pytest.approx(exact, rel=1e-12, abs=1e-12)
        # threshold placement: flagged exactly from N = 8 on (7 -> 2.167, 8 -> 3.143)
        assert bool(O.outlier_mask(W, g)[0]) == (N >= 8)


@pytest.mark.parametrize("N", [2, 4, 10, 64, 1000])
def test_two_point_symmetric_is_minus_two(N):
    vals = np.where(np.arange(N) % 2 == 0, 0.5, -0.5)
    W, g = _col(vals, gamma=1.25)
    kap, _ = O.channel_kurtosis(W, g)
    assert kap[0] == pytest.approx(-2.0, abs=1e-13)
    assert not O.outlier_mask(W, g)[0]


@pytest.mark.parametrize("N,n1", [(10, 1), (10, 3), (50, 7), (200, 199), (97, 45)])
def test_bernoulli_closed_form(N, n1):
    vals = np.zeros(N)
    vals[np.random.default_rng(N + n1).choice(N, n1, replace=False)] = 2.0
    W, g = _col(vals)
    p = n1 / N
    pq = p * (1 - p)
    kap, _ = O.channel_kurtosis(W, g)
    assert kap[0] == pytest.approx((1 - 6 * pq) / pq, rel=1e-12, abs=1e-12)


def test_matches_scipy_fisher_population_kurtosis():
    rng = np.random.default_rng(7)
    W = (rng.standard_t(4, size=(333, 40)) * 0.1).astype(np.float16)
    g = rng.uniform(0.5, 1.5, 40).astype(np.float16)
    kap, _ = O.channel_kurtosis(W, g)
    S = W.astype(np.float64) * g.astype(np.float64)
    ref = scipy.stats.kurtosis(S, axis=0, fisher=True, bias=True)
    np.testing.assert_allclose(kap, ref, rtol=1e-12, atol=1e-12)


def test_gain_scaling_invariance():
    rng = np.random.default_rng(3)
    W = (rng.standard_normal((513, 16)) * 0.02).astype(np.float16)
    W[:, 5] = (rng.standard_t(3, 513) * 0.2).astype(np.float16)
    ones = np.ones(16, dtype=np.float16)
    k1, _ = O.channel_kurtosis(W, ones)
    # a power-of-two gain scales s exactly, so kappa is bit-identical
    for j in (-3, 1, 4):
        kj, _ = O.channel_kurtosis(W, np.full(16, 2.0 ** j, dtype=np.float16))
        assert np.array_equal(k1, kj)
    # a negative gain leaves kappa (even moments) unchanged up to rounding
    kn, _ = O.channel_kurtosis(W, -ones)
    np.testing.assert_allclose(kn, k1, rtol=1e-13)
    # gain 0: the channel is constant, never heavy-tailed
    g0 = ones.copy()
    g0[5] = 0
    assert O.outlier_mask(W, ones)[5] and not O.outlier_mask(W, g0)[5]


def test_constant_and_single_row_columns_are_bulk():
    W = np.full((6, 3), 0.5, dtype=np.float16)
    assert not O.outlier_mask(W, np.ones(3, np.float16)).any()
    W1 = np.array([[1.0, -2.0, 3.0]], dtype=np.float16)
    assert not O.outlier_mask(W1, np.ones(3, np.float16)).any()


def test_row_order_does_not_change_mask():
    W, g, _ = synth.random_case(700, 96, 4, seed=11)
    m = O.outlier_mask(W, g)
    perm = np.random.default_rng(0).permutation(700)
    assert np.array_equal(m, O.outlier_mask(W[perm], g))


def test_planted_heavy_tailed_channels_are_found():
    lin = synth.workload(1).linears[0]
    W = synth.weights(lin, 1)
    g = synth.gamma(lin, 1)
    m = O.outlier_mask(W, g)
    planted = synth.outlier_channels(lin, 1)
    # at N = 2048 every t(3) column and no Gaussian column exceeds 3.0
    assert np.array_equal(np.nonzero(m)[0], planted)


# --------------------------------------------------------------------------
# permutation
# --------------------------------------------------------------------------
def test_permutation_invariants():
    mask = np.zeros(77, bool)
    mask[[0, 5, 6, 40, 76]] = True
    p = O.permutation(mask)
    assert sorted(p.tolist()) == list(range(77))
    kb = 77 - 5
    assert np.all(np.diff(p[:kb]) > 0) and np.all(np.diff(p[kb:]) > 0)
    assert not mask[p[:kb]].any() and mask[p[kb:]].all()


# --------------------------------------------------------------------------
# quantizer
# --------------------------------------------------------------------------
def _grid_group(rng, e, z, n_members=32):
    q = rng.integers(0, 16, n_members)
    q[rng.choice(n_members, 2, replace=False)] = [0, 15]
    return (q - z) * 2.0 ** e, q


@pytest.mark.parametrize("e", [-24, -20, -14, -10, -6, -3, 0, 3])
def test_grid_valued_groups_round_trip_exactly(e):
    rng = np.random.default_rng(100 + e)
    for z in range(16):
        for n_members in (32, 17, 1 + (z % 5) + 1):
            w, q = _grid_group(rng, e, z, n_members)
            if n_members < 2:
                continue
            assert np.all(w.astype(np.float16).astype(np.float64) == w)  # fp16-exact inputs
            qq, zz, s16 = O.quantize_groups(w[None, :])
            assert float(s16[0, 0]) == 2.0 ** e
            assert int(zz[0, 0]) == z
            assert np.array_equal(qq[0, 0, :n_members], q)
            assert np.all(qq[0, 0, n_members:] == z)  # padding dequantizes to 0
            wh = O.dequantize_groups(qq, zz, s16, n_members)
            assert np.array_equal(wh[0], w)


def test_all_zero_group():
    q, z, s16 = O.quantize_groups(np.zeros((1, 40)))
    assert np.all(s16 == 0) and np.all(z == 0) and np.all(q == 0)
    assert np.all(O.dequantize_groups(q, z, s16, 40) == 0)


def test_tiny_range_group_underflows_to_zero_scale():
    # range 15 * 2^-26 -> s = 2^-26 < 2^-25 (half the smallest fp16 subnormal) -> s16 = 0
    w = np.zeros((1, 32))
    w[0, 3] = 15 * 2.0 ** -26
    q, z, s16 = O.quantize_groups(w)
    assert s16[0, 0] == 0 and z[0, 0] == 0 and np.all(q == 0)


def test_one_signed_groups():
    w = np.abs(np.random.default_rng(1).standard_normal((3, 64))) * 0.01 + 1e-3
    _, z, _ = O.quantize_groups(w)
    assert np.all(z == 0)          # lo = 0
    _, z, _ = O.quantize_groups(-w)
    assert np.all(z == 15)         # hi = 0 -> -lo/s16 = 15 * s/s16 ~ 15


def test_error_bound_and_monotonicity():
    rng = np.random.default_rng(5)
    for scale in (1e-6, 3e-5, 1e-3, 0.02, 1.0, 300.0):
        for skew in (0.0, 0.8, -0.8):
            w = (rng.standard_normal((64, 96)) + skew) * scale
            w = w.astype(np.float16).astype(np.float64)
            q, z, s16 = O.quantize_groups(w)
            wh = O.dequantize_groups(q, z, s16, 96)
            wp = w.reshape(64, 3, 32)
            lo = np.minimum(0, wp.min(axis=2))
            hi = np.maximum(0, wp.max(axis=2))
            s = (hi - lo) / 15
            sd = s16.astype(np.float64)
            bound = sd / 2 + 15 * np.abs(s - sd)
            err = np.abs(wp - wh.reshape(64, 3, 32))
            assert np.all(err <= bound[:, :, None] * (1 + 1e-12) + 1e-300)
            # codes are monotone in w within each group
            order = np.argsort(wp, axis=2, kind="stable")
            qs = np.take_along_axis(q.astype(int), order, axis=2)
            assert np.all(np.diff(qs, axis=2) >= 0)


# --------------------------------------------------------------------------
# container image
# --------------------------------------------------------------------------
def _read_golden(name):
    size = None
    img = None
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.split("#", 1)[0].strip()
            if not line:
                continue
            if line.startswith("size"):
                size = int(line.split()[1])
                img = bytearray(size)
                continue
            parts = line.split()
            off = int(parts[0])
            data = bytes(int(h, 16) for h in parts[1:])
            img[off:off + len(data)] = data
    return bytes(img)


def test_tiny_container_matches_hand_derived_bytes():
    W = np.zeros((8, 3), dtype=np.float16)
    W[0, 0] = 1.0
    n = np.arange(8)
    W[:, 1] = (-n / 16.0).astype(np.float16) + np.float16(0)
    W[:, 2] = ((15 - n) / 16.0).astype(np.float16)
    W[0, 1] = 0.0
    img = O.pack(W, np.ones(3, np.float16))
    assert img == _read_golden("tiny_container.txt")


def test_code_word_bit_placement_fixture():
    # group with q_e = e mod 16: word d holds members 8d..8d+7 -> even members in the
    # low half (bits 0,4,8,12), odd members in the high half (bits 16,20,24,28).
    q = (np.arange(32) % 16).astype(np.uint8).reshape(1, 1, 32)
    words = O.encode_codes(q)[0, 0]
    assert [hex(int(v)) for v in words] == ["0x75316420", "0xfdb9eca8", "0x75316420", "0xfdb9eca8"]
    assert np.array_equal(O.decode_codes(words.reshape(1, 1, 4)), q)


@pytest.mark.parametrize("N,K,n_out,seed", [(1, 1, 0, 0), (3, 31, 1, 1), (17, 33, 2, 2),
                                            (64, 200, 9, 3), (40, 64, 0, 4), (9, 97, 5, 5)])
def test_pack_unpack_round_trip_and_footprint(N, K, n_out, seed):
    W, g, _ = synth.random_case(N, K, n_out, seed)
    img = O.pack(W, g)
    u = O.unpack(img)
    mask = O.outlier_mask(W, g)
    assert np.array_equal(u["mask"], mask)
    assert u["n_out"] == int(mask.sum()) and u["K_b"] == K - u["n_out"]
    assert u["G"] == -(-u["K_b"] // 32)
    # heavy-tailed channels pass through bit-exact
    assert np.array_equal(u["O"].view(np.uint16), W[:, u["perm"][u["K_b"]:]].view(np.uint16))
    oc = u["perm"][u["K_b"]:]
    assert np.array_equal(u["W_hat"][:, oc], W[:, oc].astype(np.float64))
    # footprint closed form equals the payload sections
    sz = O.section_sizes(K, N, u["n_out"])
    assert O.footprint(K, N, u["n_out"]) == sz["codes"] + sz["scales"] + sz["zeros"] + sz["outliers"]
    assert len(img) == u["total"] and len(img) % 256 == 0
    # reconstruction of selected rows agrees with the whole
    rows = np.arange(N)[::2]
    assert np.array_equal(O.reconstruct_rows(img, rows), u["W_hat"][rows])


def test_footprint_bits_per_weight():
    # K_b a multiple of 32: 4.625 bits per bulk weight + 16 per heavy-tailed weight
    for N, K, n_out in [(128, 2048 + 16, 16), (10, 4096 + 41, 41), (7, 320, 0)]:
        bits = O.footprint(K, N, n_out) * 8
        assert bits == pytest.approx(N * ((K - n_out) * 4.625 + n_out * 16), abs=4)
    # the single 2048x2048 linear with 16 heavy-tailed channels: K_b = 2032 pads to
    # 64 groups per row -> 2048*64*18.5 + 2048*16*2 bytes, 3.37x smaller than fp16
    assert O.footprint(2048, 2048, 16) == 2048 * 64 * 18 + 2048 * 32 + 2048 * 16 * 2


def test_nonfinite_rejected():
    W = np.zeros((4, 4), np.float16)
    W[1, 2] = np.inf
    with pytest.raises(ValueError):
        O.pack(W, np.ones(4, np.float16))
    with pytest.raises(ValueError):
        O.pack(np.zeros((4, 4), np.float16), np.array([1, np.nan, 1, 1], np.float16))


def test_all_channels_heavy_tailed():
    # every column a single spike in 9 rows -> all flagged, no bulk
    W = np.zeros((9, 5), np.float16)
    for k in range(5):
        W[k, k] = 1.0 + k
    img = O.pack(W, np.ones(5, np.float16))
    u = O.unpack(img)
    assert u["n_out"] == 5 and u["K_b"] == 0 and u["G"] == 0
    assert np.array_equal(u["W_hat"], W.astype(np.float64))


# --------------------------------------------------------------------------
# product
# --------------------------------------------------------------------------
def _brute(W_hat, x):
    M, K = len(x), len(x[0])
    N = len(W_hat)
    y = [[0.0] * N for _ in range(M)]
    for m in range(M):
        for n in range(N):
            acc = 0.0
            for k in range(K):
                acc += float(x[m][k]) * float(W_hat[n][k])
            y[m][n] = acc
    return y


@pytest.mark.parametrize("N,K,n_out,M,seed", [(5, 40, 2, 1, 0), (16, 64, 3, 3, 1), (33, 50, 0, 2, 2)])
def test_matmul_ref_brute_force(N, K, n_out, M, seed):
    W, g, x = synth.random_case(N, K, n_out, seed, M=M)
    u = O.unpack(O.pack(W, g))
    y = O.matmul_ref(u["W_hat"], x)
    yb = np.array(_brute(u["W_hat"].tolist(), x.astype(np.float64).tolist()))
    np.testing.assert_allclose(y, yb, rtol=1e-13, atol=1e-15)


def test_one_hot_inputs_select_columns():
    W, g, _ = synth.random_case(48, 70, 3, 9)
    W[:, 7] = (np.random.default_rng(1).standard_t(3, 48) * 0.2).astype(np.float16)
    img = O.pack(W, g)
    u = O.unpack(img)
    for k in range(70):
        x = np.zeros((1, 70), np.float16)
        x[0, k] = 1.0
        y = O.matmul_ref(u["W_hat"], x)[0]
        if u["mask"][k]:
            assert np.array_equal(y, W[:, k].astype(np.float64))   # exact pass-through
        else:
            j = int(np.nonzero(u["perm"] == k)[0][0])
            g_, e = divmod(j, 32)
            wh = (u["q"][:, g_, e].astype(np.float64) - u["z"][:, g_]) * u["s16"][:, g_].astype(np.float64)
            assert np.array_equal(y, wh)


def test_tolerance_definition_shape_and_floor():
    # by hand: |W_hat| |x|^T for W_hat rows (1, -2), (0, 0), (-4, 0.5) and
    # x rows (3, 1), (-2, -6): row 0 of x gives 5, 0, 12.5; row 1 gives 14,
    # 0, 11 (an absolute value dropped on either operand, or W_hat not
    # transposed, changes every one of them)
    W_hat = np.array([[1.0, -2.0], [0.0, 0.0], [-4.0, 0.5]])
    x = np.array([[3.0, 1.0], [-2.0, -6.0]], np.float16)
    t = O.tolerance(W_hat, x)
    assert t.shape == (2, 3)
    np.testing.assert_allclose(t, 1e-3 * np.array([[5.0, 0.0, 12.5], [14.0, 0.0, 11.0]]) + 1e-6, rtol=1e-12)
    assert t[0, 1] == t[1, 1] == pytest.approx(1e-6)  # the floor


# --------------------------------------------------------------------------
# row gather (fused embedding)
# --------------------------------------------------------------------------
def _grid_table(N, K, spike_ch, e, seed):
    """A table whose bulk groups are grid-valued (codes 0 and 15 present in
    every row and group, scale 2^e) and whose channel spike_ch is a single
    spike (flagged heavy-tailed for N >= 8): the gather must return it
    bit-exactly."""
    rng = np.random.default_rng(seed)
    bulk = [k for k in range(K) if k != spike_ch]
    W = np.zeros((N, K), np.float64)
    for n in range(N):
        for g0 in range(0, len(bulk), 32):
            chans = bulk[g0:g0 + 32]
            z = int(rng.integers(0, 16))
            q = rng.integers(0, 16, len(chans))
            q[rng.choice(len(chans), 2, replace=False)] = [0, 15]
            W[n, chans] = (q - z) * 2.0 ** e
    W[3, spike_ch] = 1.5
    W16 = W.astype(np.float16)
    assert np.array_equal(W16.astype(np.float64), W)
    return W16


@pytest.mark.parametrize("N,K,spike,e,seed", [(40, 65, 5, -6, 0), (24, 97, 96, -10, 1), (64, 33, 0, -3, 2)])
def test_embed_ref_grid_table_is_exact(N, K, spike, e, seed):
    W = _grid_table(N, K, spike, e, seed)
    img = O.pack(W, np.ones(K, np.float16))
    u = O.unpack(img)
    assert u["mask"][spike] and u["n_out"] == 1
    ids = np.array([0, 3, N - 1, 3, 7 % N])
    out = O.embed_ref(img, ids)
    assert out.dtype == np.float16
    assert np.array_equal(out.view(np.uint16), W[ids].view(np.uint16))


def test_embed_ref_out_of_range_rows_are_zero_and_match_unpack():
    W, g, _ = synth.random_case(30, 70, 3, 11)
    img = O.pack(W, g)
    ids = np.array([-1, 0, 29, 30, 12, 12, 1 << 40])
    out = O.embed_ref(img, ids)
    ref = O.unpack(img)["W_hat"].astype(np.float16)
    for i, t in enumerate(ids):
        if 0 <= t < 30:
            assert np.array_equal(out[i].view(np.uint16), ref[t].view(np.uint16))
        else:
            assert not out[i].any()
    assert O.embed_ref(img, np.zeros(0, np.int64)).shape == (0, 70)


# --------------------------------------------------------------------------
# Group-32 4-bit KV cache
# --------------------------------------------------------------------------
def test_kv_quantize_grid_vectors_round_trip():
    rng = np.random.default_rng(21)
    T, H, D, e = 5, 3, 128, -7
    x = np.zeros((T, H, D))
    for t in range(T):
        for h in range(H):
            for g in range(D // 32):
                z = int(rng.integers(0, 16))
                q = rng.integers(0, 16, 32)
                q[rng.choice(32, 2, replace=False)] = [0, 15]
                x[t, h, 32 * g:32 * g + 32] = (q - z) * 2.0 ** e
    x16 = x.astype(np.float16)
    assert np.array_equal(x16.astype(np.float64), x)
    q, z, s16 = O.kv_quantize(x16)
    assert np.all(s16.astype(np.float64) == 2.0 ** e)
    assert np.array_equal(O.kv_dequantize(q, z, s16), x)


def test_kv_quantize_is_the_weight_quantizer_per_head():
    x16 = (np.random.default_rng(22).standard_normal((4, 2, 64))).astype(np.float16)
    q, z, s16 = O.kv_quantize(x16)
    q2, z2, s2 = O.quantize_groups(x16.reshape(8, 64).astype(np.float64))
    assert np.array_equal(q.reshape(8, 2, 32), q2) and np.array_equal(z.reshape(8, 2), z2)
    assert np.array_equal(s16.reshape(8, 2), s2)


def _attend_brute(q, K, V):
    import math
    Hq, D = len(q), len(q[0])
    L, Hkv = len(K), len(K[0])
    rep = Hq // Hkv
    out = []
    for h in range(Hq):
        kv = h // rep
        s = [sum(float(q[h][d]) * K[t][kv][d] for d in range(D)) / math.sqrt(D) for t in range(L)]
        m = max(s)
        w = [math.exp(v - m) for v in s]
        tot = sum(w)
        out.append([sum(w[t] * V[t][kv][d] for t in range(L)) / tot for d in range(D)])
    return out


@pytest.mark.parametrize("L,Hkv,rep,D,seed", [(1, 1, 1, 32, 0), (7, 2, 2, 32, 1), (13, 1, 4, 64, 2)])
def test_kv_attend_ref_brute_force(L, Hkv, rep, D, seed):
    rng = np.random.default_rng(seed)
    q16 = rng.standard_normal((Hkv * rep, D)).astype(np.float16)
    K = rng.standard_normal((L, Hkv, D))
    V = rng.standard_normal((L, Hkv, D))
    ref = O.kv_attend_ref(q16, K, V)
    brute = np.array(_attend_brute(q16.astype(np.float64).tolist(), K.tolist(), V.tolist()))
    np.testing.assert_allclose(ref, brute, rtol=1e-12, atol=1e-14)
    if L == 1:
        assert np.allclose(ref, np.repeat(V[0], rep, axis=0))


def test_kv_attend_equal_keys_average_values():
    rng = np.random.default_rng(23)
    L, D = 9, 32
    K = np.tile(rng.standard_normal((1, 1, D)), (L, 1, 1))
    V = rng.standard_normal((L, 1, D))
    q16 = rng.standard_normal((1, D)).astype(np.float16)
    np.testing.assert_allclose(O.kv_attend_ref(q16, K, V)[0], V[:, 0, :].mean(axis=0), rtol=1e-13)


# --------------------------------------------------------------------------
# rounding ties: codes, zero points and scales round half to even
# --------------------------------------------------------------------------
def test_code_and_zero_point_ties_round_half_to_even():
    # {0, 15, 2.5}: lo = 0, hi = 15, s16 = 1, z = 0; 2.5 is a tie -> code 2
    # (half up would give 3).  {-6.5, 8.5}: s16 = 1, -lo/s16 = 6.5 is a tie ->
    # z = 6 (half up: 7); codes rint(-6.5) + 6 = 0 and rint(8.5) + 6 = 14.
    q, z, s16 = O.quantize_groups(np.array([[0.0, 15.0, 2.5]]))
    assert float(s16[0, 0]) == 1.0 and int(z[0, 0]) == 0
    assert list(q[0, 0, :3]) == [0, 15, 2]
    q, z, s16 = O.quantize_groups(np.array([[-6.5, 8.5]]))
    assert float(s16[0, 0]) == 1.0 and int(z[0, 0]) == 6
    assert list(q[0, 0, :2]) == [0, 14]
    # the same groups through the container: one row per group, fp16 inputs
    W = np.zeros((2, 3), np.float16)
    W[0] = [0.0, 15.0, 2.5]
    W[1] = [-6.5, 8.5, 0.0]
    u = O.unpack(O.pack(W, np.ones(3, np.float16)))
    assert u["n_out"] == 0
    assert list(u["q"][0, 0, :3]) == [0, 15, 2] and int(u["z"][0, 0]) == 0
    assert list(u["q"][1, 0, :3]) == [0, 14, 6] and int(u["z"][1, 0]) == 6


def test_scale_ties_round_half_to_even():
    # (hi - lo)/15 exactly halfway between two binary16 values: 1 + 2^-11 goes
    # down to 1 (even significand), 1 + 3*2^-11 up to 1 + 2^-9 (even), where
    # truncation would give 1 + 2^-10 and rounding half up 1 + 2^-10 for both.
    q, z, s16 = O.quantize_groups(np.array([[0.0, 15.0 + 15 * 2.0 ** -11], [0.0, 15.0 + 45 * 2.0 ** -11]]))
    assert float(s16[0, 0]) == 1.0
    assert float(s16[1, 0]) == 1.0 + 2.0 ** -9
    # through the container with fp16 inputs: lo = -15*2^-11 and -45*2^-11
    W = np.zeros((4, 32), np.float16)
    W[0, 0], W[0, 1] = 15.0, -15 * 2.0 ** -11
    W[1, 0], W[1, 1] = 15.0, -45 * 2.0 ** -11
    W[2, 0], W[2, 1] = 7.5, -15 * 2.0 ** -12
    W[3, 0], W[3, 1] = -3.0, 2.0 ** -14
    s = O.unpack(O.pack(W, np.ones(32, np.float16)))["s16"]
    assert float(s[0, 0]) == 1.0 and float(s[1, 0]) == 1.0 + 2.0 ** -9
    assert float(s[2, 0]) == 0.5                     # 0.5 + 2^-12 is a tie -> 0.5
    # (3 + 2^-14)/15 = 0.2000041 lies between 1638 * 2^-13 and 1639 * 2^-13: nearest is the lower
    assert float(s[3, 0]) == 1638 * 2.0 ** -13


# --------------------------------------------------------------------------
# KV attention tolerance: a value computed by hand
# --------------------------------------------------------------------------
def test_kv_attend_tolerance_hand_value():
    # Two cached tokens, one head of two channels.  q = (1, 0); keys give
    # scores 0 and ln 3 after the 1/sqrt(2) scaling, so p = (1/4, 3/4).
    # V = (2, -4), (-8, 1): out = p V = (-5.5, -0.25); the bound is
    # 1e-3 * p |V| + 1e-6 = 1e-3 * (6.5, 1.75) + 1e-6.
    q = np.array([[1.0, 0.0]], np.float16)
    K_hat = np.array([[[0.0, 0.0]], [[np.log(3.0) * np.sqrt(2.0), 0.0]]])
    V_hat = np.array([[[2.0, -4.0]], [[-8.0, 1.0]]])
    out = O.kv_attend_ref(q, K_hat, V_hat)
    np.testing.assert_allclose(out[0], [-5.5, -0.25], rtol=1e-12)
    tol = O.kv_attend_tolerance(q, K_hat, V_hat)
    np.testing.assert_allclose(tol[0], [6.5e-3 + 1e-6, 1.75e-3 + 1e-6], rtol=1e-12)


# --------------------------------------------------------------------------
# the library's hand-written binary64 -> binary16 conversion against numpy
# --------------------------------------------------------------------------
def _conversion_lib(tmp_path_factory):
    import ctypes
    import shutil
    import subprocess
    hipcc = shutil.which("hipcc") or ("/opt/rocm/bin/hipcc" if os.path.exists("/opt/rocm/bin/hipcc") else None)
    if hipcc is None:
        pytest.skip("hipcc is not available to build the host harness")
    d = tmp_path_factory.mktemp("fp16conv")
    so = str(d / "libconv.so")
    src = os.path.join(os.path.dirname(__file__), "fp16_conversion_harness.hip")
    r = subprocess.run([hipcc, "-O2", "-std=c++17", "-fPIC", "-shared", "--offload-arch=gfx950", src, "-o", so],
                       capture_output=True, text=True)
    assert r.returncode == 0, r.stderr
    lib = ctypes.CDLL(so)
    lib.convert_batch.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int64]
    return lib


def test_device_fp16_conversion_matches_numpy(tmp_path_factory):
    """Every finite binary16 value, every midpoint between neighbours (ties),
    points just either side of each midpoint, the subnormal range, overflow
    and the smallest magnitudes: the library's conversion equals numpy's
    float64 -> float16 (round to nearest, ties to even) bit for bit."""
    lib = _conversion_lib(tmp_path_factory)
    bits = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    h = bits.view(np.float16)
    fin = np.isfinite(h)
    vals = h[fin].astype(np.float64)
    pos = np.sort(np.unique(np.abs(vals)))
    nxt = np.append(pos[1:], 65536.0)  # 2^16: the value past the largest finite one
    mids = (pos + nxt) / 2
    probes = np.concatenate([
        vals, mids, -mids,
        np.nextafter(mids, np.inf), np.nextafter(mids, -np.inf),
        -np.nextafter(mids, np.inf), -np.nextafter(mids, -np.inf),
        [2.0 ** -25, -2.0 ** -25, 2.0 ** -26, 3 * 2.0 ** -26, 2.0 ** -30, 1e-300, 5e-324, 0.0, -0.0,
         65519.99, 65520.0, 65536.0, 1e6, -1e6, 1e300, np.inf, -np.inf],
    ])
    got = np.empty(probes.size, np.uint16)
    lib.convert_batch(probes.ctypes.data, got.ctypes.data, probes.size)
    with np.errstate(over="ignore"):  # values past the binary16 range become infinities
        want = probes.astype(np.float16).view(np.uint16)
    bad = np.nonzero(got != want)[0]
    assert bad.size == 0, f"{bad.size} differ; first {probes[bad[0]]!r}: {got[bad[0]]:#06x} vs numpy {want[bad[0]]:#06x}"
    nan = np.array([np.nan], np.float64)
    out = np.empty(1, np.uint16)
    lib.convert_batch(nan.ctypes.data, out.ctypes.data, 1)
    assert (int(out[0]) & 0x7C00) == 0x7C00 and (int(out[0]) & 0x03FF) != 0  # a NaN stays a NaN
