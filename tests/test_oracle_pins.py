"""Pins of the CPU oracle against what the pages and the mathematics fix.

Each test ties an oracle function to something other than itself: hand-derived
tie tables, exhaustive nibble tables, closed-form error bounds, exact integer
products, a special case that reduces to a plain matrix product, planted-set
recovery and byte totals printed on the pages.
"""
from fractions import Fraction

import numpy as np
import pytest

import oracle as O
import synth
from conftest import read_golden


# ---------------------------------------------------------------- INT8 -------

def test_int8_ties_round_half_even():
    rows = [ln.split() for ln in read_golden("int8_ties.txt")]
    W = np.array([[float(r[0]) for r in rows]], np.float32)
    want = np.array([[int(r[1]) for r in rows]], np.int8)
    q, s = O.quantize_int8(W)
    assert s == np.float32(2.0 ** -7)
    np.testing.assert_array_equal(q, want)


@pytest.mark.parametrize("seed", [0, 1, 2])
def test_int8_closed_form_bound(seed):
    rng = np.random.default_rng(seed)
    W = (rng.standard_normal((37, 301)) * 0.02).astype(np.float32)
    W[5, 7] = -0.2          # largest magnitude is negative
    q, s = O.quantize_int8(W)
    s64 = float(s)
    assert s == np.float32(np.float32(0.2) / np.float32(127))
    assert q[5, 7] == -127
    err = np.abs(W.astype(np.float64) - q.astype(np.float64) * s64)
    # |W/s - q| <= 1/2 plus the fp32 rounding of W/s (|W/s| <= 127)
    assert np.all(err <= s64 * (0.5 + 127 * 2.0 ** -23))
    # q is the nearest code: neither neighbour is closer
    for d in (-1, 1):
        alt = np.abs(W.astype(np.float64) - (q.astype(np.float64) + d) * s64)
        assert np.all(err <= alt + s64 * 1e-5)
    assert q.min() >= -127 and q.max() <= 127


def test_int8_zero_tensor_and_empty():
    q, s = O.quantize_int8(np.zeros((3, 4), np.float32))
    assert s == 0 and not q.any()
    # max|W| = 2^-149 (smallest subnormal): max/127 underflows to 0
    q, s = O.quantize_int8(np.array([[np.float32(2.0 ** -149), 0]], np.float32))
    assert s == 0 and not q.any()
    with pytest.raises(ValueError):
        O.quantize_int8(np.array([[1.0, np.nan]], np.float32))
    q, s = O.quantize_int8(np.zeros((0, 4), np.float32))
    assert q.shape == (0, 4)


def test_int8_on_grid_is_lossless_and_product_is_matmul():
    rng = np.random.default_rng(3)
    q0 = rng.integers(-127, 128, size=(19, 70)).astype(np.int8)
    q0[0, 0] = 127
    s0 = np.float32(2.0 ** -9)
    W = q0.astype(np.float32) * s0
    q, s = O.quantize_int8(W)
    assert s == s0
    np.testing.assert_array_equal(q, q0)
    x = rng.standard_normal((3, 70)).astype(np.float16)
    y = O.linear_int8(q, s, x)
    np.testing.assert_allclose(y, x.astype(np.float64) @ W.astype(np.float64).T, rtol=0, atol=1e-12)


def _exact_int8(q, s, x):
    """s * sum_k q x with x scaled to integers (every finite fp16 times 2^24 is an integer)."""
    xi = (x.astype(np.float64) * 2.0 ** 24).astype(np.int64)
    out = np.empty((x.shape[0], q.shape[0]), object)
    for b in range(x.shape[0]):
        for n in range(q.shape[0]):
            acc = sum(int(a) * int(c) for a, c in zip(q[n], xi[b]))
            out[b, n] = Fraction(acc, 2 ** 24) * Fraction(float(s))
    return out


def test_int8_product_exact_integer():
    rng = np.random.default_rng(4)
    W = (rng.standard_normal((5, 97)) * 0.02).astype(np.float32)
    x = rng.standard_normal((2, 97)).astype(np.float16)
    x[0, 3] = np.float16(6.0e-8)          # subnormal fp16 input
    q, s = O.quantize_int8(W)
    y = O.linear_int8(q, s, x)
    ex = _exact_int8(q, s, x)
    for b in range(2):
        for n in range(5):
            assert abs(Fraction(float(y[b, n])) - ex[b, n]) <= Fraction(1, 10 ** 13)


def test_int8_orientation_unit_vectors():
    rng = np.random.default_rng(5)
    W = (rng.standard_normal((6, 11)) * 0.02).astype(np.float32)
    q, s = O.quantize_int8(W)
    for j in (0, 4, 10):
        x = np.zeros((1, 11), np.float16)
        x[0, j] = 1
        y = O.linear_int8(q, s, x)
        np.testing.assert_array_equal(y[0], q[:, j].astype(np.float64) * float(s))


# ---------------------------------------------------------------- INT4 -------

def _one_group_row(values):
    w = np.zeros((1, 128), np.float32)
    w[0, : len(values)] = values
    return w


def test_int4_ties_round_half_even():
    rows = [ln.split() for ln in read_golden("int4_ties.txt")]
    W = _one_group_row([float(r[0]) for r in rows])
    want = np.array([int(r[1]) for r in rows], np.int8)
    perm = O.global_perm(128, np.zeros(0, np.int64))
    codes, scales, w_out = O.quantize_int4o(W, perm, 0)
    assert scales.shape == (1, 1) and scales[0, 0] == np.float16(2.0 ** -8)
    assert w_out.shape == (1, 0)
    np.testing.assert_array_equal(codes[0, : len(want)], want)
    assert not codes[0, len(want):].any()


@pytest.mark.parametrize("K,n_out", [(300, 3), (257, 0), (1000, 10)])
def test_int4_closed_form_bound(K, n_out):
    rng = np.random.default_rng(K)
    W = (rng.standard_normal((23, K)) * 0.02).astype(np.float32)
    perm = O.global_perm(K, rng.choice(K, n_out, replace=False))
    codes, scales, w_out = O.quantize_int4o(W, perm, n_out)
    geo = O.int4o_geometry(K, n_out)
    Wp = W[:, perm].astype(np.float64)
    s = np.repeat(scales.astype(np.float64), 128, axis=1)[:, : geo["K_bg"]]
    c = codes[:, : geo["K_bg"]].astype(np.float64)
    err = np.abs(Wp[:, : geo["K_bg"]] - c * s)
    assert np.all(err <= s * (0.5 + 8 * 2.0 ** -23))
    assert codes.min() >= -7 and codes.max() <= 7            # nibble 0x8 never used
    # the largest magnitude of every group maps to +-7
    for g in range(geo["G"]):
        lo, hi = 128 * g, min(128 * g + 128, geo["K_bg"])
        blk = np.abs(Wp[:, lo:hi])
        arg = blk.argmax(axis=1)
        assert np.all(np.abs(codes[np.arange(23), lo + arg]) == 7)
    assert not codes[:, geo["K_bg"]:].any()                    # zero padding


def test_int4_tiny_group_clamps_and_zero_group():
    # a group max of 5e-7 gives a subnormal fp16 scale of one ulp (2^-24), so
    # W/scale exceeds 7.5 and the clamp decides the code
    W = np.zeros((2, 128), np.float32)
    W[0, 0] = 5e-7
    W[0, 1] = -5e-7
    perm = O.global_perm(128, np.zeros(0, np.int64))
    codes, scales, _ = O.quantize_int4o(W, perm, 0)
    assert scales[0, 0] == np.float16(2.0 ** -24)
    assert codes[0, 0] == 7 and codes[0, 1] == -7
    assert scales[1, 0] == 0 and not codes[1].any()


def test_int4_scale_overflow_raises():
    W = np.zeros((1, 128), np.float32)
    W[0, 0] = 1e6
    with pytest.raises(ValueError):
        O.quantize_int4o(W, O.global_perm(128, np.zeros(0, np.int64)), 0)


def test_nibble_pack_worked_example():
    lines = dict(ln.split(":", 1) for ln in read_golden("nibble_pack_example.txt"))
    codes = np.array([[int(v) for v in lines["codes"].split()]], np.int8)
    want = np.array([[int(v, 16) for v in lines["bytes"].split()]], np.uint8)
    np.testing.assert_array_equal(O.pack_int4(codes), want)
    np.testing.assert_array_equal(O.unpack_int4(want), codes)


def test_nibble_pack_all_pairs_roundtrip():
    vals = np.arange(-7, 8)
    pairs = np.array([[a, b] for a in vals for b in vals], np.int8)      # 225 pairs
    packed = O.pack_int4(pairs)
    assert packed.shape == (225, 1)
    assert len(np.unique(packed)) == 225                                  # injective
    np.testing.assert_array_equal(O.unpack_int4(packed), pairs)
    assert 0x08 not in (packed & 0xF) and 0x80 not in (packed & 0xF0)   # -8 never appears
    # byte value == low nibble + 16 * high nibble, nibble = code mod 16
    assert packed[vals.tolist().index(1) * 15 + vals.tolist().index(0), 0] == 0x01
    assert packed[vals.tolist().index(0) * 15 + vals.tolist().index(1), 0] == 0x10
    # two's complement: nibble 0x8 reads as -8 and 0xF as -1
    np.testing.assert_array_equal(O.unpack_int4(np.array([[0x8F]], np.uint8)), [[-1, -8]])


def test_outliers_kept_exactly_and_reconstruction():
    rng = np.random.default_rng(7)
    K = 450
    W = (rng.standard_normal((9, K)) * 0.02).astype(np.float32)
    O_set = np.sort(rng.choice(K, 5, replace=False))
    W[:, O_set] *= 10
    perm = O.global_perm(K, O_set)
    codes, scales, w_out = O.quantize_int4o(W, perm, 5)
    np.testing.assert_array_equal(w_out.view(np.uint16), W[:, O_set].astype(np.float16).view(np.uint16))
    R = O.reconstruct_int4o(codes, scales, w_out, perm)
    np.testing.assert_array_equal(R[:, O_set], W[:, O_set].astype(np.float16).astype(np.float64))


def test_perm_is_bijection_and_split_inverts():
    rng = np.random.default_rng(8)
    K = 333
    outs = rng.choice(K, 4, replace=False)
    perm = O.global_perm(K, outs)
    assert sorted(perm.tolist()) == list(range(K))
    assert set(perm[-4:].tolist()) == set(outs.tolist())
    assert np.all(np.diff(perm[:-4]) > 0) and np.all(np.diff(perm[-4:]) > 0)
    x = rng.standard_normal((3, K)).astype(np.float16)
    x_bg, x_out = O.permute_split(x, perm, 4)
    geo = O.int4o_geometry(K, 4)
    xp = np.concatenate([x_bg[:, : geo["K_bg"]], x_out], axis=1)
    np.testing.assert_array_equal(xp[:, np.argsort(perm)], x)
    assert not x_bg[:, geo["K_bg"]:].any()


def test_topk_ties_lower_index():
    g = dict(ln.split(":", 1) for ln in read_golden("topk_ties.txt"))
    scores = np.array([float(v) for v in g["scores"].split()])
    got = O.select_outliers(scores, int(g["n_out"]))
    np.testing.assert_array_equal(got, [int(v) for v in g["expected"].split()])


def test_topk_matches_brute_force_tiny():
    rng = np.random.default_rng(9)
    from itertools import combinations
    for _ in range(20):
        K = int(rng.integers(2, 9))
        n = int(rng.integers(0, K + 1))
        scores = rng.integers(0, 4, K).astype(np.float64)      # many ties
        best = None
        for c in combinations(range(K), n):
            key = (-sum(scores[list(c)]), list(c))             # largest sum, then lexicographically lowest
            if best is None or key < best:
                best = key
        np.testing.assert_array_equal(O.select_outliers(scores, n), best[1])


def test_planted_channels_recovered():
    spec = synth.small_stack_spec(2, layers=2)
    for space in synth.SPACES:
        K = spec.space_width(space)
        colabs = np.zeros(K)
        for layer in range(spec.layers):
            for lin in spec.linears():
                if lin.space == space:
                    colabs += O.column_abs_sum(synth.weight(spec, layer, lin))
        sc = O.outlier_scores(colabs, synth.profile(spec, space))
        got = O.select_outliers(sc, O.n_outliers(K))
        np.testing.assert_array_equal(got, synth.planted_set(spec, space))


def test_scores_use_magnitudes_of_both_factors():
    # channel 1 has the largest signed sums but the smallest magnitudes
    W = np.array([[1.0, 0.1, -3.0], [1.0, 0.1, 3.0]], np.float32)
    xprof = np.array([[1, 1, -1], [1, 1, 1]], np.float16)
    sc = O.outlier_scores(O.column_abs_sum(W), xprof)
    np.testing.assert_array_equal(O.select_outliers(sc, 1), [2])


def _grid_int4o(rng, N, K, n_out):
    """A weight matrix that the outlier-INT4 encoding represents exactly:
    background = code * 2^-e per (row, group) with a +-7 in every group,
    outlier columns = fp16 values.  Returns (W, outlier set)."""
    geo = O.int4o_geometry(K, n_out)
    outs = np.sort(rng.choice(K, n_out, replace=False)) if n_out else np.zeros(0, np.int64)
    perm = O.global_perm(K, outs)
    Wp = np.zeros((N, K), np.float32)
    for g in range(geo["G"]):
        lo, hi = 128 * g, min(128 * g + 128, geo["K_bg"])
        c = rng.integers(-7, 8, size=(N, hi - lo)).astype(np.float32)
        c[:, 0] = rng.choice([-7, 7], N)
        e = rng.integers(5, 12, size=(N, 1))
        Wp[:, lo:hi] = c * (2.0 ** -e).astype(np.float32)
    Wp[:, geo["K_bg"]:] = (rng.standard_normal((N, n_out)) * 0.3).astype(np.float16)
    W = np.empty_like(Wp)
    W[:, perm] = Wp
    return W, outs, perm


@pytest.mark.parametrize("N", [1, 3, 17])
@pytest.mark.parametrize("K", [2, 130, 257])
@pytest.mark.parametrize("b", [1, 8])
def test_int4o_on_grid_product_is_matmul(N, K, b):
    rng = np.random.default_rng(N * 1000 + K * 10 + b)
    for n_out in sorted({0, O.n_outliers(K)}):
        W, outs, perm = _grid_int4o(rng, N, K, n_out)
        codes, scales, w_out = O.quantize_int4o(W, perm, n_out)
        np.testing.assert_array_equal(O.reconstruct_int4o(codes, scales, w_out, perm), W.astype(np.float64))
        x = rng.standard_normal((b, K)).astype(np.float16)
        x_bg, x_out = O.permute_split(x, perm, n_out)
        y = O.linear_int4o(codes, scales, w_out, x_bg, x_out)
        ref = x.astype(np.float64) @ W.astype(np.float64).T
        np.testing.assert_allclose(y, ref, rtol=1e-13, atol=1e-13)


def test_int4o_product_exact_integer():
    rng = np.random.default_rng(11)
    K, N, n_out = 300, 4, 3
    W = (rng.standard_normal((N, K)) * 0.02).astype(np.float32)
    outs = np.sort(rng.choice(K, n_out, replace=False))
    perm = O.global_perm(K, outs)
    codes, scales, w_out = O.quantize_int4o(W, perm, n_out)
    x = rng.standard_normal((1, K)).astype(np.float16)
    x_bg, x_out = O.permute_split(x, perm, n_out)
    y = O.linear_int4o(codes, scales, w_out, x_bg, x_out)
    # exact: every fp16 is an integer multiple of 2^-24
    xi = [int(v) for v in (x_bg[0].astype(np.float64) * 2 ** 24)]
    xo = [int(v) for v in (x_out[0].astype(np.float64) * 2 ** 24)]
    for n in range(N):
        acc = Fraction(0)
        for g in range(scales.shape[1]):
            part = sum(int(codes[n, k]) * xi[k] for k in range(128 * g, 128 * g + 128))
            acc += Fraction(float(scales[n, g])) * part
        wo = [Fraction(float(v)) for v in w_out[n]]
        acc += sum(w * v for w, v in zip(wo, xo))
        exact = acc / 2 ** 24
        assert abs(Fraction(float(y[0, n])) - exact) <= abs(exact) * Fraction(1, 10 ** 14) + Fraction(1, 10 ** 18)


# ------------------------------------------------------ INT8 vocabulary ----

def test_embed_lookup_hand_table():
    """Single-entry lookups derived by hand, including a double rounding."""
    for ln in read_golden("embed_int8_lookup.txt"):
        c, m, e, bits = ln.split()[:4]
        s = np.float32(int(m) * 2.0 ** int(e))
        assert float(s) == int(m) * 2.0 ** int(e)
        y = O.embed_int8(np.array([[int(c)]], np.int8), s, [0])
        assert y.dtype == np.float16 and y.shape == (1, 1)
        assert int(y.view(np.uint16)[0, 0]) == int(bits, 16), ln


def test_embed_lookup_rows_ids_and_bound():
    """Rows follow the ids (repeats allowed); ids outside the table give zero
    rows; every entry is within half an fp16 ulp (plus half an fp32 ulp of the
    product) of the exact code * scale."""
    rng = np.random.default_rng(11)
    V, H = 37, 50
    E = rng.standard_normal((V, H)).astype(np.float32)
    q, s = O.quantize_int8(E)
    ids = np.array([5, 0, V - 1, 5, -1, V, 2 ** 31 - 1, 12], np.int64)
    y = O.embed_int8(q, s, ids)
    assert y.shape == (ids.size, H) and y.dtype == np.float16
    for r, t in enumerate(ids):
        if not 0 <= t < V:
            assert not y[r].view(np.uint16).any()
            continue
        exact = np.array([Fraction(int(c)) * Fraction(float(s)) for c in q[t]], dtype=object)
        for j in range(H):
            v = Fraction(float(y[r, j]))
            ulp16 = Fraction(float(np.spacing(np.float16(abs(float(exact[j]))))))
            ulp32 = Fraction(float(np.spacing(np.float32(abs(float(exact[j]))))))
            assert abs(v - exact[j]) <= ulp16 / 2 + ulp32 / 2
    np.testing.assert_array_equal(y[0], y[3])
    assert O.embed_int8(q, s, np.array([], np.int64)).shape == (0, H)


def test_embed_lookup_power_of_two_scale_is_exact():
    """With scale 2^-7 every code * scale is exact in fp16, so the lookup is the
    dequantised row itself."""
    rng = np.random.default_rng(12)
    q = rng.integers(-127, 128, size=(9, 70)).astype(np.int8)
    y = O.embed_int8(q, np.float32(2.0 ** -7), np.arange(9))
    np.testing.assert_array_equal(y.astype(np.float64), q.astype(np.float64) / 128.0)


# ------------------------------------------------------------ byte totals ----

def _golden_totals():
    return {ln.split()[0]: (float(ln.split()[1]), float(ln.split()[2])) for ln in read_golden("page_byte_totals.txt")}


def test_int8_pool_matches_page_total():
    val, tol = _golden_totals()["int8_pool_gib"]
    spec = synth.stack_spec(3)
    codes = spec.layers * sum(O.algorithmic_bytes_int8(l.N, l.K, 0) - 4 for l in spec.linears())
    assert abs(codes / 2 ** 30 - val) <= tol


def test_int4o_3b_footprint_matches_page_total():
    val, tol = _golden_totals()["int4o_3b_gb"]
    spec = synth.stack_spec(2)
    lin = spec.layers * sum(O.algorithmic_bytes_int4o(l.N, l.K, 0) for l in spec.linears())
    emb = 128256 * 3072
    assert abs((lin + emb) / 1e9 - val) <= tol


def test_normwise_error_helper():
    assert O.normwise_rel_err([1.0, 2.0], [1.0, 2.0]) == 0
    assert O.normwise_rel_err([1.0, 2.002], [1.0, 2.0]) == pytest.approx(1e-3)


def test_space_column_sum_is_the_stacked_column_sum():
    """Summing column_abs_sum over the linears of a space equals the column
    sums of the linears stacked along N (integer-valued weights: exact)."""
    rng = np.random.default_rng(11)
    Ws = [rng.integers(-9, 10, (n, 13)).astype(np.float32) for n in (1, 4, 7)]
    np.testing.assert_array_equal(O.space_column_abs_sum(Ws), O.column_abs_sum(np.concatenate(Ws)))
    # a column whose signed sum cancels still counts its magnitude
    W = np.array([[3, -1], [-3, 1]], np.float32)
    np.testing.assert_array_equal(O.space_column_abs_sum([W, -W]), [12, 4])


def test_absolute_term_sums_brute_force_and_special_cases():
    """linear_*_abs against explicit loops over |w x| on tiny cases; for
    non-negative codes, scales and activations they equal the products
    themselves; flipping the sign of any activation leaves them unchanged."""
    rng = np.random.default_rng(5)
    # INT8
    q = rng.integers(-127, 128, (3, 5)).astype(np.int8)
    s = np.float32(0.03125)
    x = rng.standard_normal((2, 5)).astype(np.float16)
    want = np.zeros((2, 3))
    for b in range(2):
        for n in range(3):
            want[b, n] = sum(abs(float(q[n, k]) * float(s) * float(x[b, k])) for k in range(5))
    np.testing.assert_allclose(O.linear_int8_abs(q, s, x), want, rtol=1e-15)
    qp = np.abs(q).astype(np.int8)
    np.testing.assert_array_equal(O.linear_int8_abs(qp, s, np.abs(x)), O.linear_int8(qp, s, np.abs(x)))
    flip = x * np.where(rng.random(5) < 0.5, -1, 1).astype(np.float16)
    np.testing.assert_array_equal(O.linear_int8_abs(q, s, flip), O.linear_int8_abs(q, s, x))
    # INT4O, K = 130 with 2 outliers: 128 background channels, one group
    K, n_out = 130, 2
    perm = O.global_perm(K, np.array([7, 99]))
    W = rng.standard_normal((3, K)).astype(np.float32)
    c, sc, wo = O.quantize_int4o(W, perm, n_out)
    xf = rng.standard_normal((1, K)).astype(np.float16)
    x_bg, x_out = O.permute_split(xf, perm, n_out)
    got = O.linear_int4o_abs(c, sc, wo, x_bg, x_out)
    for n in range(3):
        t = sum(abs(float(c[n, k]) * float(sc[n, k // 128]) * float(x_bg[0, k])) for k in range(c.shape[1]))
        t += sum(abs(float(wo[n, i]) * float(x_out[0, i])) for i in range(n_out))
        assert got[0, n] == pytest.approx(t, rel=1e-14)
    cp, scp, wop = np.abs(c).astype(np.int8), np.abs(sc), np.abs(wo)
    np.testing.assert_allclose(O.linear_int4o_abs(cp, scp, wop, np.abs(x_bg), np.abs(x_out)),
                               O.linear_int4o(cp, scp, wop, np.abs(x_bg), np.abs(x_out)), rtol=1e-15)
    # always an upper bound of the product's magnitude
    assert np.all(got >= np.abs(O.linear_int4o(c, sc, wo, x_bg, x_out)) * (1 - 1e-15))


def test_componentwise_error_helper():
    y = np.array([[1.0, 2.0, 0.0, 5.0]])
    ref = np.array([[1.5, 2.0, 0.0, 4.0]])
    absref = np.array([[10.0, 2.0, 0.0, 100.0]])
    assert O.componentwise_rel_err(y, ref, absref) == pytest.approx(0.05)
    assert O.componentwise_rel_err(ref, ref, absref) == 0.0
    assert O.componentwise_rel_err(y[:, 2:3], ref[:, 2:3], absref[:, 2:3]) == 0.0   # no terms at all
