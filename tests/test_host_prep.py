"""Host-side library functions against the oracle, bit for bit (CPU only).

The library's quantisers, outlier selection, packing and layout transforms run
on the host, so they are checked here without a GPU; the ABI checks confirm the
built library exports every function the header declares.
"""
import os
import sys
import re

import numpy as np
import pytest

import oracle as O
import synth
from weight_only_quantized_quantize_amd import woq

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module", autouse=True)
def _lib():
    if not os.path.exists(woq.LIB_PATH):
        pytest.fail("libwoq.so is not built: run `python -m weight_only_quantized_quantize_amd.build`")
    woq.lib()


def header_functions():
    text = open(os.path.join(ROOT, "include", "woq.h")).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(woq_[a-z0-9_]+)\s*\(", text)))


def test_library_exports_every_header_function():
    names = header_functions()
    assert len(names) >= 18
    lib = woq.lib()
    missing = [n for n in names if not hasattr(lib, n)]
    assert not missing, missing
    assert set(names) == set(woq.EXPORTS), set(names) ^ set(woq.EXPORTS)
    assert lib.woq_abi_version() == 1
    assert lib.woq_strerror(-1) == b"invalid argument"


# --------------------------------------------------------------------- INT8

def test_quantize_int8_config1_bit_exact():
    W, _ = synth.config1_inputs()
    q, s = woq.woq_quantize_int8(W)
    qo, so = O.quantize_int8(W)
    assert s.view(np.uint32) == so.view(np.uint32)
    np.testing.assert_array_equal(q, qo)
    # the config-1 weights contain exact .5 ties, which the two must agree on
    t = W / so
    assert np.count_nonzero(np.abs(t - np.trunc(t)) == 0.5) > 0


def test_quantize_int8_ties_and_edges():
    W = np.array([[0.9921875, 0.01171875, -0.01953125, 0.02734375, 0.0]], np.float32)
    q, s = woq.woq_quantize_int8(W)
    np.testing.assert_array_equal(q, O.quantize_int8(W)[0])
    q, s = woq.woq_quantize_int8(np.zeros((3, 5), np.float32))
    assert s == 0 and not q.any()
    q, s = woq.woq_quantize_int8(np.array([[2.0 ** -149]], np.float32))
    assert s == 0 and not q.any()
    with pytest.raises(woq.WoqError) as e:
        woq.woq_quantize_int8(np.array([[1.0, np.inf]], np.float32))
    assert e.value.status == woq.WOQ_ERANGE


@pytest.mark.parametrize("N,K", [(1, 1), (7, 33), (130, 77)])
def test_quantize_int8_random_shapes(N, K):
    rng = np.random.default_rng(N * K)
    W = (rng.standard_normal((N, K)) * rng.uniform(1e-3, 10)).astype(np.float32)
    q, s = woq.woq_quantize_int8(W)
    qo, so = O.quantize_int8(W)
    assert s == so
    np.testing.assert_array_equal(q, qo)


def test_int8_layout_roundtrip_and_padding():
    rng = np.random.default_rng(1)
    q = rng.integers(-127, 128, size=(6, 70)).astype(np.int8)
    dev = woq.woq_layout_int8(q)
    assert dev.size == 8 * 128
    d = dev.reshape(8, 128)
    np.testing.assert_array_equal(d[:6, :70].astype(np.int16) - 128, q)
    assert np.all(d[:, 70:] == 128) and np.all(d[6:] == 128)
    np.testing.assert_array_equal(woq.woq_layout_int8_inverse(dev, 6, 70), q)


# -------------------------------------------------------------------- INT4O

def _colabs_lib(spec, space):
    K = spec.space_width(space)
    cs = np.zeros(K)
    for layer in range(spec.layers):
        for lin in spec.linears():
            if lin.space == space:
                woq.woq_colabs_accumulate(synth.weight(spec, layer, lin), cs)
    return cs


def test_outlier_select_matches_oracle_planted():
    spec = synth.small_stack_spec(2, layers=2)
    for space in synth.SPACES:
        K = spec.space_width(space)
        cs = _colabs_lib(spec, space)
        co = np.zeros(K)
        for layer in range(spec.layers):
            for lin in spec.linears():
                if lin.space == space:
                    co += O.column_abs_sum(synth.weight(spec, layer, lin))
        np.testing.assert_allclose(cs, co, rtol=1e-14)
        xprof = synth.profile(spec, space)
        perm = woq.woq_outlier_select(cs, xprof)
        po = O.global_perm(K, O.select_outliers(O.outlier_scores(co, xprof), O.n_outliers(K)))
        np.testing.assert_array_equal(perm, po)
        np.testing.assert_array_equal(np.sort(perm[-O.n_outliers(K):]), synth.planted_set(spec, space))


@pytest.mark.parametrize("cfg,layers", [(2, 2), (4, 1)])
def test_outlier_perm_full_width_spaces_match_oracle(cfg, layers):
    """The single-call selection (woq_outlier_perm over every linear of the
    first layers that reads a space, full widths of the 3B- and 70B-shaped
    stacks) is bit-identical to the oracle's selection over the same linears;
    the per-linear sums form (woq_outlier_perm_sums) gives the same table."""
    spec = synth.stack_spec(cfg)
    for space in synth.SPACES:
        K = spec.space_width(space)
        Ws = [synth.weight(spec, layer, lin) for layer in range(layers) for lin in spec.linears()
              if lin.space == space]
        xprof = synth.profile(spec, space)
        perm = woq.woq_outlier_perm(Ws, xprof)
        parts = [woq.woq_colabs_accumulate(W, np.zeros(K)) for W in Ws]
        np.testing.assert_array_equal(woq.woq_outlier_perm_sums(parts, xprof), perm)
        co = O.space_column_abs_sum(Ws)
        del Ws, parts
        po = O.global_perm(K, O.select_outliers(O.outlier_scores(co, xprof), O.n_outliers(K)))
        np.testing.assert_array_equal(perm, po, err_msg=f"cfg {cfg} space {space}")
        np.testing.assert_array_equal(np.sort(perm[-O.n_outliers(K):]), synth.planted_set(spec, space))


def test_outlier_perm_orders_and_errors():
    """Hand case: the sums of two linears decide the selection (either alone
    would pick another channel); argument errors are refused."""
    K = 4
    W1 = np.array([[9, 0, 1, 0]], np.float32)          # channel 0 alone would win
    W2 = np.array([[0, 5, 1, 0], [0, 5, 1, 0]], np.float32)
    xprof = np.array([[1, 1, 2, 1]], np.float16)       # channel 2 scores 2 * 2 = 4 x profile
    # column sums: [9, 10, 3, 0]; scores: [9, 10, 6, 0] -> top-1 is channel 1
    perm = woq.woq_outlier_perm([W1, W2], xprof, 1)
    np.testing.assert_array_equal(perm, [0, 2, 3, 1])
    assert woq.woq_outlier_perm([W1], xprof, 1)[-1] == 0
    parts = [woq.woq_colabs_accumulate(W, np.zeros(K)) for W in (W1, W2)]
    np.testing.assert_array_equal(woq.woq_outlier_perm_sums(parts, xprof, 1), perm)
    L = woq.lib()
    p = np.empty(K, np.int32)
    xp = np.ascontiguousarray(xprof).view(np.uint16)
    assert L.woq_outlier_perm(None, None, 0, K, xp.ctypes.data, 1, 1, p.ctypes.data) == woq.WOQ_EINVAL
    assert L.woq_outlier_perm_sums(None, 0, K, xp.ctypes.data, 1, 1, p.ctypes.data) == woq.WOQ_EINVAL
    bad = np.array([np.nan, 1, 1, 1], np.float64)
    with pytest.raises(woq.WoqError) as e:
        woq.woq_outlier_perm_sums([bad], xprof, 1)
    assert e.value.status == woq.WOQ_ERANGE


def test_outlier_select_ties_and_all_or_none():
    cs = np.array([3, 5, 5, 1, 5, 0], np.float64)
    xprof = np.ones((2, 6), np.float16)
    perm = woq.woq_outlier_select(cs, xprof, 2)
    np.testing.assert_array_equal(perm, [0, 3, 4, 5, 1, 2])
    np.testing.assert_array_equal(woq.woq_outlier_select(cs, xprof, 0), np.arange(6))
    np.testing.assert_array_equal(woq.woq_outlier_select(cs, xprof, 6), np.arange(6))


@pytest.mark.parametrize("N,K,n_out", [(5, 300, 3), (4, 257, 0), (9, 1000, -1), (3, 8, 8), (2, 129, 1)])
def test_quantize_int4o_bit_exact(N, K, n_out):
    rng = np.random.default_rng(N + K)
    W = (rng.standard_normal((N, K)) * 0.02).astype(np.float32)
    n = O.n_outliers(K) if n_out < 0 else n_out
    outs = np.sort(rng.choice(K, n, replace=False))
    W[:, outs] *= 10
    W[0, : K // 3] = 0                      # rows/groups of zeros: scale 0
    if N > 1:
        W[1, :5] = 5e-7                     # subnormal scale: the clamp decides
    perm = O.global_perm(K, outs)
    packed, scales, w_out = woq.woq_quantize_int4o(W, perm, n)
    codes_o, scales_o, w_out_o = O.quantize_int4o(W, perm, n)
    np.testing.assert_array_equal(packed, O.pack_int4(codes_o))
    np.testing.assert_array_equal(scales.view(np.uint16), scales_o.view(np.uint16))
    np.testing.assert_array_equal(w_out.view(np.uint16), w_out_o.view(np.uint16))
    np.testing.assert_array_equal(woq.woq_unpack_int4(packed), codes_o)


def test_quantize_int4o_config2_layer_bit_exact():
    spec = synth.stack_spec(2)
    space = "h"
    K = spec.space_width(space)
    S = synth.planted_set(spec, space)
    perm = O.global_perm(K, S)          # the planted set is what selection recovers
    W = synth.weight(spec, 0, "k")
    packed, scales, w_out = woq.woq_quantize_int4o(W, perm)
    codes_o, scales_o, w_out_o = O.quantize_int4o(W, perm, O.n_outliers(K))
    np.testing.assert_array_equal(packed, O.pack_int4(codes_o))
    np.testing.assert_array_equal(scales.view(np.uint16), scales_o.view(np.uint16))
    np.testing.assert_array_equal(w_out.view(np.uint16), w_out_o.view(np.uint16))


def test_quantize_int4o_errors():
    W = np.zeros((2, 130), np.float32)
    perm = np.arange(130, dtype=np.int32)
    bad = perm.copy()
    bad[3] = 4
    with pytest.raises(woq.WoqError) as e:
        woq.woq_quantize_int4o(W, bad, 2)
    assert e.value.status == woq.WOQ_EINVAL
    W[0, 0] = 1e6
    with pytest.raises(woq.WoqError) as e:
        woq.woq_quantize_int4o(W, perm, 2)
    assert e.value.status == woq.WOQ_ERANGE
    W[0, 0] = np.nan
    with pytest.raises(woq.WoqError) as e:
        woq.woq_quantize_int4o(W, perm, 2)
    assert e.value.status == woq.WOQ_ERANGE


@pytest.mark.parametrize("N,K,n_out", [(6, 300, 3), (5, 1000, -1), (4, 129, 1), (3, 16, 16)])
def test_int4o_layout_roundtrip(N, K, n_out):
    rng = np.random.default_rng(K)
    W = (rng.standard_normal((N, K)) * 0.02).astype(np.float32)
    g = woq.woq_int4o_geometry(K, n_out)
    perm = O.global_perm(K, np.sort(rng.choice(K, g.n_out, replace=False)))
    packed, scales, w_out = woq.woq_quantize_int4o(W, perm, g.n_out)
    dc, ds, dw = woq.woq_layout_int4o(packed, scales, w_out, g)
    N16 = -(-N // 16) * 16
    assert dc.size == N16 * 64 * g.G4 and ds.size == N16 * g.G4 and dw.size == N16 * g.n_out8
    p2, s2, w2 = woq.woq_layout_int4o_inverse(dc, ds, dw, N, g)
    np.testing.assert_array_equal(p2, packed)
    np.testing.assert_array_equal(s2.view(np.uint16), scales.view(np.uint16))
    np.testing.assert_array_equal(w2.view(np.uint16), w_out.view(np.uint16))


def test_int4o_device_nibble_placement():
    """The device chunk of channels 0..31 holds code+8 at the documented nibbles."""
    g = woq.woq_int4o_geometry(128, 0)
    codes = np.zeros((1, 128), np.int8)
    codes[0, :32] = (np.arange(32) % 15) - 7
    packed = O.pack_int4(codes)
    dc, _, _ = woq.woq_layout_int4o(packed, np.ones((1, 1), np.float16), np.zeros((1, 0), np.float16), g)
    dw = dc[:16].view(np.uint32)
    lo_pos, hi_pos = [0, 4, 2, 6], [1, 5, 3, 7]
    for c in range(32):
        P, t = divmod(c, 16)
        e, j = (t // 4, t % 4) if t < 8 else ((t - 8) // 4, (t - 8) % 4)
        pos = (lo_pos if t < 8 else hi_pos)[j]
        nib = (int(dw[2 * P + e]) >> (4 * pos)) & 0xF
        assert nib == codes[0, c] + 8, c
    assert np.all(dc[16:] == 0x88)          # rows 1..15 and the other chunks: code 0


def test_int4o_device_tile_placement():
    """Tiles of 16 rows: chunk (row r, group g, chunk c) at byte
    ((r // 16 * G4 + g) * 4 + c) * 256 + (r % 16) * 16; scale (r, g) at
    (r // 16 * G4 + g) * 16 + r % 16; outlier weight (r, i) in the 8-wide chunk
    ((r // 16 * no8 + i // 8) * 16 + r % 16) at element i % 8."""
    N, K, n_out = 20, 300, 3
    g = woq.woq_int4o_geometry(K, n_out)
    assert (g.G, g.G4, g.n_out8) == (3, 4, 8)
    codes = np.zeros((N, g.K_pad), np.int8)
    r, gi, c, t = 17, 1, 2, 5                  # channel 128*1 + 32*2 + 5 of row 17
    codes[r, 128 * gi + 32 * c + t] = -6
    packed = O.pack_int4(codes)
    scales = np.zeros((N, g.G), np.float16)
    scales[r, 2] = np.float16(0.5)
    w_out = np.zeros((N, n_out), np.float16)
    w_out[r, 2] = np.float16(-3.0)
    dc, ds, dw = woq.woq_layout_int4o(packed, scales, w_out, g)
    off = ((r // 16 * g.G4 + gi) * 4 + c) * 256 + (r % 16) * 16
    chunk = dc[off:off + 16].view(np.uint32)
    e, j = (t // 4, t % 4)
    assert (int(chunk[e]) >> (4 * [0, 4, 2, 6][j])) & 0xF == -6 + 8
    others = np.delete(dc, np.arange(off, off + 16))
    assert np.all(others == 0x88)
    assert ds[(r // 16 * g.G4 + 2) * 16 + r % 16] == np.float16(0.5).view(np.uint16)
    assert np.count_nonzero(ds) == 1
    no8 = g.n_out8 // 8
    assert dw[((r // 16 * no8 + 0) * 16 + r % 16) * 8 + 2] == np.float16(-3.0).view(np.uint16)
    assert np.count_nonzero(dw) == 1


def test_geometry_of_configs():
    for K, n_out, K_bg, G, K_pad in [(3072, 31, 3041, 24, 3072), (8192, 82, 8110, 64, 8192),
                                     (28672, 287, 28385, 222, 28416)]:
        g = woq.woq_int4o_geometry(K)
        assert (g.n_out, g.K_bg, g.G, g.K_pad) == (n_out, K_bg, G, K_pad)
        geo = O.int4o_geometry(K)
        assert (geo["n_out"], geo["K_bg"], geo["G"], geo["K_pad"]) == (n_out, K_bg, G, K_pad)
    with pytest.raises(woq.WoqError):
        woq.woq_int4o_geometry(0)
    with pytest.raises(woq.WoqError):
        woq.woq_int4o_geometry(10, 11)


def test_device_entry_points_reject_bad_arguments_without_launching():
    """Argument checks run before any HIP call, so they work without a GPU."""
    lib = woq.lib()
    g = woq.woq_int4o_geometry(256, 2)
    w = woq.Int4oW()
    w.N, w.geom = 8, g
    w.codes, w.scales, w.w_out = 16, 16, 16
    # b out of range
    assert lib.woq_qgemv_int4o(w, 16, 65, 16, 8, None) == woq.WOQ_EINVAL
    # misaligned activations
    assert lib.woq_qgemv_int4o(w, 18, 1, 16, 8, None) == woq.WOQ_EALIGN
    # ldy < N
    assert lib.woq_qgemv_int4o(w, 16, 1, 16, 4, None) == woq.WOQ_EINVAL
    # b == 0 is a no-op
    assert lib.woq_qgemv_int4o(w, 16, 0, 16, 8, None) == woq.WOQ_OK
    # a geometry that does not match its own K / n_out
    bad = woq.Int4oW.from_buffer_copy(w)
    bad.geom.G4 = 99
    assert lib.woq_qgemv_int4o(bad, 16, 1, 16, 8, None) == woq.WOQ_EINVAL
    w8 = woq.Int8W()
    w8.codes, w8.N, w8.K, w8.nseg = 16, 8, 64, 1
    w8.seg_end[0] = 7                       # segments must end at N
    assert lib.woq_qgemv_int8(w8, 16, 64, 1, 16, 8, None) == woq.WOQ_EINVAL
    w8.seg_end[0] = 8
    assert lib.woq_qgemv_int8(w8, 16, 60, 1, 16, 8, None) == woq.WOQ_EINVAL   # ldx < K
    assert lib.woq_qgemv_int8(w8, 16, 68, 1, 16, 8, None) == woq.WOQ_EALIGN   # ldx % 8
    assert lib.woq_qgemv_int8(w8, 16, 64, 9, 16, 8, None) == woq.WOQ_EINVAL   # b > 8
    assert lib.woq_permute_x(16, 100, 16, 1, g, 16, None) == woq.WOQ_EINVAL    # ldx < K
    # the matrix-core one-launch form: argument checks before the support
    # check and before any HIP call
    assert lib.woq_qgemm_int4o_x(w, 16, 200, 16, 1, 16, 8, None) == woq.WOQ_EINVAL     # ldx < K
    assert lib.woq_qgemm_int4o_x(w, 16, 256, 16, -1, 16, 8, None) == woq.WOQ_EINVAL    # b < 0
    assert lib.woq_qgemm_int4o_x(w, 16, 256, 16, 1, 16, 4, None) == woq.WOQ_EINVAL     # ldy < N
    assert lib.woq_qgemm_int4o_x(w, 16, 256, 16, 0, 16, 8, None) == woq.WOQ_OK         # b == 0: no-op
    assert lib.woq_qgemm_int4o_x(w, 18, 256, 16, 1, 16, 8, None) == woq.WOQ_EALIGN     # x misaligned
    assert lib.woq_qgemm_int4o_x(w, 16, 260, 16, 1, 16, 8, None) == woq.WOQ_EALIGN     # ldx % 8
    assert lib.woq_qgemm_int4o_x(w, 16, 256, 24, 1, 16, 8, None) == woq.WOQ_EALIGN     # pos misaligned
    assert lib.woq_qgemm_int4o_x(w, None, 256, 16, 1, 16, 8, None) == woq.WOQ_EINVAL   # no x
    assert lib.woq_qgemm_int4o_x(bad, 16, 256, 16, 1, 16, 8, None) == woq.WOQ_EINVAL   # bad geometry
    # rows under 64 groups and batches above 8 are never supported
    assert lib.woq_qgemm_int4o_x(w, 16, 256, 16, 1, 16, 8, None) == woq.WOQ_EUNSUPPORTED
    assert not woq.woq_qgemm_int4o_x_supported(woq.woq_int4o_geometry(3072), 4096, 8)
    assert not woq.woq_qgemm_int4o_x_supported(woq.woq_int4o_geometry(8192), 8192, 9)
    assert not woq.woq_qgemm_int4o_x_supported(woq.woq_int4o_geometry(8192), 0, 8)


# -------------------------------------------------------------------- pager

def test_pager_create_validates_before_allocating():
    """Argument checks of woq_pager_create run before any device call, so
    they are exercised without a GPU."""
    import ctypes
    lib = woq.lib()
    pool = np.zeros(4096, np.uint8)
    N, K = 8, 64
    need = lib.woq_int8_dev_bytes(N, K)

    def create(code_offset, layer_bytes, n=N, nseg=1, seg_end=None, max_b=1):
        st = woq.PagerStep()
        st.code_offset = code_offset
        st.w.N, st.w.K, st.w.nseg = n, K, nseg
        st.w.seg_end[0] = n if seg_end is None else seg_end
        st.w.seg_scale[0] = 1.0
        steps = (woq.PagerStep * 1)(st)
        off = (ctypes.c_int64 * 1)(0)
        nb = (ctypes.c_int64 * 1)(layer_bytes)
        h = ctypes.c_void_p()
        return lib.woq_pager_create(woq._ptr(pool), off, nb, 1, steps, 1, max_b, ctypes.byref(h))

    assert create(8, 4096) == woq.WOQ_EINVAL                 # codes not 16-byte aligned
    assert create(4096 - need + 16, 4096) == woq.WOQ_EINVAL  # codes run past the block
    assert create(0, 4096, seg_end=N - 1) == woq.WOQ_EINVAL   # segments do not cover N
    assert create(0, 4096, nseg=0) == woq.WOQ_EINVAL
    assert create(0, 4096, max_b=9) == woq.WOQ_EINVAL
    assert create(0, 0) == woq.WOQ_EINVAL
    assert lib.woq_pager_destroy(None) == woq.WOQ_OK


def test_tiered_create_validates_streamed_offsets():
    """A streamed INT4O step's codes, scales and outlier arrays must lie inside
    its layer's block at 16-byte aligned offsets (checked before any device
    call)."""
    import ctypes
    lib = woq.lib()
    pool = np.zeros(1 << 16, np.uint8)
    N, K = 32, 300
    g = woq.woq_int4o_geometry(K)
    cb, sb, wb = ctypes.c_int64(), ctypes.c_int64(), ctypes.c_int64()
    assert lib.woq_int4o_dev_sizes(N, ctypes.byref(g), ctypes.byref(cb), ctypes.byref(sb), ctypes.byref(wb)) == 0
    cb, sb, wb = cb.value, sb.value, wb.value
    total = cb + sb + wb

    def create(codes, scales, wout, layer_bytes):
        st = woq.StackStep()
        st.fmt, st.in_slot, st.out_slot = woq.FMT_INT4O, 0, 0
        st.w4.codes, st.w4.scales, st.w4.w_out = codes, scales, wout
        st.w4.N, st.w4.geom = N, g
        st.perm = 16          # never read: creation stops at the offset checks
        steps = (woq.StackStep * 1)(st)
        off = (ctypes.c_int64 * 1)(0)
        nb = (ctypes.c_int64 * 1)(layer_bytes)
        h = ctypes.c_void_p()
        return lib.woq_tiered_create(woq._ptr(pool), off, nb, 1, steps, 1, 1, ctypes.byref(h))

    assert create(0, cb, cb + sb, total - 16) == woq.WOQ_EINVAL     # outliers run past the block
    assert create(8, cb + 16, cb + sb + 16, total + 64) == woq.WOQ_EINVAL   # codes misaligned
    assert create(0, cb + 4, cb + sb + 16, total + 64) == woq.WOQ_EINVAL    # scales misaligned
    h = ctypes.c_void_p()
    assert lib.woq_tiered_create(None, None, None, 1, None, 1, 1, ctypes.byref(h)) == woq.WOQ_EINVAL


def test_plan_tiers_properties():
    """Resident layers form a prefix; the plan fits the budget; one more
    resident layer would not; everything resident when the model fits; two
    slots are the floor."""
    rng = np.random.default_rng(3)
    for trial in range(200):
        L = int(rng.integers(1, 12))
        lb = rng.integers(1, 1000, L)
        budget = int(rng.integers(0, int(lb.sum()) + 2000))
        try:
            res, dev = woq.woq_plan_tiers(lb, budget)
        except woq.WoqError as e:
            assert e.status == woq.WOQ_ENOMEM
            assert budget < 2 * lb.max() and budget < lb.sum()
            continue
        nA = int(res.sum())
        assert np.all(res[:nA] == 1) and np.all(res[nA:] == 0)

        def need(n):
            return int(lb[:n].sum()) + (2 * int(lb[n:].max()) if n < L else 0)
        assert dev == need(nA) <= budget
        assert all(need(n) > budget for n in range(nA + 1, L + 1))
        if budget >= lb.sum():
            assert nA == L and dev == lb.sum()


def test_plan_tiers_equal_layers_closed_form():
    """Equal blocks of B bytes: n_A = L if L*B fits, else floor(budget/B) - 2
    (two slots), and not enough for two slots is an error."""
    B, L = 454_000_000, 80
    for budget_gb in (1, 16, 24, 30, 36.3, 36.4, 288):
        budget = int(budget_gb * 1e9)
        if budget < 2 * B:
            with pytest.raises(woq.WoqError):
                woq.woq_plan_tiers([B] * L, budget)
            continue
        res, dev = woq.woq_plan_tiers([B] * L, budget)
        want = L if L * B <= budget else min(L - 1, budget // B - 2)
        assert res.sum() == want, budget_gb
    with pytest.raises(woq.WoqError) as e:
        woq.woq_plan_tiers([0, 5], 100)
    assert e.value.status == woq.WOQ_EINVAL


def test_binding_refuses_batches_larger_than_buffers():
    """The C ABI takes plain pointers; the binding checks row counts first."""
    x = np.zeros((4, 64), np.float16)
    y = np.zeros((8, 16), np.float16)
    woq.need_rows(4, x, y)
    with pytest.raises(ValueError):
        woq.need_rows(8, x, y)
    with pytest.raises(ValueError):
        woq.woq_qgemv_int8(woq.Int8W(), x, y, b=8)


def test_binding_refuses_unbound_or_mismatched_slots():
    """Stack.bind / Pager.bind refuse, before any pointer reaches the library,
    a slot list that misses a slot a step names, and a tensor that is not
    fp16, not contiguous, not 2-D, not on the GPU, or not exactly as wide as
    the step's input (K) or output (N)."""
    import torch
    widths = [(0, 64, 1, 32), (1, 32, 2, 48)]        # step 1 reads step 0's output

    def t(r, c, **kw):
        return torch.zeros(r, c, dtype=kw.get("dtype", torch.float16))

    good_in = [t(2, 64), t(2, 32)]
    good_out = [t(2, 8), t(2, 32), t(2, 48)]
    good_out[1] = good_in[1]                        # the chained slot is one tensor
    woq.check_slots(widths, good_in, good_out, device_type="cpu")
    bad_cases = [
        ([t(2, 64)], good_out),                                 # input slot 1 missing
        (good_in, good_out[:2]),                                # output slot 2 missing
        ([t(2, 64, dtype=torch.float32), good_in[1]], good_out),
        ([t(2, 65), good_in[1]], good_out),                     # wider than K
        ([t(2, 64), good_in[1]], [t(2, 8), good_in[1], t(2, 47)]),
        ([t(2, 128)[:, ::2], good_in[1]], good_out),            # strided view
        ([torch.zeros(128, dtype=torch.float16), good_in[1]], good_out),
    ]
    for ins, outs in bad_cases:
        with pytest.raises(ValueError):
            woq.check_slots(widths, ins, outs, device_type="cpu")
    with pytest.raises(ValueError, match="not on the GPU"):
        woq.check_slots(widths, good_in, good_out)
    # the widths the binding derives from runner and pager steps
    st = woq.StackStep()
    st.fmt, st.in_slot, st.out_slot = woq.FMT_INT8, 3, 5
    st.w8.N, st.w8.K = 48, 64
    ps = woq.PagerStep()
    ps.w.N, ps.w.K = 16, 24
    assert woq.slot_widths([st]) == [(3, 64, 5, 48)]
    assert woq.slot_widths([ps, ps]) == [(0, 24, 0, 16), (1, 24, 1, 16)]


def test_decode_input_rows_for_any_batch():
    """Inputs have exactly b rows, also above the workload's largest batch,
    and a smaller batch is a prefix of a larger one."""
    spec = synth.stack_spec(3)
    x8 = synth.decode_input(spec, 1, 2, 8)
    assert x8.shape == (8, spec.space_width("h"))        # input 2 (gate|up) reads the hidden space
    np.testing.assert_array_equal(synth.decode_input(spec, 1, 2, 4), x8[:4])
    np.testing.assert_array_equal(synth.decode_input(spec, 1, 2), x8[:spec.bmax])


# ------------------------------------------------------- persisted pool

def test_pool_roundtrip_and_damage(tmp_path):
    """Blocks and metadata come back byte for byte; a flipped byte in a block,
    in the table or in the magic, and a truncated file, are reported."""
    rng = np.random.default_rng(8)
    blocks = [rng.integers(0, 256, n, dtype=np.uint8) for n in (0, 1, 4095, 4096, (1 << 20) + 13, 3 << 20)]
    meta = b'{"hello": "pool"}'
    path = str(tmp_path / "p.woqpool")
    woq.woq_pool_save(path, meta, blocks)
    m, sizes = woq.woq_pool_info(path)
    assert m == meta and sizes == [b.size for b in blocks]
    for i, b in enumerate(blocks):
        dst = np.full(b.size + 7, 0xEE, np.uint8)
        woq.woq_pool_read_block(path, i, dst)
        np.testing.assert_array_equal(dst[:b.size], b)
        assert np.all(dst[b.size:] == 0xEE)
    with pytest.raises(woq.WoqError) as e:
        woq.woq_pool_read_block(path, 4, np.empty(10, np.uint8))        # too small
    assert e.value.status == woq.WOQ_EINVAL
    raw = bytearray(open(path, "rb").read())
    assert len(raw) % 4096 == 0

    def damaged(mutate, block=4):
        bad = bytearray(raw)
        mutate(bad)
        p2 = str(tmp_path / "bad.woqpool")
        open(p2, "wb").write(bytes(bad))
        with pytest.raises(woq.WoqError) as e:
            woq.woq_pool_read_block(p2, block, np.empty(sizes[block], np.uint8))
        return e.value.status

    off4 = int(np.frombuffer(bytes(raw[32 + 24 * 4: 32 + 24 * 4 + 8]), np.uint64)[0])
    assert damaged(lambda b: b.__setitem__(off4 + 12345, b[off4 + 12345] ^ 1)) == woq.WOQ_EFORMAT
    assert damaged(lambda b: b.__setitem__(40, b[40] ^ 1)) == woq.WOQ_EFORMAT      # table
    assert damaged(lambda b: b.__setitem__(0, ord("X"))) == woq.WOQ_EFORMAT      # magic
    assert damaged(lambda b: b.__delitem__(slice(off4 + 100, None))) == woq.WOQ_EFORMAT   # truncated
    with pytest.raises(woq.WoqError) as e:
        woq.woq_pool_info(str(tmp_path / "missing.woqpool"))
    assert e.value.status == woq.WOQ_EIO


# ------------------------------------------------- permutation positions

@pytest.mark.parametrize("K", [8, 130, 1000, 3072])
def test_perm_positions_invert_the_oracle_split(K):
    """xp (the oracle's permute/split, padded as the device row) at pos[j] is
    x[j] for every channel; table padding is 0xFFFF."""
    rng = np.random.default_rng(K)
    n_out = O.n_outliers(K)
    perm = O.global_perm(K, O.select_outliers(rng.random(K), n_out)).astype(np.int32)
    g = woq.woq_int4o_geometry(K)
    pos = woq.woq_perm_positions(perm, g)
    x = rng.standard_normal((2, K)).astype(np.float16)
    x_bg, x_out = O.permute_split(x, perm, n_out)
    xp = np.zeros((2, g.xp_len))
    xp[:, :x_bg.shape[1]] = x_bg          # background, zero-padded to whole groups
    xp[:, 128 * g.G4:128 * g.G4 + n_out] = x_out
    assert pos.shape == (-(-K // 8) * 8,)
    np.testing.assert_array_equal(xp[:, pos[:K].astype(np.int64)], x)
    assert np.all(pos[K:] == 0xFFFF)
    assert len(set(pos[:K].tolist())) == K


def test_perm_positions_rejects_non_permutations():
    K = 64
    g = woq.woq_int4o_geometry(K)
    perm = np.arange(K, dtype=np.int32)
    perm[5] = 6
    with pytest.raises(woq.WoqError) as e:
        woq.woq_perm_positions(perm, g)
    assert e.value.status == woq.WOQ_EINVAL
    perm[5] = K
    with pytest.raises(woq.WoqError):
        woq.woq_perm_positions(perm, g)
    big = woq.woq_int4o_geometry(70000)
    with pytest.raises(woq.WoqError) as e:
        woq.woq_perm_positions(np.arange(70000, dtype=np.int32), big)
    assert e.value.status == woq.WOQ_EUNSUPPORTED
    assert woq.woq_qgemv_int4o_x_supported(woq.woq_int4o_geometry(28672), 1)
    assert not woq.woq_qgemv_int4o_x_supported(woq.woq_int4o_geometry(28672), 2)
    assert not woq.woq_qgemv_int4o_x_supported(woq.woq_int4o_geometry(3072), 8)


def test_library_loads_after_torchs_hip_runtime():
    """torch ships its own HIP runtime; the binding imports torch before it
    loads the library, so that both use one runtime."""
    import subprocess
    code = ("import sys; from weight_only_quantized_quantize_amd import woq; "
            "assert 'torch' not in sys.modules; woq.lib(); assert 'torch' in sys.modules")
    subprocess.run([sys.executable, "-c", code], cwd=ROOT, check=True, timeout=300)
