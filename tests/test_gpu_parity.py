"""GPU parity: the HIP kernels, called through the C ABI, against the oracle.

Outputs are compared element by element with the float64 oracle on the same
seeded inputs; the gate is the normwise relative error
max|y - y_ref| / max|y_ref| <= 2e-3 (fp32 accumulation, fp16 output).  Where
the oracle also gives the sum of absolute terms A = sum_k |w_nk x_k| of every
output, the componentwise error max |y - y_ref| / A is reported and held to
2^-10: the fp16 rounding of the output contributes at most 2^-11 (|fp32 sum|
<= A), and the fp32 accumulation of exact fp16 products (including the
kernels' biased-code products and their once-per-chunk correction) is
allowed as much again.  The
permutation kernel is integer work and must match bit for bit.  Full-size
shapes are checked on sampled output rows, which the oracle can compute one by
one because every output row depends only on its own weight row.
"""
import numpy as np
import pytest

import oracle as O
import synth
from weight_only_quantized_quantize_amd import woq

pytestmark = pytest.mark.gpu

TOL = 2e-3
CW_TOL = 2.0 ** -10


def _dev(a):
    import torch
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def _host(t):
    import torch
    torch.cuda.synchronize()
    return t.cpu().numpy()


def _empty16(*shape):
    import torch
    return torch.empty(*shape, dtype=torch.float16, device="cuda")


def _print_case(*args):
    print("case:", *args, flush=True)


# ------------------------------------------------------------------ helpers

def int8_case(W_parts, x):
    """Quantise with the library (bit-exactness to the oracle is a CPU test),
    run the kernel, and return (y_gpu, y_oracle)."""
    parts = [woq.woq_quantize_int8(W) for W in W_parts]
    dw = woq.DeviceInt8(parts)
    # the ABI wants a leading dimension that is a multiple of 8 fp16 values
    K = x.shape[1]
    xpad = np.zeros((x.shape[0], -(-K // 8) * 8), np.float16)
    xpad[:, :K] = x
    xd = _dev(xpad)
    y = _empty16(x.shape[0], dw.N)
    woq.woq_qgemv_int8(dw.desc, xd, y)
    qs = [O.quantize_int8(W) for W in W_parts]
    ref = np.concatenate([O.linear_int8(*qw, x) for qw in qs], axis=1)
    absref = np.concatenate([O.linear_int8_abs(*qw, x) for qw in qs], axis=1)
    return _host(y).astype(np.float64), (ref, absref)


def int4o_parts(W_list, perm, n_out):
    return [woq.woq_quantize_int4o(W, perm, n_out) for W in W_list]


def int4o_run(parts, g, perm, x, force_mfma=False):
    """Permute + product through the two public calls; where the one-launch
    form (permutation folded into the product) supports the case, it must give
    the same bits."""
    dw = woq.DeviceInt4o(parts, g)
    xd = _dev(x)
    xp = _empty16(x.shape[0], g.xp_len)
    woq.woq_permute_x(xd, _dev(perm), g, xp)
    y = _empty16(x.shape[0], dw.N)
    (woq.woq_qgemm_int4o if force_mfma else woq.woq_qgemv_int4o)(dw.desc, xp, y)
    y_host = _host(y)
    b = x.shape[0]
    if not force_mfma and woq.woq_qgemv_int4o_x_supported(g, b):
        y1 = one_launch(dw, g, perm, x)
        if b <= 2 or -(-dw.N // 16) < 384:
            # the two-call form runs the same vector kernel: identical bits
            np.testing.assert_array_equal(y1.view(np.uint16), y_host.view(np.uint16),
                                          err_msg="one-launch permutation+product differs from the two-call form")
        else:
            # the two-call form runs the matrix-core kernel here: same values up to summation order
            assert O.normwise_rel_err(y1.astype(np.float64), y_host.astype(np.float64)) <= TOL
    if (force_mfma or b > 4) and woq.woq_qgemm_int4o_x_supported(g, dw.N, b):
        # the matrix-core product with the permutation folded in: the same bits
        y2 = one_launch(dw, g, perm, x, mfma=True)
        np.testing.assert_array_equal(y2.view(np.uint16), y_host.view(np.uint16),
                                      err_msg="one-launch matrix-core product differs from the two-call form")
    return y_host.astype(np.float64), _host(xp)


def one_launch(dw, g, perm, x, ldx=None, mfma=False):
    """woq_qgemv_int4o_x (mfma: woq_qgemm_int4o_x) on x stored with leading
    dimension ldx (>= K, multiple of 8)."""
    b, K = x.shape
    ldx = ldx or -(-K // 8) * 8
    xpad = np.full((b, ldx), np.float16(3.0), np.float16)     # padding must not leak into the result
    xpad[:, :K] = x
    pos = _dev(woq.woq_perm_positions(perm, g))
    y = _empty16(b, dw.N)
    y.fill_(7.0)
    (woq.woq_qgemm_int4o_x if mfma else woq.woq_qgemv_int4o_x)(dw.desc, _dev(xpad), pos, y, ldx=ldx)
    return _host(y)


def int4o_ref(W_list, perm, n_out, x):
    """(oracle output, sum of absolute terms) of the linears in W_list, stacked along N."""
    x_bg, x_out = O.permute_split(x, perm, n_out)
    ys, abs_ = [], []
    for W in W_list:
        c, s, wo = O.quantize_int4o(W, perm, n_out)
        ys.append(O.linear_int4o(c, s, wo, x_bg, x_out))
        abs_.append(O.linear_int4o_abs(c, s, wo, x_bg, x_out))
    return np.concatenate(ys, axis=1), np.concatenate(abs_, axis=1)


def check(y, ref, what):
    """ref is the oracle's output, or (output, sum of absolute terms)."""
    absref = None
    if isinstance(ref, tuple):
        ref, absref = ref
    err = O.normwise_rel_err(y, ref)
    cw = O.componentwise_rel_err(y, ref, absref) if absref is not None else None
    print(f"{what}: normwise rel err {err:.3e}" + (f", componentwise {cw:.3e}" if cw is not None else ""), flush=True)
    assert np.all(np.isfinite(y)), what
    assert err <= TOL, (what, err)
    if cw is not None:
        assert cw <= CW_TOL, (what, "componentwise", cw)
    return err


# ------------------------------------------------------------- permutation

@pytest.mark.parametrize("K,n_out,b", [(3072, -1, 1), (300, 3, 5), (129, 1, 2), (256, 0, 3), (16, 16, 1),
                                       (28672, -1, 2)])
def test_permute_x_bit_exact(gpu_lib, K, n_out, b):
    _print_case("permute", K, n_out, b)
    rng = np.random.default_rng(K)
    g = woq.woq_int4o_geometry(K, n_out)
    perm = O.global_perm(K, np.sort(rng.choice(K, g.n_out, replace=False)))
    x = rng.standard_normal((b, K)).astype(np.float16)
    xd = _dev(x)
    xp = _empty16(b, g.xp_len)
    xp.fill_(7.0)                      # padding must be overwritten with zeros
    woq.woq_permute_x(xd, _dev(perm), g, xp)
    got = _host(xp)
    x_bg, x_out = O.permute_split(x, perm, g.n_out)
    want = np.zeros((b, g.xp_len), np.float16)
    want[:, : g.K_pad] = x_bg
    want[:, 128 * g.G4: 128 * g.G4 + g.n_out] = x_out
    np.testing.assert_array_equal(got.view(np.uint16), want.view(np.uint16))


# -------------------------------------------------------------------- INT8

def test_int8_single_linear_4096(gpu_lib):
    _print_case("int8 4096x4096 b=1 seed 0")
    W, x = synth.config1_inputs()
    y, ref = int8_case([W], x)
    check(y, ref, "int8 4096^2")


@pytest.mark.parametrize("N,K", [(1, 64), (5, 33), (130, 1000), (67, 3584), (4, 17)])
@pytest.mark.parametrize("b", [1, 2, 4, 8])
def test_int8_ragged(gpu_lib, N, K, b):
    _print_case("int8", N, K, b)
    rng = np.random.default_rng(N * 7 + K + b)
    W = (rng.standard_normal((N, K)) * 0.02).astype(np.float32)
    x = rng.standard_normal((b, K)).astype(np.float16)
    y, ref = int8_case([W], x)
    check(y, ref, f"int8 {N}x{K} b={b}")


@pytest.mark.parametrize("N,K,b", [(16389, 3000, 5), (16389, 3000, 8), (8200, 1000, 7), (8200, 1000, 8),
                                   (28672, 3584, 6), (16384, 3584, 4), (8200, 1004, 6), (16389, 1000, 4),
                                   (16389, 1000, 3), (16389, 3500, 8), (8200, 3000, 8), (8200, 5000, 7),
                                   (28700, 1000, 8), (40000, 700, 5)])
def test_int8_matrix_core_sizes(gpu_lib, N, K, b):
    """Products that run the matrix-core INT8 kernel (N >= 16384 from b = 4,
    N >= 8192 from b = 7: ragged N and K, K not a multiple of 64, a last piece
    that ends inside 8 channels, K chunks that fill the unrolled loop body and
    ones that leave a remainder under every plan) and neighbours on the vector
    kernel, on sampled rows including the first and last.  On 256 compute
    units, 1025-1792 tiles run seven tiles per workgroup, 1794 and 2500 eight."""
    _print_case("int8 mfma", N, K, b)
    rng = np.random.default_rng(N + K + b)
    W = (rng.standard_normal((N, K)) * 0.02).astype(np.float32)
    x = rng.standard_normal((b, K)).astype(np.float16)
    q, s = woq.woq_quantize_int8(W)
    dw = woq.DeviceInt8([(q, s)])
    ldx = -(-K // 8) * 8
    xpad = np.full((b, ldx), np.float16(np.inf), np.float16)   # padding past K must not reach the sum
    xpad[:, :K] = x
    y = _empty16(b, N)
    woq.woq_qgemv_int8(dw.desc, _dev(xpad), y)
    rows = np.concatenate([np.arange(16), np.sort(rng.choice(N, 100, replace=False)), np.arange(N - 16, N)])
    qo, so = O.quantize_int8(W, rows=rows)
    check(_host(y)[:, rows].astype(np.float64), (O.linear_int8(qo, so, x), O.linear_int8_abs(qo, so, x)),
          f"int8 mfma {N}x{K} b={b}")


def test_int8_fused_segments(gpu_lib):
    _print_case("int8 fused q|k|v")
    spec = synth.small_stack_spec(3, layers=1)
    Ws = [synth.weight(spec, 0, n) for n in ("q", "k", "v")]
    Ws[1] = Ws[1] * np.float32(7.0)        # distinct per-tensor scales
    x = synth.decode_input(spec, 0, 0, 4)
    y, ref = int8_case(Ws, x)
    check(y, ref, "int8 fused")


def test_int8_config3_full_shapes_sampled(gpu_lib):
    spec = synth.stack_spec(3)
    rng = np.random.default_rng(3)
    for lin in spec.linears():
        _print_case("int8 cfg3", lin.name, lin.N, lin.K)
        W = synth.weight(spec, 0, lin)
        x = synth.decode_input(spec, 0, lin.inp, 4)
        q, s = woq.woq_quantize_int8(W)
        dw = woq.DeviceInt8([(q, s)])
        for b in (1, 4):
            y = _empty16(b, lin.N)
            woq.woq_qgemv_int8(dw.desc, _dev(x[:b]), y)
            rows = np.sort(rng.choice(lin.N, 64, replace=False))
            qo, so = O.quantize_int8(W, rows=rows)
            ref = (O.linear_int8(qo, so, x[:b]), O.linear_int8_abs(qo, so, x[:b]))
            check(_host(y)[:, rows].astype(np.float64), ref, f"int8 cfg3 {lin.name} b={b}")


# ------------------------------------------------------------------- INT4O

@pytest.mark.parametrize("N,K,n_out", [(4, 128, 0), (5, 300, 3), (130, 1000, -1), (9, 129, 1), (8, 16, 16),
                                       (67, 3072, -1), (3, 700, 0)])
@pytest.mark.parametrize("b", [1, 2, 3, 7])
def test_int4o_valu_ragged(gpu_lib, N, K, n_out, b):
    _print_case("int4o valu", N, K, n_out, b)
    rng = np.random.default_rng(N + K + b)
    g = woq.woq_int4o_geometry(K, n_out)
    outs = np.sort(rng.choice(K, g.n_out, replace=False))
    W = (rng.standard_normal((N, K)) * 0.02).astype(np.float32)
    W[:, outs] *= 10
    x = rng.standard_normal((b, K)).astype(np.float32)
    x[:, outs] *= 20
    x = x.astype(np.float16)
    perm = O.global_perm(K, outs)
    y, _ = int4o_run(int4o_parts([W], perm, g.n_out), g, perm, x)
    check(y, int4o_ref([W], perm, g.n_out, x), f"int4o {N}x{K} n_out={g.n_out} b={b}")


# (rows, channels, groups per tile row, plan T x S): waves of 9, 9 or 8, 5, 8,
# 18, 10, 17 and 16 groups
@pytest.mark.parametrize("N,K,G4,plan", [(100, 4655, 36, "1x4"), (100, 8405, 68, "1x8"), (100, 2110, 20, "1x4"),
                                         (100, 8275, 64, "1x8"), (16400, 4655, 36, "2x2"), (16400, 2100, 20, "2x2"),
                                         (4100, 8405, 68, "1x4"), (300, 16529, 128, "1x8")])
@pytest.mark.parametrize("b", [1, 2])
def test_int4o_valu_window_lengths(gpu_lib, N, K, G4, plan, b):
    """The vector kernel's weight window holds 8 groups per wave: rows whose
    waves take fewer, exactly 8, 8 + 1, several whole windows, and whole
    windows + a remainder, under each tile plan (T tiles x S waves): the last
    window takes no refills, earlier ones refill each slot after using it."""
    _print_case("int4o window", N, K, G4, plan, b)
    rng = np.random.default_rng(N + 3 * K + b)
    g = woq.woq_int4o_geometry(K)
    assert g.G4 == G4
    outs = np.sort(rng.choice(K, g.n_out, replace=False))
    W = (rng.standard_normal((N, K)) * 0.02).astype(np.float32)
    W[:, outs] *= 10
    x = rng.standard_normal((b, K)).astype(np.float32)
    x[:, outs] *= 20
    x = x.astype(np.float16)
    perm = O.global_perm(K, outs)
    y, _ = int4o_run(int4o_parts([W], perm, g.n_out), g, perm, x)
    check(y, int4o_ref([W], perm, g.n_out, x), f"int4o window {N}x{K} G4={G4} plan {plan} b={b}")


@pytest.mark.parametrize("N,K,n_out", [(16, 128, 0), (37, 300, 3), (130, 1000, -1), (64, 3072, -1), (20, 16, 16)])
@pytest.mark.parametrize("b", [1, 8, 16, 17, 32, 64])
def test_int4o_mfma_ragged(gpu_lib, N, K, n_out, b):
    _print_case("int4o mfma", N, K, n_out, b)
    rng = np.random.default_rng(N * 3 + K + b)
    g = woq.woq_int4o_geometry(K, n_out)
    outs = np.sort(rng.choice(K, g.n_out, replace=False))
    W = (rng.standard_normal((N, K)) * 0.02).astype(np.float32)
    W[:, outs] *= 10
    x = rng.standard_normal((b, K)).astype(np.float32)
    x[:, outs] *= 20
    x = x.astype(np.float16)
    perm = O.global_perm(K, outs)
    y, _ = int4o_run(int4o_parts([W], perm, g.n_out), g, perm, x, force_mfma=True)
    check(y, int4o_ref([W], perm, g.n_out, x), f"int4o mfma {N}x{K} n_out={g.n_out} b={b}")


def test_int4o_small_stack_layer_fused(gpu_lib):
    """A reduced config-2 layer: global perms from the library's own selection,
    q|k|v and gate|up fused along N."""
    spec = synth.small_stack_spec(2, layers=2)
    perms = {}
    for space in synth.SPACES:
        K = spec.space_width(space)
        cs = np.zeros(K)
        for layer in range(spec.layers):
            for lin in spec.linears():
                if lin.space == space:
                    woq.woq_colabs_accumulate(synth.weight(spec, layer, lin), cs)
        perms[space] = woq.woq_outlier_select(cs, synth.profile(spec, space))
    for layer in range(spec.layers):
        for names, inp in ((("q", "k", "v"), 0), (("o",), 1), (("gate", "up"), 2), (("down",), 3)):
            _print_case("int4o small stack", layer, names)
            lin0 = spec.linear(names[0])
            perm = perms[lin0.space]
            g = woq.woq_int4o_geometry(lin0.K)
            Ws = [synth.weight(spec, layer, n) for n in names]
            x = synth.decode_input(spec, layer, inp, 1)
            y, _ = int4o_run(int4o_parts(Ws, perm, g.n_out), g, perm, x)
            check(y, int4o_ref(Ws, perm, g.n_out, x), f"layer {layer} {'|'.join(names)}")


@pytest.mark.parametrize("cfg", [2, 4])
def test_int4o_full_shapes_sampled(gpu_lib, cfg):
    """Every linear shape of the 3B- and 70B-shaped stacks at full size (layer 0),
    in the launch configuration the benchmark uses, on sampled output rows.
    The permutation is the planted set, which selection recovers (CPU test)."""
    spec = synth.stack_spec(cfg)
    rng = np.random.default_rng(cfg)
    for lin in spec.linears():
        K = lin.K
        g = woq.woq_int4o_geometry(K)
        perm = O.global_perm(K, synth.planted_set(spec, lin.space))
        W = synth.weight(spec, 0, lin)
        part = woq.woq_quantize_int4o(W, perm, g.n_out)
        rows = np.sort(rng.choice(lin.N, 48, replace=False))
        c, s, wo = O.quantize_int4o(W[rows], perm, g.n_out)
        del W
        x = synth.decode_input(spec, 0, lin.inp)
        for b in spec.batches:
            _print_case("int4o full", cfg, lin.name, lin.N, K, b)
            y, _ = int4o_run([part], g, perm, x[:b])
            x_bg, x_out = O.permute_split(x[:b], perm, g.n_out)
            check(y[:, rows], (O.linear_int4o(c, s, wo, x_bg, x_out), O.linear_int4o_abs(c, s, wo, x_bg, x_out)),
                  f"cfg{cfg} {lin.name} b={b}")


@pytest.mark.parametrize("N,K,b,ldx", [(1, 8, 1, 8), (5, 300, 3, 320), (4100, 1000, 2, 1000 + 24),
                                       (4100, 1000, 1, 1000), (11205, 1000, 1, 1000 + 8),
                                       (16500, 3072, 1, 3072), (33, 8192, 3, 8192), (17, 28672, 1, 28672 + 8)])
def test_int4o_one_launch_matches_oracle(gpu_lib, N, K, b, ldx):
    """The permutation folded into the product, including row strides above K,
    every tile/split plan of the vector kernel (N from 1 to 16500 rows) and the
    largest supported row."""
    _print_case("int4o one launch", N, K, b, ldx)
    rng = np.random.default_rng(N + 7 * K + b)
    g = woq.woq_int4o_geometry(K)
    assert woq.woq_qgemv_int4o_x_supported(g, b)
    outs = np.sort(rng.choice(K, g.n_out, replace=False))
    W = (rng.standard_normal((N, K)) * 0.02).astype(np.float32)
    W[:, outs] *= 10
    x = rng.standard_normal((b, K)).astype(np.float32)
    x[:, outs] *= 20
    x = x.astype(np.float16)
    perm = O.global_perm(K, outs)
    parts = int4o_parts([W], perm, g.n_out)
    dw = woq.DeviceInt4o(parts, g)
    y = one_launch(dw, g, perm, x, ldx).astype(np.float64)
    check(y, int4o_ref([W], perm, g.n_out, x), f"one launch {N}x{K} b={b}")


def test_int4o_one_launch_rejects_unsupported(gpu_lib):
    g = woq.woq_int4o_geometry(28672)
    rng = np.random.default_rng(1)
    perm = O.global_perm(28672, np.sort(rng.choice(28672, g.n_out, replace=False)))
    W = (rng.standard_normal((4, 28672)) * 0.02).astype(np.float32)
    dw = woq.DeviceInt4o(int4o_parts([W], perm, g.n_out), g)
    x = _dev(np.zeros((2, 28672), np.float16))
    pos = _dev(woq.woq_perm_positions(perm, g))
    with pytest.raises(woq.WoqError) as e:
        woq.woq_qgemv_int4o_x(dw.desc, x, pos, _empty16(2, 4))
    assert e.value.status == woq.WOQ_EUNSUPPORTED


def test_int4o_mfma_one_launch_rejects_unsupported(gpu_lib):
    """The matrix-core one-launch form refuses what it does not cover (b above
    8, rows whose permuted row does not fit on chip, rows under 64 groups)
    with WOQ_EUNSUPPORTED, before any launch."""
    for K, N, b in [(28672, 8192, 8), (8192, 4096, 9), (3072, 4096, 8)]:
        g = woq.woq_int4o_geometry(K)
        assert not woq.woq_qgemm_int4o_x_supported(g, N, b), (K, N, b)
    g = woq.woq_int4o_geometry(28672)
    rng = np.random.default_rng(2)
    perm = O.global_perm(28672, np.sort(rng.choice(28672, g.n_out, replace=False)))
    W = (rng.standard_normal((4, 28672)) * 0.02).astype(np.float32)
    dw = woq.DeviceInt4o(int4o_parts([W], perm, g.n_out), g)
    x = _dev(np.zeros((8, 28672), np.float16))
    pos = _dev(woq.woq_perm_positions(perm, g))
    with pytest.raises(woq.WoqError) as e:
        woq.woq_qgemm_int4o_x(dw.desc, x, pos, _empty16(8, 4))
    assert e.value.status == woq.WOQ_EUNSUPPORTED


@pytest.mark.parametrize("N,K,b", [(10240, 8192, 8), (8192, 8192, 8), (57344, 8192, 8), (8192, 8192, 5),
                                   (10240, 8192, 3), (57344, 8192, 1), (8190, 8300, 7), (12300, 8200, 6),
                                   (700, 8200, 4), (16, 8192, 2)])
def test_int4o_mfma_one_launch_full_shapes(gpu_lib, N, K, b):
    """The matrix-core product with the permutation folded in
    (woq_qgemm_int4o_x) against the two-call form (woq_permute_x, then
    woq_qgemm_int4o) bit for bit, on random device weights in the 70B-shaped
    products' layout and plans (every plan of 8 staged columns: one tile per
    workgroup below 256 tiles, two, three and four tiles of one workgroup per
    compute unit, seven or eight tiles of two per wave from 2048 tiles),
    with a random permutation and x stored with a padded leading dimension
    whose padding must not leak into the result."""
    import torch
    _print_case("int4o mfma one launch", N, K, b)
    g = woq.woq_int4o_geometry(K)
    assert woq.woq_qgemm_int4o_x_supported(g, N, b)
    gen = torch.Generator(device="cuda")
    gen.manual_seed(N + K + b)
    cb, sb, wb = woq.woq_int4o_dev_sizes(N, g)
    codes = torch.randint(0, 256, (cb,), dtype=torch.uint8, device="cuda", generator=gen)
    scales = (torch.rand(sb // 2, device="cuda", generator=gen) * 0.01).half()
    wout = (torch.rand(max(1, wb // 2), device="cuda", generator=gen) * 0.01).half()
    w = woq.Int4oW()
    w.codes, w.scales, w.w_out, w.N, w.geom = codes.data_ptr(), scales.data_ptr(), wout.data_ptr(), N, g
    perm = np.random.default_rng(K).permutation(K).astype(np.int32)
    ldx = -(-K // 8) * 8 + 24
    x = torch.full((b, ldx), 3.0, dtype=torch.float16, device="cuda")
    x[:, :K] = torch.randn(b, K, device="cuda", generator=gen).half()
    xp = _empty16(b, g.xp_len)
    woq.woq_permute_x(x[:, :K].contiguous(), _dev(perm), g, xp)
    y2 = _empty16(b, N)
    woq.woq_qgemm_int4o(w, xp, y2)
    y1 = _empty16(b, N)
    y1.fill_(7.0)
    woq.woq_qgemm_int4o_x(w, x, _dev(woq.woq_perm_positions(perm, g)), y1, ldx=ldx)
    h1, h2 = _host(y1), _host(y2)
    assert np.all(np.isfinite(h2))
    np.testing.assert_array_equal(h1.view(np.uint16), h2.view(np.uint16))


def test_batch_prefix_invariant(gpu_lib):
    """Row 0 of a b=32 matrix-core call agrees with the b=1 vector-ALU call."""
    _print_case("prefix invariant")
    rng = np.random.default_rng(5)
    K, N = 1000, 96
    g = woq.woq_int4o_geometry(K)
    perm = O.global_perm(K, np.sort(rng.choice(K, g.n_out, replace=False)))
    W = (rng.standard_normal((N, K)) * 0.02).astype(np.float32)
    x = rng.standard_normal((32, K)).astype(np.float16)
    parts = int4o_parts([W], perm, g.n_out)
    y32, _ = int4o_run(parts, g, perm, x)
    y1, _ = int4o_run(parts, g, perm, x[:1])
    assert O.normwise_rel_err(y32[:1], y1) <= 1e-3


@pytest.mark.parametrize("b,N,K", [(33, 32800, 200), (64, 32800, 200), (3, 32885, 1000), (8, 32885, 1000),
                                   (20, 32885, 1000), (32, 32885, 1000), (8, 57344, 200), (8, 57400, 200),
                                   (32, 57400, 200)])
def test_int4o_mfma_wide_batch_wide_product(gpu_lib, b, N, K):
    """The widest tile plan (N >= 32768 rows: one wave per tile, two tiles
    per wave for up to two column tiles, one for three and four; on 256
    compute units seven waves per workgroup for up to two column tiles here,
    eight for more, and eight from 3585 tiles), with a ragged last workgroup
    and a partial last tile (N = 32885: 2056 tiles, the last with 5 rows;
    N = 57400: 3588 tiles, the last with 8), checked on sampled rows
    including the first and last."""
    _print_case("int4o mfma wide", b, N, K)
    rng = np.random.default_rng(b)
    g = woq.woq_int4o_geometry(K)
    outs = np.sort(rng.choice(K, g.n_out, replace=False))
    W = (rng.standard_normal((N, K)) * 0.02).astype(np.float32)
    W[:, outs] *= 10
    x = rng.standard_normal((b, K)).astype(np.float32)
    x[:, outs] *= 20
    x = x.astype(np.float16)
    perm = O.global_perm(K, outs)
    y, _ = int4o_run(int4o_parts([W], perm, g.n_out), g, perm, x)
    rows = np.concatenate([np.arange(16), np.sort(rng.choice(N, 200, replace=False)), np.arange(N - 16, N)])
    check(y[:, rows], int4o_ref([W[rows]], perm, g.n_out, x), f"mfma wide b={b}")


# (b, rows, channels): the matrix-core plan, then K chunks per row = whole
# unrolled loop bodies + a remainder: T1S8 6 = 0 + 6; T1S8 (8 staged columns)
# 7 = 4 + 3; T1S8, two column tiles 13 = 12 + 1; T2S4 6 = 4 + 2; T2S4, two
# column tiles 25 = 24 + 1; T4S2 (8 staged columns) 7 = 6 + 1; T2S2, three
# column tiles 22 = 20 + 2; T7S1 with two tiles per wave, two column tiles
# 11 = 10 + 1, and one column tile 9 = 8 + 1
@pytest.mark.parametrize("b,N,K", [(8, 200, 5600), (8, 200, 12800), (24, 200, 12800), (8, 5000, 5600),
                                   (24, 5000, 12800), (8, 12000, 12800), (40, 12000, 5600), (32, 33000, 5600),
                                   (8, 33000, 4500)])
def test_int4o_mfma_chunk_remainders(gpu_lib, b, N, K):
    """The matrix-core kernel runs whole unrolled bodies of K chunks and then
    the remaining chunks one by one, with its loads issued in the same order
    in the prologue as in the loop: every plan, with and without a remainder,
    checked on sampled rows including the first and last."""
    _print_case("int4o mfma chunks", b, N, K)
    rng = np.random.default_rng(b + N + K)
    g = woq.woq_int4o_geometry(K)
    outs = np.sort(rng.choice(K, g.n_out, replace=False))
    W = (rng.standard_normal((N, K)) * 0.02).astype(np.float32)
    W[:, outs] *= 10
    x = rng.standard_normal((b, K)).astype(np.float32)
    x[:, outs] *= 20
    x = x.astype(np.float16)
    perm = O.global_perm(K, outs)
    y, _ = int4o_run(int4o_parts([W], perm, g.n_out), g, perm, x, force_mfma=True)
    rows = np.unique(np.concatenate([np.arange(16), np.sort(rng.choice(N, min(N, 150), replace=False)),
                                     np.arange(N - 16, N)]))
    check(y[:, rows], int4o_ref([W[rows]], perm, g.n_out, x), f"mfma chunks b={b} {N}x{K}")


@pytest.mark.parametrize("b,N,K", [(3, 6200, 8200), (5, 700, 28700), (8, 4100, 8300), (8, 700, 28700),
                                   (6, 300, 10000), (8, 16, 8100), (7, 10250, 8300), (5, 8190, 8300),
                                   (8, 12300, 8300), (4, 8200, 8300)])
def test_int4o_mfma_long_rows_small_batch(gpu_lib, b, N, K):
    """Matrix-core products on rows of 64 groups or more at b <= 8, which stage
    only 8 activation columns in chunks of 16 groups: ragged row counts, a
    partial last chunk, and every plan of one workgroup per compute unit on
    256 of them - two tiles of eight waves (N = 4100: 257 tiles; 8190: 512
    tiles, the last of 14 rows), three of four (N = 8200: 513 tiles; 10250:
    641 tiles, the last of 10 rows), four of four (N = 12300: 769 tiles, the
    last of 12 rows) - on sampled rows including the first and last."""
    _print_case("int4o mfma long rows", b, N, K)
    rng = np.random.default_rng(b * 7 + N + K)
    g = woq.woq_int4o_geometry(K)
    outs = np.sort(rng.choice(K, g.n_out, replace=False))
    W = (rng.standard_normal((N, K)) * 0.02).astype(np.float32)
    W[:, outs] *= 10
    x = rng.standard_normal((b, K)).astype(np.float32)
    x[:, outs] *= 20
    x = x.astype(np.float16)
    perm = O.global_perm(K, outs)
    y, _ = int4o_run(int4o_parts([W], perm, g.n_out), g, perm, x, force_mfma=True)
    rows = np.unique(np.concatenate([np.arange(min(N, 16)), np.sort(rng.choice(N, min(N, 100), replace=False)),
                                     np.arange(max(0, N - 16), N)]))
    check(y[:, rows], int4o_ref([W[rows]], perm, g.n_out, x), f"mfma long rows b={b} {N}x{K}")


@pytest.mark.parametrize("b,N,K", [(9, 10250, 8300), (16, 8200, 8300), (17, 8190, 8300), (20, 12300, 8300),
                                   (32, 10250, 8300), (32, 8190, 8300)])
def test_int4o_mfma_long_rows_wide_batch(gpu_lib, b, N, K):
    """Matrix-core products on rows of 64 groups or more at 9 <= b <= 32 (one
    or two column tiles of 16 batch columns), in every plan of one workgroup
    per compute unit: two tiles of eight waves (512 tiles, the last of 14
    rows), three of four (513 tiles, the last of 8 rows; 641 tiles, the last
    of 10 rows), four of four (769 tiles, the last of 12 rows); sampled rows
    including the first and last against the oracle."""
    _print_case("int4o mfma long rows wide batch", b, N, K)
    rng = np.random.default_rng(b * 11 + N + K)
    g = woq.woq_int4o_geometry(K)
    outs = np.sort(rng.choice(K, g.n_out, replace=False))
    W = (rng.standard_normal((N, K)) * 0.02).astype(np.float32)
    W[:, outs] *= 10
    x = rng.standard_normal((b, K)).astype(np.float32)
    x[:, outs] *= 20
    x = x.astype(np.float16)
    perm = O.global_perm(K, outs)
    y, _ = int4o_run(int4o_parts([W], perm, g.n_out), g, perm, x, force_mfma=True)
    rows = np.unique(np.concatenate([np.arange(16), np.sort(rng.choice(N, 100, replace=False)),
                                     np.arange(N - 16, N)]))
    check(y[:, rows], int4o_ref([W[rows]], perm, g.n_out, x), f"mfma long rows b={b} {N}x{K}")


@pytest.mark.parametrize("b,N,K", [(24, 32770, 1100), (9, 32800, 2200), (32, 32790, 4100), (17, 36000, 1000)])
def test_int4o_mfma_wide_plans_above_b8(gpu_lib, b, N, K):
    """The widest matrix-core plans above b = 8 (seven or eight tiles of two
    per wave, one wave per tile group), which multiply the biased codes and
    seed each group's low-nibble sum with minus its activation correction:
    ragged tile counts (a last workgroup only partly filled), groups that
    end inside the last chunk and rows whose last group is partial, on
    sampled rows including the first and last against the oracle."""
    _print_case("int4o mfma wide plans", b, N, K)
    rng = np.random.default_rng(b * 13 + N + K)
    g = woq.woq_int4o_geometry(K)
    outs = np.sort(rng.choice(K, g.n_out, replace=False))
    W = (rng.standard_normal((N, K)) * 0.02).astype(np.float32)
    W[:, outs] *= 10
    x = rng.standard_normal((b, K)).astype(np.float32)
    x[:, outs] *= 20
    x = x.astype(np.float16)
    perm = O.global_perm(K, outs)
    y, _ = int4o_run(int4o_parts([W], perm, g.n_out), g, perm, x, force_mfma=True)
    rows = np.unique(np.concatenate([np.arange(16), np.sort(rng.choice(N, 100, replace=False)),
                                     np.arange(N - 16, N)]))
    check(y[:, rows], int4o_ref([W[rows]], perm, g.n_out, x), f"mfma wide plans b={b} {N}x{K}")


@pytest.mark.parametrize("b,N,K,splits", [(3, 1000, 16400, 8), (8, 1000, 16400, 2), (17, 300, 16400, 5),
                                          (32, 2056, 16400, 8), (8, 16, 2000, 16), (5, 33, 1000, 1)])
def test_int4o_splitk_entry_point(gpu_lib, b, N, K, splits):
    """The matrix-core product over K ranges with partial sums in a caller
    workspace: against the oracle on sampled rows, against the single-launch
    product within rounding, and deterministic from call to call (more splits
    than groups leave empty ranges)."""
    import torch
    _print_case("int4o split-K", b, N, K, splits)
    rng = np.random.default_rng(b + N + K + splits)
    g = woq.woq_int4o_geometry(K)
    outs = np.sort(rng.choice(K, g.n_out, replace=False))
    W = (rng.standard_normal((N, K)) * 0.02).astype(np.float32)
    W[:, outs] *= 10
    x = rng.standard_normal((b, K)).astype(np.float32)
    x[:, outs] *= 20
    x = x.astype(np.float16)
    perm = O.global_perm(K, outs)
    y1, xp_host = int4o_run(int4o_parts([W], perm, g.n_out), g, perm, x, force_mfma=True)
    dw = woq.DeviceInt4o(int4o_parts([W], perm, g.n_out), g)
    xp = _dev(xp_host.astype(np.float16))
    nbytes = woq.lib().woq_qgemm_int4o_splitk_workspace(N, b, splits)
    ws = torch.full((nbytes // 4,), float("nan"), dtype=torch.float32, device="cuda")
    y = _empty16(b, N)
    woq.woq_qgemm_int4o_splitk(dw.desc, xp, y, splits, ws)
    ys = _host(y)
    woq.woq_qgemm_int4o_splitk(dw.desc, xp, y, splits, ws)
    np.testing.assert_array_equal(_host(y).view(np.uint16), ys.view(np.uint16))
    rows = np.unique(np.concatenate([np.arange(min(N, 16)), np.sort(rng.choice(N, min(N, 100), replace=False)),
                                     np.arange(max(0, N - 16), N)]))
    check(ys.astype(np.float64)[:, rows], int4o_ref([W[rows]], perm, g.n_out, x), f"split-K b={b} s={splits}")
    assert O.normwise_rel_err(ys.astype(np.float64), y1) <= TOL
    with pytest.raises(woq.WoqError) as e:
        woq.woq_qgemm_int4o_splitk(dw.desc, xp, y, splits, ws[:nbytes // 4 - 1])
    assert e.value.status == woq.WOQ_EINVAL


@pytest.mark.parametrize("N,K", [(1280, 8192), (7168, 8192), (8192, 1024), (8192, 3584)])
@pytest.mark.parametrize("b", [1, 8, 32])
def test_int4o_tp8_share_shapes(gpu_lib, N, K, b):
    """One GPU's share of the 70B-shaped products under 8-way tensor
    parallelism (q|k|v and gate|up split along N, o and down along K), on
    sampled rows."""
    _print_case("int4o tp8 share", N, K, b)
    rng = np.random.default_rng(N + K + b)
    g = woq.woq_int4o_geometry(K)
    outs = np.sort(rng.choice(K, g.n_out, replace=False))
    W = (rng.standard_normal((N, K)) * 0.015).astype(np.float32)
    W[:, outs] *= 10
    x = rng.standard_normal((b, K)).astype(np.float32)
    x[:, outs] *= 20
    x = x.astype(np.float16)
    perm = O.global_perm(K, outs)
    y, _ = int4o_run(int4o_parts([W], perm, g.n_out), g, perm, x)
    rows = np.sort(rng.choice(N, 64, replace=False))
    check(y[:, rows], int4o_ref([W[rows]], perm, g.n_out, x), f"tp8 {N}x{K} b={b}")


def test_stream_read_entry_point(gpu_lib):
    import torch
    buf = torch.zeros(1 << 20, dtype=torch.uint8, device="cuda")
    woq.woq_stream_read(buf)
    torch.cuda.synchronize()
    with pytest.raises(woq.WoqError) as e:
        woq.woq_stream_read(buf[:15])
    assert e.value.status == woq.WOQ_EINVAL
