"""GPU tests of degenerate and boundary cases of the device entry points:
empty batches and products are no-ops, all-zero weights or activations give
exact zeros, argument errors come back as status codes before any launch."""
import numpy as np
import pytest

import oracle as O
from weight_only_quantized_quantize_amd import woq

pytestmark = pytest.mark.gpu


def _dev(a):
    import torch
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def _host(t):
    import torch
    torch.cuda.synchronize()
    return t.cpu().numpy()


def _filled(b, n, v=7.0):
    import torch
    return torch.full((b, n), v, dtype=torch.float16, device="cuda")


def _int4o(N, K, rng, zero=False):
    g = woq.woq_int4o_geometry(K)
    outs = np.sort(rng.choice(K, g.n_out, replace=False))
    W = np.zeros((N, K), np.float32) if zero else (rng.standard_normal((N, K)) * 0.02).astype(np.float32)
    perm = O.global_perm(K, outs)
    return g, perm, woq.DeviceInt4o([woq.woq_quantize_int4o(W, perm, g.n_out)], g)


def test_empty_batch_is_a_no_op(gpu_lib):
    rng = np.random.default_rng(1)
    g, perm, dw = _int4o(40, 300, rng)
    xp = _filled(0, g.xp_len)
    y = _filled(2, 40)
    woq.woq_qgemv_int4o(dw.desc, xp, y, b=0)
    woq.woq_qgemm_int4o(dw.desc, xp, y, b=0)
    d8 = woq.DeviceInt8([woq.woq_quantize_int8((rng.standard_normal((40, 64)) * 0.02).astype(np.float32))])
    woq.woq_qgemv_int8(d8.desc, _filled(0, 64), y, b=0)
    woq.woq_permute_x(_filled(0, 300), _dev(perm), g, xp)
    assert np.all(_host(y) == 7.0)


def test_zero_weights_and_zero_activations_give_exact_zeros(gpu_lib):
    rng = np.random.default_rng(2)
    for b in (1, 3, 8, 32):
        g, perm, dz = _int4o(50, 1000, rng, zero=True)
        x = rng.standard_normal((b, 1000)).astype(np.float16)
        xp = _filled(b, g.xp_len)
        woq.woq_permute_x(_dev(x), _dev(perm), g, xp)
        y = _filled(b, 50)
        woq.woq_qgemv_int4o(dz.desc, xp, y)
        assert not _host(y).view(np.uint16).any(), b          # +0.0 everywhere
        g, perm, dw = _int4o(50, 1000, rng)
        woq.woq_permute_x(_dev(np.zeros((b, 1000), np.float16)), _dev(perm), g, xp)
        woq.woq_qgemv_int4o(dw.desc, xp, y)
        assert np.all(_host(y) == 0.0), b
    d8 = woq.DeviceInt8([woq.woq_quantize_int8(np.zeros((20, 64), np.float32))])
    y = _filled(2, 20)
    woq.woq_qgemv_int8(d8.desc, _dev(rng.standard_normal((2, 64)).astype(np.float16)), y)
    assert np.all(_host(y) == 0.0)


def test_argument_errors_are_reported_before_launch(gpu_lib):
    import torch
    rng = np.random.default_rng(3)
    g, perm, dw = _int4o(40, 300, rng)
    xp = _filled(65, g.xp_len)
    y = _filled(65, 40)
    with pytest.raises(woq.WoqError) as e:
        woq.woq_qgemm_int4o(dw.desc, xp, y)                  # b = 65 > 64
    assert e.value.status == woq.WOQ_EINVAL
    with pytest.raises(woq.WoqError) as e:
        woq.woq_qgemv_int4o(dw.desc, xp[:2], _filled(2, 39))  # ldy < N
    assert e.value.status == woq.WOQ_EINVAL
    bad = woq.Int4oW()
    bad.codes, bad.scales, bad.w_out, bad.N, bad.geom = dw.desc.codes + 8, dw.desc.scales, dw.desc.w_out, 40, g
    with pytest.raises(woq.WoqError) as e:
        woq.woq_qgemv_int4o(bad, xp[:1], y[:1])              # codes not 16-byte aligned
    assert e.value.status == woq.WOQ_EALIGN
    g2 = woq.woq_int4o_geometry(300)
    g2.G4 += 4                                                # not what woq_int4o_geometry gives
    bad = woq.Int4oW()
    bad.codes, bad.scales, bad.w_out, bad.N, bad.geom = dw.desc.codes, dw.desc.scales, dw.desc.w_out, 40, g2
    with pytest.raises(woq.WoqError) as e:
        woq.woq_qgemv_int4o(bad, xp[:1], y[:1])
    assert e.value.status == woq.WOQ_EINVAL
    d8 = woq.DeviceInt8([woq.woq_quantize_int8((rng.standard_normal((40, 64)) * 0.02).astype(np.float32))])
    with pytest.raises(woq.WoqError) as e:
        woq.woq_qgemv_int8(d8.desc, _filled(9, 64), _filled(9, 40))   # b = 9 > 8
    assert e.value.status == woq.WOQ_EINVAL
    with pytest.raises(woq.WoqError) as e:
        woq.woq_qgemv_int8(d8.desc, _filled(1, 60)[:, :60], _filled(1, 40))  # ldx < K
    assert e.value.status == woq.WOQ_EINVAL
    with pytest.raises(ValueError):
        woq.woq_qgemv_int8(d8.desc, _filled(2, 64), _filled(1, 40))  # the binding: y has 1 row for b = 2
    torch.cuda.synchronize()


def test_products_of_one_row_and_one_channel_group(gpu_lib):
    """N = 1 (one row in a 16-row tile) at every kernel, against the oracle."""
    rng = np.random.default_rng(4)
    K = 130
    g = woq.woq_int4o_geometry(K)
    outs = np.sort(rng.choice(K, g.n_out, replace=False))
    W = (rng.standard_normal((1, K)) * 0.02).astype(np.float32)
    W[:, outs] *= 10
    perm = O.global_perm(K, outs)
    dw = woq.DeviceInt4o([woq.woq_quantize_int4o(W, perm, g.n_out)], g)
    c, s, wo = O.quantize_int4o(W, perm, g.n_out)
    for b, fn in ((1, woq.woq_qgemv_int4o), (3, woq.woq_qgemm_int4o), (40, woq.woq_qgemm_int4o)):
        x = rng.standard_normal((b, K)).astype(np.float16)
        xp = _filled(b, g.xp_len)
        woq.woq_permute_x(_dev(x), _dev(perm), g, xp)
        y = _filled(b, 1)
        fn(dw.desc, xp, y)
        x_bg, x_out = O.permute_split(x, perm, g.n_out)
        err = O.normwise_rel_err(_host(y).astype(np.float64), O.linear_int4o(c, s, wo, x_bg, x_out))
        assert err <= 2e-3, (b, err)


def test_dispatch_floor_measurement(gpu_lib):
    """The empty-launch measurement: positive and finite, not longer than a
    real product's launch, and argument errors reported."""
    import torch
    s = torch.cuda.current_stream()
    span, interval = woq.woq_dispatch_floor(256, 256, 50, s)
    assert 0.0 < span < 1000.0, span
    assert 0.0 < interval < 1000.0, interval
    for bad in ((0, 256, 10), (256, 0, 10), (256, 2048, 10), (256, 256, 0)):
        with pytest.raises(woq.WoqError) as e:
            woq.woq_dispatch_floor(*bad, s)
        assert e.value.status == woq.WOQ_EINVAL


def test_allocation_failures_are_reported_and_release_everything(gpu_lib):
    """Allocation failure paths, forced from the host with requests larger
    than the device: a runner whose permuted-activation workspace would need
    about 1 TB, and a pager whose two slots would need 1 TB each, return
    WOQ_ENOMEM from create, and the device's free memory is where it was (the
    buffers allocated before the failing one are released)."""
    import ctypes
    import torch
    torch.cuda.synchronize()
    free0 = torch.cuda.mem_get_info()[0]
    # runner: one INT4O step over an input space of 2^33 channels at max_b = 64
    K = 1 << 33
    g = woq.woq_int4o_geometry(K)
    assert 64 * g.xp_len * 2 > 2 * torch.cuda.get_device_properties(0).total_memory
    dummy = torch.zeros(64, dtype=torch.uint8, device="cuda")
    st = woq.StackStep()
    st.fmt, st.in_slot, st.out_slot = woq.FMT_INT4O, 0, 0
    st.w4.codes = st.w4.scales = st.w4.w_out = dummy.data_ptr()
    st.w4.N, st.w4.geom = 16, g
    st.perm = dummy.data_ptr()
    h = ctypes.c_void_p()
    steps = (woq.StackStep * 1)(st)
    assert woq.lib().woq_stack_create(steps, 1, 64, ctypes.byref(h)) == woq.WOQ_ENOMEM
    assert not h.value
    # pager: one streamed INT8 layer whose block (and so each slot) is 1 TB
    pool = torch.zeros(4096, dtype=torch.uint8).pin_memory()
    q = np.zeros((64, 64), np.int8)
    ps = woq.PagerStep()
    ps.code_offset = 0
    ps.w.N, ps.w.K, ps.w.nseg = 64, 64, 1
    ps.w.seg_end[0], ps.w.seg_scale[0] = 64, 1.0
    off = (ctypes.c_int64 * 1)(0)
    nbytes = (ctypes.c_int64 * 1)(1 << 40)
    psteps = (woq.PagerStep * 1)(ps)
    hp = ctypes.c_void_p()
    rc = woq.lib().woq_pager_create(ctypes.c_void_p(pool.data_ptr()), off, nbytes, 1, psteps, 1, 1, ctypes.byref(hp))
    assert rc == woq.WOQ_ENOMEM, rc
    assert not hp.value
    assert woq.lib().woq_last_hip_error() == 2          # hipErrorOutOfMemory, kept by the library
    torch.cuda.synchronize()
    free1 = torch.cuda.mem_get_info()[0]
    print(f"free memory before {free0}, after {free1}", flush=True)
    assert free1 >= free0 - (4 << 20), (free0, free1)
    # the runtime's own error state is clear: the caller's next HIP work is unaffected
    t = torch.ones(1 << 20, device="cuda")
    torch.cuda.synchronize()
    assert float(t.sum()) == float(1 << 20)
    del q, t
