"""GPU tests of the on-device encoders: INT8 and outlier-aware INT4 encodings
computed by the GPU from fp32 weights in device memory, written into the
device layouts.  Compared bit for bit with the oracle's encoding (through the
host layout inverse) and with the host library's layout, including the
hand-derived tie tables and the error cases."""
import numpy as np
import pytest

import oracle as O
import synth
from conftest import read_golden
from weight_only_quantized_quantize_amd import woq

pytestmark = pytest.mark.gpu


def _case(*a):
    print("case:", *a, flush=True)


def dev_int8(W):
    """(layout bytes, scale, status) from the device encoder."""
    import torch
    N, K = W.shape
    Wd = torch.from_numpy(np.ascontiguousarray(W, np.float32)).cuda()
    dev = torch.full((woq.lib().woq_int8_dev_bytes(N, K),), 0x5A, dtype=torch.uint8, device="cuda")
    scale = torch.full((1,), 3.0, dtype=torch.float32, device="cuda")
    status = torch.full((1,), 99, dtype=torch.int32, device="cuda")
    woq.woq_quantize_int8_dev(Wd, dev, scale, status)
    torch.cuda.synchronize()
    return dev.cpu().numpy(), np.float32(scale.cpu().numpy()[0]), int(status.cpu().numpy()[0])


def dev_int4o(W, perm, n_out=-1):
    import torch
    N, K = W.shape
    g = woq.woq_int4o_geometry(K, n_out)
    cb, sb, wb = woq.woq_int4o_dev_sizes(N, g)
    codes = torch.full((cb,), 0x5A, dtype=torch.uint8, device="cuda")
    scales = torch.full((sb // 2,), 0x5A5A, dtype=torch.int16, device="cuda")
    w_out = torch.full((wb // 2,), 0x5A5A, dtype=torch.int16, device="cuda") if wb else None
    status = torch.full((1,), 99, dtype=torch.int32, device="cuda")
    woq.woq_quantize_int4o_dev(torch.from_numpy(np.ascontiguousarray(W, np.float32)).cuda(),
                               torch.from_numpy(np.ascontiguousarray(perm, np.int32)).cuda(), g,
                               codes, scales, w_out, status)
    torch.cuda.synchronize()
    return (g, codes.cpu().numpy(), scales.cpu().numpy().view(np.uint16),
            w_out.cpu().numpy().view(np.uint16) if w_out is not None else np.zeros(0, np.uint16),
            int(status.cpu().numpy()[0]))


@pytest.mark.parametrize("N,K,seed", [(1, 1, 0), (3, 130, 1), (17, 257, 2), (300, 4096, 3), (4, 64, 4)])
def test_int8_device_encoder_matches_oracle_and_host(gpu_lib, N, K, seed):
    _case("int8 device encoder", N, K)
    rng = np.random.default_rng(seed)
    W = (rng.standard_normal((N, K)) * 0.02).astype(np.float32)
    dev, s, st = dev_int8(W)
    assert st == 0
    q_ref, s_ref = O.quantize_int8(W)
    assert s.view(np.uint32) == np.float32(s_ref).view(np.uint32)
    np.testing.assert_array_equal(woq.woq_layout_int8_inverse(dev, N, K), q_ref)
    q_host, s_host = woq.woq_quantize_int8(W)
    np.testing.assert_array_equal(dev, woq.woq_layout_int8(q_host))     # padding included


def test_int8_device_encoder_ties_table(gpu_lib):
    """The hand-derived tie table of the INT8 encoding (round half to even)."""
    rows = [ln.split() for ln in read_golden("int8_ties.txt")]
    W = np.array([[float(r[0]) for r in rows]], np.float32)
    want = np.array([[int(r[1]) for r in rows]], np.int8)
    dev, s, st = dev_int8(W)
    assert st == 0 and s == np.float32(2.0 ** -7)
    np.testing.assert_array_equal(woq.woq_layout_int8_inverse(dev, 1, W.shape[1]), want)


def test_int8_device_encoder_zero_and_nonfinite(gpu_lib):
    dev, s, st = dev_int8(np.zeros((5, 70), np.float32))
    assert st == 0 and s == 0 and np.all(dev == 128)
    W = np.ones((3, 40), np.float32)
    W[1, 7] = np.inf
    dev, s, st = dev_int8(W)
    assert st == woq.WOQ_ERANGE and np.isnan(s) and np.all(dev == 128)
    W[1, 7] = np.nan
    dev, s, st = dev_int8(W)
    assert st == woq.WOQ_ERANGE and np.isnan(s)


def int4o_case(W, perm, n_out):
    g, codes, scales, w_out, st = dev_int4o(W, perm, n_out)
    assert st == 0
    N = W.shape[0]
    packed, sc, wo = woq.woq_layout_int4o_inverse(codes, scales, w_out, N, g)
    c_ref, s_ref, wo_ref = O.quantize_int4o(W, perm, g.n_out)
    np.testing.assert_array_equal(woq.woq_unpack_int4(packed), c_ref)
    np.testing.assert_array_equal(sc.view(np.uint16), s_ref.view(np.uint16))
    np.testing.assert_array_equal(wo.view(np.uint16), wo_ref.view(np.uint16))
    hp, hs, hw = woq.woq_quantize_int4o(W, perm, g.n_out)
    hc, hsd, hwd = woq.woq_layout_int4o(hp, hs, hw, g)
    np.testing.assert_array_equal(codes, hc)                             # padding included
    np.testing.assert_array_equal(scales, hsd)
    np.testing.assert_array_equal(w_out, hwd)


@pytest.mark.parametrize("N,K,n_out,seed", [(1, 130, -1, 0), (17, 257, -1, 1), (33, 3072, -1, 2), (5, 300, 3, 3),
                                            (16, 256, 0, 4), (40, 1000, 10, 5), (3, 16, 16, 6)])
def test_int4o_device_encoder_matches_oracle_and_host(gpu_lib, N, K, n_out, seed):
    _case("int4o device encoder", N, K, n_out)
    rng = np.random.default_rng(seed)
    g = woq.woq_int4o_geometry(K, n_out)
    outs = np.sort(rng.choice(K, g.n_out, replace=False))
    W = (rng.standard_normal((N, K)) * 0.02).astype(np.float32)
    W[:, outs] *= 10
    if N > 2:
        W[2, :] = 0.0                     # an all-zero row: every scale 0
    perm = O.global_perm(K, outs).astype(np.int32)
    int4o_case(W, perm, g.n_out)


def test_int4o_device_encoder_ties_table(gpu_lib):
    rows = [ln.split() for ln in read_golden("int4_ties.txt")]
    W = np.zeros((1, 128), np.float32)
    W[0, :len(rows)] = [float(r[0]) for r in rows]
    want = np.array([int(r[1]) for r in rows], np.int8)
    perm = np.arange(128, dtype=np.int32)
    g, codes, scales, w_out, st = dev_int4o(W, perm, 0)
    assert st == 0
    packed, sc, _ = woq.woq_layout_int4o_inverse(codes, scales, w_out, 1, g)
    assert sc[0, 0] == np.float16(2.0 ** -8)
    q = woq.woq_unpack_int4(packed)[0]
    np.testing.assert_array_equal(q[:len(want)], want)
    assert not q[len(want):].any()


def test_int4o_device_encoder_errors(gpu_lib):
    K = 300
    rng = np.random.default_rng(9)
    W = (rng.standard_normal((4, K)) * 0.02).astype(np.float32)
    perm = O.global_perm(K, np.arange(3)).astype(np.int32)
    W2 = W.copy()
    W2[1, 100] = np.nan
    assert dev_int4o(W2, perm, 3)[-1] == woq.WOQ_ERANGE
    W3 = W.copy()
    W3[0, 50] = 1e6                       # group scale 1e6 / 7 overflows fp16
    assert dev_int4o(W3, perm, 3)[-1] == woq.WOQ_ERANGE
    bad = perm.copy()
    bad[10] = K + 5
    assert dev_int4o(W, bad, 3)[-1] == woq.WOQ_EINVAL
    bad = perm.copy()
    bad[K - 1] = -1                       # an outlier slot
    assert dev_int4o(W, bad, 3)[-1] == woq.WOQ_EINVAL


def test_int4o_device_encoder_70b_gate_size(gpu_lib):
    """A full 70B-shaped gate weight (28672 x 8192): device layout equal to the
    host library's, and sampled rows equal to the oracle's encoding."""
    spec = synth.stack_spec(4)
    _case("int4o device encoder 70B gate")
    W = synth.weight(spec, 0, "gate")
    perm = O.global_perm(W.shape[1], synth.planted_set(spec, "h")).astype(np.int32)
    g, codes, scales, w_out, st = dev_int4o(W, perm)
    assert st == 0
    hp, hs, hw = woq.woq_quantize_int4o(W, perm, g.n_out)
    hc, hsd, hwd = woq.woq_layout_int4o(hp, hs, hw, g)
    np.testing.assert_array_equal(codes, hc)
    np.testing.assert_array_equal(scales, hsd)
    np.testing.assert_array_equal(w_out, hwd)
    rows = np.sort(np.random.default_rng(1).choice(W.shape[0], 8, replace=False))
    c_ref, s_ref, wo_ref = O.quantize_int4o(W[rows], perm, g.n_out)
    np.testing.assert_array_equal(woq.woq_unpack_int4(hp[rows]), c_ref)
    np.testing.assert_array_equal(hs[rows].view(np.uint16), s_ref.view(np.uint16))
