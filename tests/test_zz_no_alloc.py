"""The allocation-free split-K entry point (woq_qgemm_int4o_splitk_noalloc)
against woq_qgemm_int4o_splitk with a caller workspace: the same kernels, so
the same bits, on two calls in a row (the second smaller, so stale partial
sums of the first call would show), plus the size limit.  Both outputs are
also within tolerance of the oracle."""
import numpy as np
import pytest

import oracle as O
from weight_only_quantized_quantize_amd import woq

pytestmark = pytest.mark.gpu


def _case(N, K, b, splits, seed):
    import torch
    rng = np.random.default_rng(seed)
    g = woq.woq_int4o_geometry(K)
    perm = O.global_perm(K, np.sort(rng.choice(K, g.n_out, replace=False)))
    W = (rng.standard_normal((N, K)) * 0.02).astype(np.float32)
    dw = woq.DeviceInt4o([woq.woq_quantize_int4o(W, perm, g.n_out)], g)
    x = rng.standard_normal((b, K)).astype(np.float16)
    xp = torch.empty(b, g.xp_len, dtype=torch.float16, device="cuda")
    woq.woq_permute_x(torch.from_numpy(x).cuda(), torch.from_numpy(perm).cuda(), g, xp)
    rows = np.concatenate([np.arange(8), np.sort(rng.choice(N, 40, replace=False)), np.arange(N - 8, N)])
    c, s, wo = O.quantize_int4o(W[rows], perm, g.n_out)
    x_bg, x_out = O.permute_split(x, perm, g.n_out)
    return dw, xp, rows, O.linear_int4o(c, s, wo, x_bg, x_out)


def test_noalloc_splitk_equals_workspace_form_two_calls(gpu_lib):
    import torch
    cases = [(8192, 28672, 32, 8, 1), (1000, 3000, 5, 3, 2)]     # the second call is smaller
    for N, K, b, splits, seed in cases:
        print(f"case: noalloc split-K N={N} K={K} b={b} splits={splits}", flush=True)
        dw, xp, rows, ref = _case(N, K, b, splits, seed)
        y_ws = torch.full((b, N), 7.0, dtype=torch.float16, device="cuda")
        ws = torch.empty(woq.lib().woq_qgemm_int4o_splitk_workspace(N, b, splits) // 4, dtype=torch.float32,
                         device="cuda")
        woq.woq_qgemm_int4o_splitk(dw.desc, xp, y_ws, splits, ws)
        y_na = torch.full((b, N), 7.0, dtype=torch.float16, device="cuda")
        woq.woq_qgemm_int4o_splitk_noalloc(dw.desc, xp, y_na, splits)
        torch.cuda.synchronize()
        a, n = y_ws.cpu().numpy(), y_na.cpu().numpy()
        np.testing.assert_array_equal(n.view(np.uint16), a.view(np.uint16))
        err = O.normwise_rel_err(n[:, rows].astype(np.float64), ref)
        print(f"  normwise rel err {err:.3e}", flush=True)
        assert err <= 2e-3


def test_noalloc_splitk_refuses_more_than_its_workspace(gpu_lib):
    import torch
    N, K, b, splits = 8192, 256, 33, 8                 # 8 * 33 * 8192 * 4 B > 8 MiB
    g = woq.woq_int4o_geometry(K)
    assert splits * b * N * 4 > woq.SPLITK_NOALLOC_BYTES
    dw, xp, _, _ = _case(N, K, b, splits, 3)
    y = torch.full((b, N), 7.0, dtype=torch.float16, device="cuda")
    with pytest.raises(woq.WoqError) as e:
        woq.woq_qgemm_int4o_splitk_noalloc(dw.desc, xp, y, splits)
    assert e.value.status == woq.WOQ_EUNSUPPORTED
    torch.cuda.synchronize()
    assert np.all(y.cpu().numpy() == np.float16(7.0))   # nothing was launched
    del g
