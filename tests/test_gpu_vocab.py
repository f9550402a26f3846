"""GPU tests of the vocabulary matrix on both sides of the stack: the INT8
token lookup (bit-exact against the oracle) and the tied outlier-aware INT4
lm_head (sampled rows against the oracle), at the 3B-shaped vocabulary
128256 x 3072 and on small ragged tables."""
import numpy as np
import pytest

import oracle as O
import synth
from weight_only_quantized_quantize_amd import woq
from weight_only_quantized_quantize_amd.stack import TiedVocab

pytestmark = pytest.mark.gpu

TOL = 2e-3


def _case(*a):
    print("case:", *a, flush=True)


def _host(t):
    import torch
    torch.cuda.synchronize()
    return t.cpu().numpy()


def lookup_ref(E, ids):
    """Oracle lookup of ids from the INT8 table of E, quantising only the rows
    the ids touch (the scale still comes from the whole table)."""
    V = E.shape[0]
    ids = np.asarray(ids, np.int64)
    valid = np.unique(ids[(ids >= 0) & (ids < V)])
    q, s = O.quantize_int8(E, rows=valid)
    where = {int(t): i for i, t in enumerate(valid)}
    local = np.array([where.get(int(t), -1) for t in ids], np.int64)
    return O.embed_int8(q, s, local)


def run_lookup(E, ids, ldy=None):
    import torch
    q, s = woq.woq_quantize_int8(E)
    table = woq.DeviceInt8([(q, s)])
    b, H = len(ids), E.shape[1]
    ldy = ldy or -(-H // 8) * 8
    y = torch.full((b, ldy), 7.0, dtype=torch.float16, device="cuda")
    woq.woq_embed_int8(table.desc, torch.from_numpy(np.asarray(ids, np.int32)).cuda(), y)
    return _host(y)


@pytest.mark.parametrize("V,H,ldy", [(1000, 200, 208), (17, 8, 8), (300, 3072, 3072), (5, 64, 72)])
def test_lookup_small_tables_bit_exact(gpu_lib, V, H, ldy):
    """Every row of small tables (ragged widths included), ids repeated and
    out of range; the padding of each output row beyond H is left alone."""
    _case("lookup", V, H, ldy)
    rng = np.random.default_rng(V + H)
    E = rng.standard_normal((V, H)).astype(np.float32) * np.float32(0.02)
    ids = np.concatenate([np.arange(V), rng.integers(0, V, 40), [-1, V, 2 ** 31 - 1, -(2 ** 31)]]).astype(np.int32)
    y = run_lookup(E, ids, ldy)
    ref = lookup_ref(E, ids)
    np.testing.assert_array_equal(y[:, :H].view(np.uint16), ref.view(np.uint16))
    assert np.all(y[:, H:] == 7.0)


def test_lookup_double_rounding_case(gpu_lib):
    """A table whose scale and codes make the fp32 product land on an fp16 tie
    (the hand-derived case of the oracle's pins): the lookup must round twice."""
    import torch
    m = 13951508
    s = np.float32(m * 2.0 ** -30)
    q = np.array([[77, -77, 127, 0, 3, -3, 1, -1]], np.int8)
    table = woq.DeviceInt8([(q, s)])
    y = torch.empty((1, 8), dtype=torch.float16, device="cuda")
    woq.woq_embed_int8(table.desc, torch.zeros(1, dtype=torch.int32, device="cuda"), y)
    got = _host(y)
    ref = O.embed_int8(q, s, [0])
    np.testing.assert_array_equal(got.view(np.uint16), ref.view(np.uint16))
    assert got[0, 0] == 1.0 and got[0, 1] == -1.0


def test_lookup_argument_errors(gpu_lib):
    import torch
    q = np.ones((4, 16), np.int8)
    table = woq.DeviceInt8([(q, np.float32(0.5))])
    ids = torch.zeros(2, dtype=torch.int32, device="cuda")
    with pytest.raises(woq.WoqError) as e:
        woq.woq_embed_int8(table.desc, ids, torch.empty((2, 8), dtype=torch.float16, device="cuda"))
    assert e.value.status == woq.WOQ_EINVAL                     # ldy < H
    with pytest.raises(woq.WoqError) as e:
        woq.woq_embed_int8(table.desc, ids, torch.empty((2, 20), dtype=torch.float16, device="cuda"))
    assert e.value.status == woq.WOQ_EALIGN                     # ldy not a multiple of 8
    woq.woq_embed_int8(table.desc, ids[:0], torch.empty((0, 16), dtype=torch.float16, device="cuda"))


@pytest.fixture(scope="module")
def vocab_3b():
    """The 3B-shaped tied vocabulary matrix (128256 x 3072) and the hidden
    space's permutation, selected by the library from the matrix's column
    sums and the hidden profile."""
    spec = synth.stack_spec(2)
    E = synth.embedding(spec)
    colsum = woq.woq_colabs_accumulate(E, np.zeros(E.shape[1]))
    perm = woq.woq_outlier_select(colsum, synth.profile(spec, "h"))
    return spec, E, perm


def test_vocab_3b_perm_is_planted_set(gpu_lib, vocab_3b):
    spec, E, perm = vocab_3b
    np.testing.assert_array_equal(perm, O.global_perm(E.shape[1], synth.planted_set(spec, "h")))


@pytest.mark.parametrize("b", [1, 32])
def test_lookup_vocab_3b_bit_exact(gpu_lib, vocab_3b, b):
    spec, E, _ = vocab_3b
    _case("lookup 3B vocab", b)
    rng = np.random.default_rng(b)
    ids = rng.integers(0, E.shape[0], b).astype(np.int32)
    ids[0] = E.shape[0] - 1
    if b > 2:
        ids[1], ids[2] = -5, E.shape[0]
    y = run_lookup(E, ids)
    np.testing.assert_array_equal(y.view(np.uint16), lookup_ref(E, ids).view(np.uint16))


def head_input(spec, b, seed):
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((b, spec.hidden)).astype(np.float32)
    x[:, synth.planted_set(spec, "h")] *= np.float32(spec.x_planted_gain)
    return x.astype(np.float16)


@pytest.fixture(scope="module")
def tied_3b(vocab_3b):
    spec, E, perm = vocab_3b
    return TiedVocab(E, perm, max_b=32)


@pytest.mark.parametrize("b", [1, 4, 8, 32])
def test_lm_head_vocab_3b_sampled_rows(gpu_lib, vocab_3b, tied_3b, b):
    """Tied lm_head over the 3B vocabulary: the INT4O product at N = 128256
    (vector kernel at b = 1, matrix-core kernel above), sampled output rows
    against the oracle (which quantises just those rows)."""
    import torch
    spec, E, perm = vocab_3b
    _case("lm_head 3B vocab", b)
    tv = tied_3b
    x = head_input(spec, b, 100 + b)
    y = torch.full((b, tv.V), 7.0, dtype=torch.float16, device="cuda")
    tv.logits(torch.from_numpy(x).cuda(), y)
    got = _host(y)
    assert np.all(np.isfinite(got))
    rng = np.random.default_rng(b)
    rows = np.sort(np.concatenate([rng.choice(tv.V, 96, replace=False), [0, tv.V - 1]]))
    rows = np.unique(rows)
    g = O.int4o_geometry(E.shape[1])
    x_bg, x_out = O.permute_split(x, perm, g["n_out"])
    c, s, wo = O.quantize_int4o(E[rows], perm, g["n_out"])
    ref = O.linear_int4o(c, s, wo, x_bg, x_out)
    err = O.normwise_rel_err(got[:, rows].astype(np.float64), ref)
    print(f"lm_head b={b}: normwise rel err {err:.3e}", flush=True)
    assert err <= TOL
    # the table lookup of the same tied matrix
    ids = torch.from_numpy(np.arange(b, dtype=np.int32) * 997).cuda()
    emb = torch.empty((b, tv.H), dtype=torch.float16, device="cuda")
    tv.embed(ids, emb)
    np.testing.assert_array_equal(_host(emb).view(np.uint16),
                                  lookup_ref(E, np.arange(b) * 997).view(np.uint16))
