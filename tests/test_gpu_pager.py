"""GPU tests of the streamed INT8 pager.

A streamed pass reads each layer out of a device slot that the copy stream
filled from pinned host memory; the products it launches are the resident
INT8 products, so every output must equal the resident runner's bit for bit,
whatever the relative timing of the two streams.  The outputs are also checked
against the oracle.
"""
import numpy as np
import pytest

import oracle as O
import synth
from weight_only_quantized_quantize_amd import woq
from weight_only_quantized_quantize_amd.stack import GROUPS, ResidentStack, StreamedInt8Stack

from test_gpu_stack import TOL, _case, host, io, oracle_group

pytestmark = pytest.mark.gpu

SLEEP_CYCLES = 20_000_000          # ~10 ms of spinning at the shader clock


def weight_fn(spec):
    return lambda l, lin, out: synth.weight(spec, l, lin, out=out)


def resident_outputs(spec, b, layers):
    rs = ResidentStack(spec, weight_fn(spec), layers=layers)
    ins, outs = io(spec, rs, b)
    runner = rs.make_runner(b)
    runner.bind(ins, outs)
    runner.run(b)
    return ins, [host(t).copy() for t in outs]


def streamed(spec, b, layers, ins, delay=None, passes=1):
    import torch
    ss = StreamedInt8Stack(spec, weight_fn(spec), layers=layers)
    outs = []
    for li in range(ss.n_layers):
        for gi, (names, _) in enumerate(GROUPS):
            outs.append(torch.full((b, sum(spec.linear(n).N for n in names)), 7.0, dtype=torch.float16,
                                   device="cuda"))
    pager = ss.make_pager(b)
    pager.bind(ins, outs)
    compute, copy = torch.cuda.Stream(), torch.cuda.Stream()
    torch.cuda.synchronize()
    results = []
    for p in range(passes):
        for t in outs:
            t.fill_(7.0)
        torch.cuda.synchronize()
        if delay == "copy":
            with torch.cuda.stream(copy):
                torch.cuda._sleep(SLEEP_CYCLES)      # every copy lands late
        elif delay == "compute":
            with torch.cuda.stream(compute):
                torch.cuda._sleep(SLEEP_CYCLES)      # the products start late
        pager.run(b, compute, copy)
        compute.synchronize()
        results.append([t.cpu().numpy() for t in outs])
    pager.close()
    torch.cuda.synchronize()
    return results


@pytest.mark.parametrize("b,layers", [(1, 5), (4, 5), (1, 1), (8, 2), (3, 4)])
def test_streamed_equals_resident(gpu_lib, b, layers):
    _case("streamed small stack", b, layers)
    spec = synth.small_stack_spec(3, layers=layers, batches=(b,))
    ins, ref = resident_outputs(spec, b, layers)
    (got,) = streamed(spec, b, layers, ins)
    assert len(got) == len(ref) == 4 * layers
    for i, (r, g) in enumerate(zip(ref, got)):
        np.testing.assert_array_equal(r.view(np.uint16), g.view(np.uint16), err_msg=f"step {i}")


@pytest.mark.parametrize("delay", ["copy", "compute"])
def test_streamed_late_stream_and_repeated_passes(gpu_lib, delay):
    """A copy stream held back before the pass (every layer's products must wait
    for its copy), or a compute stream held back (the first copies must wait for
    the slots to be free of the previous pass); three passes in a row."""
    _case("streamed late", delay)
    b, layers = 2, 6
    spec = synth.small_stack_spec(3, layers=layers, batches=(b,))
    ins, ref = resident_outputs(spec, b, layers)
    runs = streamed(spec, b, layers, ins, delay=delay, passes=3)
    for p, got in enumerate(runs):
        for i, (r, g) in enumerate(zip(ref, got)):
            np.testing.assert_array_equal(r.view(np.uint16), g.view(np.uint16), err_msg=f"pass {p} step {i}")


def test_streamed_matches_oracle(gpu_lib):
    _case("streamed vs oracle")
    b, layers = 4, 3
    spec = synth.small_stack_spec(3, layers=layers, batches=(b,))
    import torch
    ins = [torch.from_numpy(synth.decode_input(spec, l, inp, b)).cuda()
           for l in range(layers) for _, inp in GROUPS]
    (got,) = streamed(spec, b, layers, ins)
    for layer in range(layers):
        for gi, (names, inp) in enumerate(GROUPS):
            ref = oracle_group(spec, None, layer, names, inp, b)
            err = O.normwise_rel_err(got[4 * layer + gi].astype(np.float64), ref)
            print(f"layer {layer} {'|'.join(names)}: {err:.3e}", flush=True)
            assert err <= TOL


def test_streamed_9b_shapes(gpu_lib):
    """Three layers at the 9B INT8 stack's full shapes, batch 1: streamed equals
    resident bit for bit; sampled rows of the last layer match the oracle."""
    _case("streamed 9B shapes, 3 layers")
    spec = synth.stack_spec(3)
    b, layers = 1, 3
    ins, ref = resident_outputs(spec, b, layers)
    (got,) = streamed(spec, b, layers, ins)
    for i, (r, g) in enumerate(zip(ref, got)):
        np.testing.assert_array_equal(r.view(np.uint16), g.view(np.uint16), err_msg=f"step {i}")
    rng = np.random.default_rng(5)
    layer = layers - 1
    for gi, (names, inp) in enumerate(GROUPS):
        rows = {n: np.sort(rng.choice(spec.linear(n).N, 16, replace=False)) for n in names}
        r = oracle_group(spec, None, layer, names, inp, b, rows)
        offs, cols = 0, []
        for n in names:
            cols.extend(offs + rows[n])
            offs += spec.linear(n).N
        err = O.normwise_rel_err(got[4 * layer + gi][:, cols].astype(np.float64), r)
        print(f"layer {layer} {'|'.join(names)}: {err:.3e}", flush=True)
        assert err <= TOL


def test_pager_rejects_shared_stream_and_large_batch(gpu_lib):
    import torch
    spec = synth.small_stack_spec(3, layers=1, batches=(4,))
    ss = StreamedInt8Stack(spec, weight_fn(spec))
    pager = ss.make_pager(2)
    ins, outs = [], []
    for names, inp in GROUPS:
        ins.append(torch.from_numpy(synth.decode_input(spec, 0, inp, 4)).cuda())
        outs.append(torch.empty(4, sum(spec.linear(n).N for n in names), dtype=torch.float16, device="cuda"))
    pager.bind(ins, outs)
    s = torch.cuda.Stream()
    with pytest.raises(woq.WoqError) as e:
        pager.run(1, s, s)
    assert e.value.status == woq.WOQ_EINVAL
    with pytest.raises(woq.WoqError) as e:
        pager.run(3, s, torch.cuda.Stream())
    assert e.value.status == woq.WOQ_EINVAL
    pager.close()
