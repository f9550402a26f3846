"""GPU tests of the persisted pool: a stack saved by TieredStack.save_pool and
loaded by PooledStack (no weight encoded again) must give the resident
runner's outputs bit for bit, for any tier plan made at load time."""
import numpy as np
import pytest

import synth
from weight_only_quantized_quantize_amd import woq
from weight_only_quantized_quantize_amd.stack import PooledStack, TieredStack

from test_gpu_tiered import assert_same, io, resident_ref, tiered_run, wfn
from test_gpu_stack import _case

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("cfg,b", [(2, 1), (2, 8), (3, 1), (3, 4)])
def test_pool_roundtrip_equals_resident(gpu_lib, tmp_path, cfg, b):
    _case("pool roundtrip", cfg, b)
    layers = 5
    spec = synth.small_stack_spec(cfg, layers=layers, batches=(b,))
    rs, ins, ref = resident_ref(spec, b, layers)
    ts = TieredStack(spec, wfn(spec), None, 0, layers=layers, resident=[0] * layers, perms=rs.perm_host or None)
    path = str(tmp_path / "stack.woqpool")
    ts.save_pool(path)
    del ts
    for resident in ([0] * layers, [1] * layers, [1, 0, 1, 0, 0]):
        ps = PooledStack(path, resident=resident)
        assert ps.n_resident == sum(resident)
        (got,) = tiered_run(ps, spec, b, ins)
        assert_same(ref, got, f"pool {resident}")
    probe = PooledStack(path, resident=[1] * layers)
    ps = PooledStack(path, budget_bytes=4 * probe.block_bytes)
    assert list(ps.resident) == [1, 1, 0, 0, 0]
    (got,) = tiered_run(ps, spec, b, ins)
    assert_same(ref, got, "pool planned")


def test_pool_damaged_block_is_refused(gpu_lib, tmp_path):
    spec = synth.small_stack_spec(2, layers=2, batches=(1,))
    ts = TieredStack(spec, wfn(spec), lambda s: synth.profile(spec, s), 0, layers=2, resident=[0, 0])
    path = str(tmp_path / "stack.woqpool")
    ts.save_pool(path)
    raw = bytearray(open(path, "rb").read())
    off = int(np.frombuffer(bytes(raw[32 + 24 * 2: 32 + 24 * 2 + 8]), np.uint64)[0])   # block 2: permutations
    raw[off + 3] ^= 0x40
    open(path, "wb").write(bytes(raw))
    with pytest.raises(woq.WoqError) as e:
        PooledStack(path, resident=[1, 1])
    assert e.value.status == woq.WOQ_EFORMAT
    with pytest.raises(ValueError):
        TieredStack(spec, wfn(spec), None, 0, layers=2, resident=[1, 0], perms=ts.perm_host).save_pool(path)
