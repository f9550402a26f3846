"""Build a resident decode stack on the GPU and run it through libwoq.

Host orchestration only: weights come from a caller-supplied generator, every
quantisation / selection / packing / layout step is a libwoq call, and the
decode pass is ``woq_stack_run``.  Per layer there are four launches groups,
each one N-stacked product: q|k|v (hidden input), o (attention output),
gate|up (hidden input), down (intermediate input).
"""
from __future__ import annotations

import json
import os
import threading
from concurrent.futures import ThreadPoolExecutor

import numpy as np

from . import woq

GROUPS = ((("q", "k", "v"), 0), (("o",), 1), (("gate", "up"), 2), (("down",), 3))


def _map_weights(spec, jobs, weight_fn, fn, threads):
    """Run fn(layer, lin, W) over jobs with W drawn into per-thread buffers."""
    jobs = list(jobs)
    if not jobs:
        return []
    maxel = max(lin.N * lin.K for _, lin in jobs)
    local = threading.local()

    def run(job):
        layer, lin = job
        buf = getattr(local, "buf", None)
        if buf is None:
            buf = local.buf = np.ones(maxel, np.float32)
        W = buf[: lin.N * lin.K].reshape(lin.N, lin.K)
        weight_fn(layer, lin, W)
        return fn(layer, lin, W)

    with ThreadPoolExecutor(threads) as ex:
        return list(ex.map(run, jobs))


def _concat(parts, i):
    return np.concatenate([p[i] for p in parts]) if len(parts) > 1 else parts[0][i]


class _QuantisedStack:
    """Global permutations (INT4O) and per-layer quantisation, shared by the
    resident and tiered stacks.

    spec: object with .fmt ("int8" | "int4o"), .layers, .linears(),
          .space_width(space), .bmax
    weight_fn(layer, lin, out): fill ``out`` (float32 [N, K]) with the weight
    profile_fn(space): fp16 activation profile [T, K] of an input space
    """

    def _setup(self, spec, weight_fn, profile_fn, device, threads, layers, log, perms=None):
        import torch
        self.spec = spec
        self.device = device
        self.fmt = spec.fmt
        self.n_layers = spec.layers if layers is None else layers
        self.threads = threads or min(16, os.cpu_count() or 1)
        self.log = log or (lambda *a: None)
        self.weight_fn = weight_fn
        self.perm_host = {}
        self.perm_dev = {}
        self.geom = {}
        if self.fmt == "int4o" and perms is not None:
            for space, perm in perms.items():           # permutations chosen elsewhere (e.g. another stack)
                self.perm_host[space] = np.ascontiguousarray(perm, np.int32)
                self.perm_dev[space] = torch.from_numpy(self.perm_host[space]).to(device)
                self.geom[space] = woq.woq_int4o_geometry(spec.space_width(space))
        elif self.fmt == "int4o":
            spaces = sorted({l.space for l in spec.linears()})
            jobs = [(layer, lin) for layer in range(spec.layers) for lin in spec.linears()]
            self.log(f"column sums over {len(jobs)} weights")

            def colsum(layer, lin, W):
                return woq.woq_colabs_accumulate(W, np.zeros(lin.K))

            sums = _map_weights(spec, jobs, weight_fn, colsum, self.threads)
            for space in spaces:
                K = spec.space_width(space)
                # the library adds the per-linear sums in (layer, linear) order and selects
                parts = [cs for (layer, lin), cs in zip(jobs, sums) if lin.space == space]
                perm = woq.woq_outlier_perm_sums(parts, profile_fn(space))
                self.perm_host[space] = perm
                self.perm_dev[space] = torch.from_numpy(perm).to(device)
                self.geom[space] = woq.woq_int4o_geometry(K)

    def _quantised_layers(self, layer_ids):
        """Yield (layer, [(names, input index, parts)]) in layer order, four
        layers quantised at a time."""
        spec = self.spec
        layer_ids = list(layer_ids)
        for c0 in range(0, len(layer_ids), 4):
            ls = layer_ids[c0:c0 + 4]
            jobs = [(layer, lin) for layer in ls for lin in spec.linears()]
            self.log(f"quantising layers {ls[0]}..{ls[-1]}")
            if self.fmt == "int4o":
                res = _map_weights(spec, jobs, self.weight_fn,
                                   lambda layer, lin, W: woq.woq_quantize_int4o(W, self.perm_host[lin.space]),
                                   self.threads)
            else:
                res = _map_weights(spec, jobs, self.weight_fn, lambda layer, lin, W: woq.woq_quantize_int8(W),
                                   self.threads)
            got = {(layer, lin.name): r for (layer, lin), r in zip(jobs, res)}
            del res
            for layer in ls:
                yield layer, [(names, inp, [got.pop((layer, n)) for n in names]) for names, inp in GROUPS]

    def _space(self, names):
        return self.spec.linear(names[0]).space

    def _device(self, names, parts):
        if self.fmt == "int4o":
            return woq.DeviceInt4o(parts, self.geom[self._space(names)], self.device)
        return woq.DeviceInt8(parts, self.device)

    def _resident_step(self, names, dev, slot):
        if self.fmt == "int4o":
            return woq.step_int4o(dev, self.perm_dev[self._space(names)], slot, slot)
        return woq.step_int8(dev, slot, slot)


class ResidentStack(_QuantisedStack):
    """All layers of a stack resident in HBM plus the runner."""

    def __init__(self, spec, weight_fn, profile_fn=None, device="cuda", threads=None, layers=None, log=None,
                 perms=None):
        self._setup(spec, weight_fn, profile_fn, device, threads, layers, log, perms)
        self.layers = []          # per layer: list of (group names, input index, device weight)
        for layer, groups in self._quantised_layers(range(self.n_layers)):
            self.layers.append([(names, inp, self._device(names, parts)) for names, inp, parts in groups])
        self.runner = None

    def steps(self):
        out = []
        for layer, groups in enumerate(self.layers):
            for gi, (names, inp, dev) in enumerate(groups):
                out.append(self._resident_step(names, dev, 4 * layer + gi))
        return out

    def make_runner(self, max_b: int):
        self.runner = woq.Stack(self.steps(), max_b)
        return self.runner

    def group_shapes(self):
        """(N, K) of every launch in step order."""
        shapes = []
        for groups in self.layers:
            for names, inp, dev in groups:
                shapes.append((dev.N, self.spec.linear(names[0]).K, names))
        return shapes

    def device_bytes(self) -> int:
        tot = 0
        for groups in self.layers:
            for _, _, dev in groups:
                for t in ("codes", "scales", "w_out"):
                    x = getattr(dev, t, None)
                    if x is not None:
                        tot += x.numel() * x.element_size()
        return tot


def _align(n: int, a: int = 256) -> int:
    return -(-n // a) * a


class TieredStack(_QuantisedStack):
    """A stack split by woq_plan_tiers under a device-memory budget: the first
    layers resident in HBM (tier A), the rest in one pinned host pool (tier B)
    streamed through the pager's two slots.  Works for both formats.

    A streamed layer's block holds, for q|k|v, o, gate|up and down in turn, the
    device layout arrays (INT4O: codes, scales, outlier weights; INT8: codes),
    each at a 256-byte aligned offset."""

    def __init__(self, spec, weight_fn, profile_fn, budget_bytes: int, device="cuda", threads=None, layers=None,
                 log=None, resident=None, perms=None):
        import torch
        self._setup(spec, weight_fn, profile_fn, device, threads, layers, log, perms)
        # block layout of one layer (identical for every layer)
        self.array_offsets = []        # per group: offsets of its arrays in the block
        o = 0
        for names, _ in GROUPS:
            N = sum(spec.linear(n).N for n in names)
            if self.fmt == "int4o":
                sizes = woq.woq_int4o_dev_sizes(N, self.geom[self._space(names)])
            else:
                sizes = (woq.lib().woq_int8_dev_bytes(N, spec.linear(names[0]).K),)
            offs = []
            for sz in sizes:
                offs.append(o)
                o += _align(sz)
            self.array_offsets.append(offs)
        self.block_bytes = o
        if resident is None:
            resident, self.planned_device_bytes = woq.woq_plan_tiers([o] * self.n_layers, budget_bytes)
        self.resident = np.asarray(resident, np.int32)
        if self.resident.shape != (self.n_layers,):
            raise ValueError(f"resident needs one flag per layer ({self.n_layers})")
        streamed = [l for l in range(self.n_layers) if not self.resident[l]]
        self.pool = torch.empty(max(1, len(streamed) * o), dtype=torch.uint8, pin_memory=True)
        pool_np = self.pool.numpy()
        self.layer_off = [0] * self.n_layers
        self.layer_bytes = [0] * self.n_layers
        for j, l in enumerate(streamed):
            self.layer_off[l] = j * o
            self.layer_bytes[l] = o
        self.devices = {}
        self.step_list = []
        for layer, groups in self._quantised_layers(range(self.n_layers)):
            for gi, (names, inp, parts) in enumerate(groups):
                slot = 4 * layer + gi
                if self.resident[layer]:
                    dev = self._device(names, parts)
                    self.devices[slot] = dev
                    self.step_list.append(self._resident_step(names, dev, slot))
                    continue
                base = self.layer_off[layer]
                offs = self.array_offsets[gi]
                st = woq.StackStep()
                st.in_slot = st.out_slot = slot
                if self.fmt == "int4o":
                    g = self.geom[self._space(names)]
                    arrays = woq.woq_layout_int4o(_concat(parts, 0), _concat(parts, 1), _concat(parts, 2), g)
                    for a, off in zip(arrays, offs):
                        v = a.view(np.uint8)
                        pool_np[base + off: base + off + v.size] = v
                    st.fmt = woq.FMT_INT4O
                    st.w4.codes, st.w4.scales, st.w4.w_out = offs
                    st.w4.N = sum(p[0].shape[0] for p in parts)
                    st.w4.geom = g
                    st.perm = self.perm_dev[self._space(names)].data_ptr()
                else:
                    q = _concat(parts, 0)
                    v = woq.woq_layout_int8(q)
                    pool_np[base + offs[0]: base + offs[0] + v.size] = v
                    st.fmt = woq.FMT_INT8
                    st.w8.codes = offs[0]
                    st.w8.N, st.w8.K, st.w8.nseg = q.shape[0], q.shape[1], len(parts)
                    end = 0
                    for i, (qi, sc) in enumerate(parts):
                        end += qi.shape[0]
                        st.w8.seg_end[i] = end
                        st.w8.seg_scale[i] = float(sc)
                self.step_list.append(st)

    @property
    def n_resident(self) -> int:
        return int(self.resident.sum())

    def streamed_bytes(self) -> int:
        return sum(self.layer_bytes)

    def make_pager(self, max_b: int):
        return woq.Pager(self.pool, self.layer_off, self.layer_bytes, self.step_list, len(GROUPS), max_b)

    def save_pool(self, path: str):
        """Persist the encoded stack: every layer's block plus the global
        permutations, with what a loader needs to rebuild the steps.  Every
        layer must be streamed (built with resident all 0), so that its block
        is in the host pool."""
        if self.n_resident:
            raise ValueError("save_pool needs every layer in the host pool (resident all 0)")
        spec = self.spec
        groups = []
        for gi, (names, inp) in enumerate(GROUPS):
            lin = spec.linear(names[0])
            groups.append({"names": list(names), "input": inp, "K": lin.K, "space": lin.space,
                           "N": sum(spec.linear(n).N for n in names), "offsets": self.array_offsets[gi]})
        int8 = []
        if self.fmt == "int8":
            for layer in range(self.n_layers):
                row = []
                for gi in range(len(GROUPS)):
                    w = self.step_list[4 * layer + gi].w8
                    row.append({"seg_end": [w.seg_end[i] for i in range(w.nseg)],
                                "seg_scale_bits": [int(np.float32(w.seg_scale[i]).view(np.uint32))
                                                   for i in range(w.nseg)]})
                int8.append(row)
        spaces, perm_parts, o = {}, [], 0
        for sp in sorted(self.perm_host):
            p = np.ascontiguousarray(self.perm_host[sp], np.int32)
            spaces[sp] = [o, int(p.size), int(self.geom[sp].n_out)]
            perm_parts.append(p)
            o += p.size
        perms = np.concatenate(perm_parts).view(np.uint8) if perm_parts else np.zeros(0, np.uint8)
        meta = {"kind": "woq stack pool", "fmt": self.fmt, "workload": spec.name, "n_layers": self.n_layers,
                "steps_per_layer": len(GROUPS), "block_bytes": self.block_bytes, "groups": groups,
                "int8_segments": int8, "perm_spaces": spaces}
        pool = self.pool.numpy()
        blocks = [pool[self.layer_off[l]: self.layer_off[l] + self.block_bytes] for l in range(self.n_layers)]
        woq.woq_pool_save(path, json.dumps(meta).encode(), blocks + [perms])


class PooledStack:
    """A stack loaded from a pool file written by TieredStack.save_pool: no
    weight is encoded again.  The tier plan is made at load time (budget, or an
    explicit resident list): resident layers are read through one pinned
    staging block into device memory, streamed layers straight into the
    pinned pool the pager copies from."""

    def __init__(self, path: str, budget_bytes: int | None = None, resident=None, device="cuda"):
        import torch
        raw, sizes = woq.woq_pool_info(path)
        meta = json.loads(raw.decode())
        if meta.get("kind") != "woq stack pool":
            raise ValueError("not a stack pool")
        self.meta = meta
        self.fmt = meta["fmt"]
        L, B = meta["n_layers"], meta["block_bytes"]
        self.n_layers, self.block_bytes = L, B
        perms = np.empty(sizes[L], np.uint8)
        woq.woq_pool_read_block(path, L, perms)
        perms = perms.view(np.int32)
        self.perm_host, self.perm_dev, self.geom = {}, {}, {}
        for sp, (o, K, n_out) in meta["perm_spaces"].items():
            self.perm_host[sp] = perms[o:o + K].copy()
            self.perm_dev[sp] = torch.from_numpy(self.perm_host[sp]).to(device)
            self.geom[sp] = woq.woq_int4o_geometry(K, n_out)
        if resident is None:
            resident, self.planned_device_bytes = woq.woq_plan_tiers([B] * L, budget_bytes)
        self.resident = np.asarray(resident, np.int32)
        if self.resident.shape != (L,):
            raise ValueError(f"resident needs one flag per layer ({L})")
        streamed = [l for l in range(L) if not self.resident[l]]
        self.pool = torch.empty(max(1, len(streamed) * B), dtype=torch.uint8, pin_memory=True)
        pool_np = self.pool.numpy()
        self.layer_off, self.layer_bytes = [0] * L, [0] * L
        self.device_blocks = {}
        staging = torch.empty(B, dtype=torch.uint8, pin_memory=True) if len(streamed) < L else None
        for l in range(L):
            if self.resident[l]:
                woq.woq_pool_read_block(path, l, staging.numpy())
                d = torch.empty(B, dtype=torch.uint8, device=device)
                d.copy_(staging)                       # synchronous: the staging block is reused
                self.device_blocks[l] = d
            else:
                j = streamed.index(l)
                self.layer_off[l], self.layer_bytes[l] = j * B, B
                woq.woq_pool_read_block(path, l, pool_np[j * B:(j + 1) * B])
        self.step_list = []
        for l in range(L):
            base = self.device_blocks[l].data_ptr() if self.resident[l] else 0
            for gi, gr in enumerate(meta["groups"]):
                st = woq.StackStep()
                st.in_slot = st.out_slot = 4 * l + gi
                offs = gr["offsets"]
                if self.fmt == "int4o":
                    st.fmt = woq.FMT_INT4O
                    st.w4.codes, st.w4.scales, st.w4.w_out = (base + o for o in offs)
                    st.w4.N = gr["N"]
                    st.w4.geom = self.geom[gr["space"]]
                    st.perm = self.perm_dev[gr["space"]].data_ptr()
                else:
                    seg = meta["int8_segments"][l][gi]
                    st.fmt = woq.FMT_INT8
                    st.w8.codes = base + offs[0]
                    st.w8.N, st.w8.K, st.w8.nseg = gr["N"], gr["K"], len(seg["seg_end"])
                    for i, (e, sb) in enumerate(zip(seg["seg_end"], seg["seg_scale_bits"])):
                        st.w8.seg_end[i] = e
                        st.w8.seg_scale[i] = float(np.uint32(sb).view(np.float32))
                self.step_list.append(st)

    @property
    def n_resident(self) -> int:
        return int(self.resident.sum())

    def streamed_bytes(self) -> int:
        return sum(self.layer_bytes)

    def make_pager(self, max_b: int):
        return woq.Pager(self.pool, self.layer_off, self.layer_bytes, self.step_list, len(GROUPS), max_b)


class StreamedInt8Stack:
    """INT8 layers in one pinned host pool, decoded through woq_pager.

    Each layer's block holds the device layouts of its four products (q|k|v,
    o, gate|up, down) back to back at 256-byte aligned offsets."""

    def __init__(self, spec, weight_fn, threads=None, layers=None, log=None):
        import torch
        assert spec.fmt == "int8"
        self.spec = spec
        self.n_layers = spec.layers if layers is None else layers
        threads = threads or min(16, os.cpu_count() or 1)
        log = log or (lambda *a: None)
        # block layout (identical for every layer)
        offs, o = [], 0
        for names, _ in GROUPS:
            N = sum(spec.linear(n).N for n in names)
            K = spec.linear(names[0]).K
            offs.append(o)
            o += -(-woq.lib().woq_int8_dev_bytes(N, K) // 256) * 256
        self.block_bytes = o
        self.group_offsets = offs
        self.pool = torch.empty(self.n_layers * o, dtype=torch.uint8, pin_memory=True)
        pool_np = self.pool.numpy()
        self.steps = []
        for l0 in range(0, self.n_layers, 4):
            ls = range(l0, min(self.n_layers, l0 + 4))
            log(f"quantising streamed layers {ls.start}..{ls.stop - 1}")
            jobs = [(layer, lin) for layer in ls for lin in spec.linears()]
            res = _map_weights(spec, jobs, weight_fn, lambda layer, lin, W: woq.woq_quantize_int8(W), threads)
            got = {(layer, lin.name): r for (layer, lin), r in zip(jobs, res)}
            for layer in ls:
                base = layer * o
                for gi, (names, _) in enumerate(GROUPS):
                    parts = [got[(layer, n)] for n in names]
                    q = np.concatenate([p[0] for p in parts]) if len(parts) > 1 else parts[0][0]
                    dev = woq.woq_layout_int8(q)
                    pool_np[base + offs[gi]: base + offs[gi] + dev.size] = dev
                    st = woq.PagerStep()
                    st.code_offset = offs[gi]
                    st.w.N, st.w.K, st.w.nseg = q.shape[0], q.shape[1], len(parts)
                    end = 0
                    for i, (qi, sc) in enumerate(parts):
                        end += qi.shape[0]
                        st.w.seg_end[i] = end
                        st.w.seg_scale[i] = float(sc)
                    self.steps.append(st)
        self.layer_off = [l * o for l in range(self.n_layers)]
        self.layer_bytes = [o] * self.n_layers

    def make_pager(self, max_b: int):
        return woq.Pager(self.pool, self.layer_off, self.layer_bytes, self.steps, len(GROUPS), max_b)


class TiedVocab:
    """The vocabulary matrix on both sides of the stack, tied: an INT8 table
    for the token lookup and the outlier-aware INT4 lm_head quantised from the
    same float matrix over the hidden space's global permutation.

    E: float32 [V, H]; perm: int32 [H], the hidden space's permutation (the one
    the stack's q|k|v and gate|up products use); max_b: largest batch.
    """

    def __init__(self, E, perm, max_b: int, device="cuda"):
        import torch
        E = np.ascontiguousarray(E, np.float32)
        self.V, self.H = E.shape
        self.max_b = max_b
        q, s = woq.woq_quantize_int8(E)
        self.table = woq.DeviceInt8([(q, s)], device)
        del q
        self.geom = woq.woq_int4o_geometry(self.H)
        self.head = woq.DeviceInt4o([woq.woq_quantize_int4o(E, perm)], self.geom, device)
        self.perm_dev = torch.from_numpy(np.ascontiguousarray(perm, np.int32)).to(device)
        self.xp = torch.zeros(max_b, self.geom.xp_len, dtype=torch.float16, device=device)

    def device_bytes(self) -> int:
        tot = self.table.nbytes
        for t in (self.head.codes, self.head.scales, self.head.w_out):
            if t is not None:
                tot += t.numel() * t.element_size()
        return tot

    def embed(self, ids, y, stream=None, b: int | None = None):
        """y[r] = table row ids[r] (fp16), ids int32 [b] on the device."""
        return woq.woq_embed_int8(self.table.desc, ids, y, stream, b)

    def logits(self, h, y, stream=None, b: int | None = None):
        """y = lm_head(h): h fp16 [b, H], y fp16 [b, >= V]."""
        b = h.shape[0] if b is None else b
        assert b <= self.max_b
        woq.woq_permute_x(h, self.perm_dev, self.geom, self.xp, stream)
        return woq.woq_qgemv_int4o(self.head.desc, self.xp, y, stream, b)
