"""Stage a synthetic workload on the GPU: pool, plan, activations, outputs.

Input plumbing only: values come from ``synth.workloads`` (drawn on the host
with numpy) and are copied to device memory and into the adapter pool through
the library's own upload calls.  Nothing here computes any part of the delta.
"""
from __future__ import annotations

from concurrent.futures import ThreadPoolExecutor

import numpy as np

from .workloads import Workload, bf16_bits, default_threads


def to_device(a: np.ndarray, dtype: str):
    import torch
    if dtype == "bf16":
        bits = bf16_bits(a).view(np.int16)
        return torch.from_numpy(bits).to("cuda").view(torch.bfloat16)
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to("cuda")


def host_weights(a: np.ndarray, dtype: str) -> np.ndarray:
    """Host array in the pool's element format (bf16 bits or float32)."""
    return bf16_bits(a) if dtype == "bf16" else np.ascontiguousarray(a, dtype=np.float32)


def from_device(t) -> np.ndarray:
    """A device tensor's values as float32 on the host (exact for bf16)."""
    import torch
    return t.detach().to(torch.float32).cpu().numpy()


class DeviceWorkload:
    """A Workload staged on the GPU.

    pool_ids:  adapters reserved in the pool (default: the whole pool, in id
               order, so touched adapters sit where a realistic pool puts them)
    upload:    adapters whose weights are uploaded (default: the touched ones)
    slab_fill: byte value written over the whole slab before uploading (e.g.
               0xFF = bf16/f32 NaN, to prove untouched extents are never read)
    on_block:  callback(aid, layer, proj, A, B) with each uploaded float32 block
    plan_opts: plan options set on the pool before the plan is built
    slab_margin: bytes allocated past the pool's slab (the pool sees only its
               own bytes; reads a little past them stay inside the allocation)
    """

    def __init__(self, w: Workload, *, hab=None, pool_ids=None, upload=None, slab_fill=None,
                 on_block=None, threads: int = 0, max_proj: int = None, layers=None,
                 plan_opts=None, slab_margin: int = 0):
        import torch
        if hab is None:
            import heterogeneous_adapter_batching_amd as hab
        self.w, self.hab = w, hab
        self.layers = list(range(w.num_layers)) if layers is None else list(layers)
        threads = threads or default_threads()
        pool_ids = np.arange(w.pool_size) if pool_ids is None else np.asarray(pool_ids)
        upload = w.touched() if upload is None else np.asarray(upload)
        h_in = [p.h_in for p in w.projs]
        h_out = [p.h_out for p in w.projs]
        from heterogeneous_adapter_batching_amd.api import make_desc
        desc = make_desc(w.num_layers, h_in, h_out, w.r_max, w.dtype)
        slab_bytes = sum(hab.extent_bytes(desc, int(w.ranks[i])) for i in pool_ids)
        slab = torch.empty(max(slab_bytes, 256) + slab_margin, dtype=torch.uint8, device="cuda")
        if slab_fill is not None:
            slab.fill_(slab_fill)
        slab = slab[:max(slab_bytes, 256)]
        self.pool = hab.Pool(w.num_layers, h_in, h_out, w.r_max, w.dtype,
                             max_slots=max(len(pool_ids), 1), slab=slab)
        for i in pool_ids:
            self.pool.reserve(int(i), int(w.ranks[i]), float(w.scales[i]))
        # layer-major, then projection, then adapter: all blocks of one
        # (layer, projection) arrive together
        blocks = [(int(a), l, p) for l in self.layers for p in range(len(w.projs))
                  for a in upload]

        def gen(key):
            a, b = w.adapter_block(*key)
            return key, host_weights(a, w.dtype), host_weights(b, w.dtype), a, b

        chunk = 4 * threads
        with ThreadPoolExecutor(threads) as ex:
            for i in range(0, len(blocks), chunk):   # bounded: results are consumed in order
                for (aid, l, p), ha, hb, a, b in ex.map(gen, blocks[i:i + chunk]):
                    self.pool.upload(aid, l, p, ha, hb)
                    if on_block is not None:
                        on_block(aid, l, p, a, b)

        self.calls = [tuple(c) for c in w.calls]
        self.max_proj = max_proj or max(len(c) for c in self.calls)
        if plan_opts:
            self.pool.set_plan_opts(**plan_opts)
        if w.merge_ids is not None:
            self.plan = hab.Plan.merge(self.pool, w.num_tokens, w.seg_starts, w.merge_ids,
                                       w.merge_w)
        else:
            self.plan = hab.Plan(self.pool, w.num_tokens, w.seg_starts, w.seg_adapter,
                                 seg_sigma=w.seg_sigma if w.sigma_kind else None)
        self.plan.upload(self.max_proj)
        # cores of jointly compressed adapters: [n][layers][proj][r_max]([r_max])
        self.sigma = None
        if w.sigma_kind:
            used = sorted({int(j) for j in w.seg_sigma if j >= 0})
            shape = (w.n_cores, w.num_layers, len(w.projs), w.r_max) + (
                (w.r_max,) if w.sigma_kind == "full" else ())
            self.sigma = torch.zeros(shape, dtype=torch.float32, device="cuda")
            for j in used:                 # one copy per core
                host = np.zeros(shape[1:], np.float32)
                for l in self.layers:
                    for p in range(len(w.projs)):
                        host[l, p] = w.core(j, l, p)
                self.sigma[j].copy_(torch.from_numpy(host))
        self.y_offsets = []
        for c in self.calls:
            offs, o = [], 0
            for p in c:
                offs.append(o)
                o += w.projs[p].h_out
            self.y_offsets.append(offs)

        # activations and outputs, per layer
        self.x, self.base, self.y = {}, {}, {}
        for l in self.layers:
            for key in w.x_keys():
                self.x[(l, key)] = to_device(w.activation(l, key), w.dtype)
            for ci, c in enumerate(self.calls):
                width = sum(w.projs[p].h_out for p in c)
                if w.has_base:
                    base = np.concatenate([w.base_out(l, p) for p in c], axis=1)
                    self.base[(l, ci)] = to_device(base, w.dtype)
                self.y[(l, ci)] = torch.zeros((w.num_tokens, width), device="cuda",
                                              dtype=torch.bfloat16 if w.dtype == "bf16"
                                              else torch.float32)

    def zero_outputs(self):
        for t in self.y.values():
            t.zero_()

    def run_fused(self, stream=None):
        """One pass of the delta over every (layer, call): y = y_in + s B (A x)."""
        hab, w = self.hab, self.w
        for l in self.layers:
            for ci, c in enumerate(self.calls):
                x = self.x[(l, w.projs[c[0]].x_key)]
                if self.sigma is not None:
                    hab.sgmv_fused_sigma(self.pool, self.plan, l, c, self.y_offsets[ci], x,
                                         self.sigma, w.sigma_kind, self.y[(l, ci)],
                                         self.base.get((l, ci)), stream=stream)
                else:
                    hab.sgmv_fused(self.pool, self.plan, l, c, self.y_offsets[ci], x,
                                   self.y[(l, ci)], self.base.get((l, ci)), stream=stream)

    def run_two_step(self, stream=None):
        """The same pass as separate shrink and expand calls through a v buffer."""
        import torch
        hab, w = self.hab, self.w
        for l in self.layers:
            for ci, c in enumerate(self.calls):
                x = self.x[(l, w.projs[c[0]].x_key)]
                y = self.y[(l, ci)]
                if w.has_base:
                    y.copy_(self.base[(l, ci)])
                v = torch.zeros((w.num_tokens, len(c) * w.r_max), dtype=torch.float32,
                                device="cuda")
                hab.sgmv_shrink(self.pool, self.plan, l, c, x, v, stream=stream)
                if self.sigma is not None:
                    hab.sgmv_expand_sigma(self.pool, self.plan, l, c, self.y_offsets[ci], v,
                                          self.sigma, w.sigma_kind, y, stream=stream)
                else:
                    hab.sgmv_expand(self.pool, self.plan, l, c, self.y_offsets[ci], v, y,
                                    stream=stream)

    def output(self, layer: int, p: int) -> np.ndarray:
        """y of projection p at ``layer`` as float32 on the host."""
        for ci, c in enumerate(self.calls):
            if p in c:
                off = self.y_offsets[ci][c.index(p)]
                t = self.y[(layer, ci)][:, off:off + self.w.projs[p].h_out]
                return from_device(t)
        raise KeyError(p)
