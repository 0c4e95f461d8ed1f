"""Batches through the library's bounds-checked debug build.

Run by tests/test_gpu_debug.py in a process of its own, with HAB_LORA_LIB
naming libhab_lora_debug.so before the binding loads it:

1. decode, prompt, mixed and two-step batches give the delta within the
   contract tolerance of the oracle, and no check fails;
2. a plan's device tables overwritten as a stray write would leave them (an
   adapter extent moved past the pool's slab, a block's token count past the
   plan, a token row past the batch): the launches complete, each sets its
   LORA_DEBUG_* bit, and the tables uploaded again give the right delta.  The
   slab tensor extends past the pool's slab by more than an adapter extent,
   and token rows past the batch fall outside the activations' buffer
   ranges, so even an unchecked access would stay inside the allocations.

Prints a line per step and exits non-zero on the first failure.
"""
import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import numpy as np  # noqa: E402
import torch  # noqa: E402

import heterogeneous_adapter_batching_amd as hab  # noqa: E402
import oracle  # noqa: E402
from synth import config, mixed_case, random_case  # noqa: E402
from synth.device import DeviceWorkload  # noqa: E402


def log(msg):
    print(msg, flush=True)


def parity(dw, what):
    w = dw.w
    for l in dw.layers:
        for p in range(len(w.projs)):
            got = dw.output(l, p)
            ref = oracle.workload_call(w, l, p, threads=4)
            tol = 1e-2 * float(np.abs(ref).max(initial=0.0)) + 1e-3
            err = float(np.abs(got.astype(np.float64) - ref).max(initial=0.0))
            assert err <= tol, f"{what} layer {l} proj {p}: max|diff| {err:.3e} > {tol:.3e}"


def run(dw, two_step=False):
    dw.zero_outputs()
    (dw.run_two_step if two_step else dw.run_fused)()
    torch.cuda.synchronize()


def records(img, pool, ids):
    """32-byte records of the plan image that name an adapter's extent and
    padded rank (the block and rank-tile descriptors of its groups)."""
    words = img.view(np.int32).reshape(-1, 8)
    found = []
    for a in ids:
        q = pool.query(int(a))
        lo, hi = q["offset"] & 0xffffffff, q["offset"] >> 32
        hit = np.nonzero((words[:, 2] == q["r_pad"]) & (words[:, 6].view(np.uint32) == lo) &
                         (words[:, 7].view(np.uint32) == hi))[0]
        found.extend(int(i) for i in hit)
    return sorted(found)


def main():
    assert torch.cuda.is_available(), "needs a GPU"
    torch.cuda.set_device(0)
    hab.load()
    enabled, bits = hab.debug_checks(clear=True)
    assert enabled, f"{hab.LIB_PATH} is not the debug build"
    log(f"[debug] {os.path.basename(hab.LIB_PATH)}: checks enabled")

    cases = [
        ("tiny f32", config(0), False),
        ("q decode", config(1), False),
        ("heterogeneous ranks", random_case(7, T=90, h_in=512, h_out=264, n_adapters=12,
                                            r_choices=[8, 16, 32, 64], has_base=True), False),
        ("mixed prompts and decode", mixed_case(8, h_in=384, h_out=264), False),
        ("two-step", random_case(9, T=70, h_in=256, h_out=128, n_adapters=5), True),
    ]
    for name, w, two in cases:
        dw = DeviceWorkload(w, threads=4)
        run(dw, two)
        parity(dw, name)
        _, bits = hab.debug_checks(clear=True)
        assert bits == 0, f"{name}: debug bits {bits:#x} on a good plan"
        log(f"[debug] {name}: parity within tolerance, no check failed")

    # stray writes into a plan's device tables
    w = random_case(10, T=40, h_in=256, h_out=128, n_adapters=6, has_base=True)
    desc = hab.api.make_desc(w.num_layers, [p.h_in for p in w.projs],
                             [p.h_out for p in w.projs], w.r_max, w.dtype)
    margin = 2 * hab.extent_bytes(desc, w.r_max)
    dw = DeviceWorkload(w, threads=4, slab_margin=margin)
    ws, plan, pool = dw.plan.ws, dw.plan, dw.pool
    slab_bytes = int(pool.slab.numel())
    good = ws.cpu().numpy().copy()
    recs = records(good, pool, w.touched())
    assert recs, "no descriptor records found in the plan image"
    order = plan.export()["token_order"]

    def corrupt(kind):
        img = good.copy()
        words = img.view(np.int32).reshape(-1, 8)
        rows = img.view(np.int32).reshape(-1, 64)
        hits = 0
        for i in recs:
            if kind == "slab":            # the extent moved to the end of the slab
                words[i, 6] = np.uint32(slab_bytes & 0xffffffff).view(np.int32)
                words[i, 7] = np.int32(slab_bytes >> 32)
                hits += 1
            elif kind == "rows":          # a token count far past the plan
                words[i, 1] = 1 << 20
                hits += 1
            else:                         # the descriptor's first token row past the batch
                off, n = int(words[i, 0]), int(words[i, 1])
                want = np.full(64, -1, np.int32)
                want[:n] = order[off:off + n]
                for j in np.nonzero((rows == want).all(axis=1))[0]:
                    rows[j, 0] = w.num_tokens + 5
                    hits += 1
        assert hits, kind
        ws.copy_(torch.from_numpy(img))
        torch.cuda.synchronize()
        return hits

    for kind, bit in (("slab", hab.LORA_DEBUG_SLAB), ("rows", hab.LORA_DEBUG_ROW),
                      ("token", hab.LORA_DEBUG_TOKEN)):
        hits = corrupt(kind)
        run(dw)
        _, bits = hab.debug_checks(clear=True)
        assert bits & bit, f"{kind}: expected bit {bit:#x}, got {bits:#x}"
        log(f"[debug] {kind}: {hits} table entries overwritten, bits {bits:#x}")
        plan.upload(dw.max_proj, ws=ws)          # the plan's own tables again
        run(dw)
        parity(dw, f"after {kind}")
        _, bits = hab.debug_checks(clear=True)
        assert bits == 0, f"after {kind}: bits {bits:#x}"
    log("[debug] all checks passed")


if __name__ == "__main__":
    main()
