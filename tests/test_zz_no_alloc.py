"""sgmv_fused_static: the fused call with its shrink partials in the
library's static device scratch (for callers that cannot allocate).

Through the C ABI, two calls in a row (a prefill batch, then a smaller decode
batch) must give sgmv_fused's outputs bit for bit, the device's free memory
must not change across calls after the first, and a call whose partials
exceed the scratch is refused before anything is enqueued.
"""
import numpy as np
import pytest

from synth import config, random_case
from synth.device import DeviceWorkload

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import heterogeneous_adapter_batching_amd as hab
    hab.load()


def _run(dw, fn):
    """One pass of every (layer, call) of the workload through `fn`; the
    outputs as bit patterns."""
    w = dw.w
    dw.zero_outputs()
    for l in dw.layers:
        for ci, c in enumerate(dw.calls):
            fn(dw.pool, dw.plan, l, c, dw.y_offsets[ci], dw.x[(l, w.projs[c[0]].x_key)],
               dw.y[(l, ci)], dw.base.get((l, ci)))
    torch.cuda.synchronize()
    return {k: v.view(torch.int16).clone() if v.dtype == torch.bfloat16 else v.clone()
            for k, v in dw.y.items()}


def test_static_scratch_matches_fused():
    import heterogeneous_adapter_batching_amd as hab
    big = DeviceWorkload(config(2), threads=8)                 # 4096-token prefill
    small = DeviceWorkload(random_case(61, T=40, h_in=264, h_out=136, has_base=True),
                           threads=4)                          # a smaller decode batch
    print("[no-alloc] workloads staged", flush=True)
    free0 = None
    for rep in range(2):
        for name, dw in (("prefill", big), ("decode", small)):
            ref = _run(dw, hab.sgmv_fused)
            got = _run(dw, hab.sgmv_fused_static)
            for k in ref:
                assert torch.equal(ref[k], got[k]), (rep, name, k)
            free = torch.cuda.mem_get_info()[0]
            if free0 is None:
                free0 = free
            else:
                assert free == free0, (rep, name, free0 - free)
            print(f"[no-alloc] rep {rep} {name}: bit-identical", flush=True)


def test_static_scratch_too_small_refused():
    """A call whose shrink partials exceed the scratch (a merge plan of two
    slots over 16384 tokens, rank 64, three projections: its long groups'
    rows run in the shrink at 64-token blocks): LORA_EINVAL, and the output
    is untouched (nothing was enqueued)."""
    import heterogeneous_adapter_batching_amd as hab
    T, h = 16384, 4096
    pool = hab.Pool(1, [h, h, h], [h, h, h], 64, "bf16", slab_bytes=4 * (64 * 8 * h * 2 + 256),
                    max_slots=4)
    for a in range(2):
        pool.reserve(a, 64, 1.0)
    plan = hab.Plan.merge(pool, T, [0, T // 2, T], np.array([[0, 1], [1, 0]], np.int32),
                          np.ones((2, 2), np.float32)).upload(3)
    x = torch.zeros((T, h), dtype=torch.bfloat16, device="cuda")
    y = torch.full((T, 3 * h), 7.0, dtype=torch.bfloat16, device="cuda")
    with pytest.raises(hab.LoraError) as ei:
        hab.sgmv_fused_static(pool, plan, 0, [0, 1, 2], [0, h, 2 * h], x, y)
    assert ei.value.status == -1 and "static scratch" in ei.value.message
    torch.cuda.synchronize()
    assert bool((y == 7.0).all())
