"""gdn_replay_decode_noalloc (the replay step on the library's fixed device scratch) against
gdn_replay_decode with a caller workspace: the same kernels, so outputs, checkpoints and rings
must agree bit for bit.  Two independent copies of the ring and checkpoint advance side by side
over calls in a row whose last ones are smaller (fewer rows, a shorter window) and cross a fold.
"""
import numpy as np
import pytest

from workloads import gen

from gpu_util import DEV, dev, host, poisoned_pool, require_gpu, say

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    require_gpu()


def _bits(t):
    a = host(t)
    return a.view(np.uint32) if a.dtype.itemsize == 4 else a.view(np.uint16)


@pytest.mark.parametrize("sdt", ["f32", "bf16"])
def test_replay_noalloc_matches_workspace_entry_point(sdt):
    import torch
    import gated_deltanet_state_gdn_amd as gdn
    cid, Hk, Hv, D, L, num_slots = 95, 16, 32, 128, 16, 80
    slot_map = gen.slot_permutation(cid, num_slots)[:64].copy()
    slot_map[[5, 40]] = [-1, num_slots]  # padded rows
    ck_a, _ = poisoned_pool(num_slots, Hv, D, D, sdt, [int(s) for s in slot_map if 0 <= s < num_slots], cid)
    ck_b = ck_a.clone()
    ring_a = gdn.new_ring(num_slots, Hk, Hv, L, D, D, torch.bfloat16, DEV)
    ring_b = gdn.new_ring(num_slots, Hk, Hv, L, D, D, torch.bfloat16, DEV)
    A_log, dt_bias = gen.head_params(cid, Hv)
    A_d, dt_d = dev(A_log), dev(dt_bias)
    # (rows, window) per call: full batch three times, then smaller calls, the last one after a fold
    for step, (B, T) in enumerate([(64, 5), (64, 5), (64, 5), (24, 2), (9, 1)]):
        inp = gen.token_inputs(cid, step, (B, T), Hk, Hv, D, D, "bf16")
        args = [dev(inp[x]) for x in "qkvab"]
        sm = torch.from_numpy(slot_map[:B].copy()).to(DEV)
        out_a = torch.full((B, T, Hv, D), float("nan"), dtype=torch.float32, device=DEV)
        say(f"replay noalloc state={sdt} step={step} B={B} T={T}")
        gdn.gdn_replay_decode_noalloc(*args, A_d, dt_d, ck_a, sm, ring_a, out_a)
        out_b = gdn.gdn_replay_decode(*args, A_d, dt_d, ck_b, sm, ring_b)
        torch.cuda.synchronize()
        assert np.array_equal(_bits(out_a), _bits(out_b)), f"outputs, call {step}"
        assert np.array_equal(_bits(ck_a), _bits(ck_b)), f"checkpoints, call {step}"
        for name in ("k", "v", "g", "beta", "start", "count"):
            assert np.array_equal(_bits(getattr(ring_a, name)) if name in ("k", "v", "g", "beta") else
                                  host(getattr(ring_a, name)),
                                  _bits(getattr(ring_b, name)) if name in ("k", "v", "g", "beta") else
                                  host(getattr(ring_b, name))), f"ring {name}, call {step}"
    cnt = host(ring_a.count)
    assert np.all(cnt[int(slot_map[0])] == 3)    # folded by the fourth call, then 2 + 1 appended
    assert np.all(cnt[int(slot_map[30])] == 15)  # only in the three full calls


def test_replay_noalloc_rejects_oversized_calls():
    """A call whose workspace would exceed the fixed scratch fails with GDN_EUNSUPPORTED before
    anything is enqueued (B = 1024, T = 5 at 32 value heads of 128 needs 162.5 MiB)."""
    import torch
    import gated_deltanet_state_gdn_amd as gdn
    B, T, Hk, Hv, D, L = 1024, 5, 16, 32, 128, 16
    q = torch.zeros((B, T, Hk, D), dtype=torch.bfloat16, device=DEV)
    v = torch.zeros((B, T, Hv, D), dtype=torch.bfloat16, device=DEV)
    g = torch.zeros((B, T, Hv), dtype=torch.bfloat16, device=DEV)
    hp = torch.zeros(Hv, dtype=torch.float32, device=DEV)
    ck = torch.zeros((4, Hv, D, D), dtype=torch.float32, device=DEV)
    ring = gdn.new_ring(4, Hk, Hv, L, D, D, torch.bfloat16, DEV)
    sm = torch.zeros(B, dtype=torch.int32, device=DEV)
    out = torch.empty((B, T, Hv, D), dtype=torch.float32, device=DEV)
    with pytest.raises(gdn.GdnError) as e:
        gdn.gdn_replay_decode_noalloc(q, q, v, g, g, hp, hp, ck, sm, ring, out)
    assert e.value.status == gdn.GDN_EUNSUPPORTED
    assert int(host(ring.count).sum()) == 0
