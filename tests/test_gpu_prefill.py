"""GPU parity of gdn_chunk_prefill (chunked form, MFMA) against the CPU oracle's
token-by-token recurrence: ragged lengths around the chunk size, every head
dim, fp32 / bf16 / fp16 states, the two-call split, padded sequences, and the
full-size 4-sequence workload on sampled (sequence, head) pairs.
"""
import numpy as np
import pytest

import oracle as O
from workloads import gen

from gpu_util import DEV, assert_close, dev, host, poisoned_pool, require_gpu, say

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    require_gpu()


def run_prefill(cid, lengths, Hk, Hv, D, sdt, in_dt="bf16", num_slots=None, slot_map=None, a_shift=0.0,
                sample=None, pool=None, states=None, step=0, check=True, chunk=64):
    """One prefill call on the GPU and on the oracle (optionally only sampled (seq, head) pairs)."""
    import torch
    import gated_deltanet_state_gdn_amd as gdn
    N = len(lengths)
    num_slots = num_slots or N + 3
    if slot_map is None:
        slot_map = gen.slot_permutation(cid, num_slots)[:N]
    slot_map = np.asarray(slot_map, np.int32)
    valid = [int(s) for s in slot_map if 0 <= s < num_slots]
    if pool is None:
        pool, st = poisoned_pool(num_slots, Hv, D, D, sdt, valid, cid)
        states = {s: st[i] for i, s in enumerate(valid)}
    cu = gen.seq_lengths_cu(lengths)
    inp = gen.token_inputs(cid, step, (int(cu[-1]),), Hk, Hv, D, D, in_dt, a_shift)
    A_log, dt_bias = gen.head_params(cid, Hv)
    say(f"prefill cid={cid} lengths={list(lengths)[:8]} Hk={Hk} Hv={Hv} D={D} state={sdt} in={in_dt} chunk={chunk}")
    out = gdn.gdn_chunk_prefill(dev(inp["q"]), dev(inp["k"]), dev(inp["v"]), dev(inp["a"]), dev(inp["b"]),
                                dev(A_log), dev(dt_bias), pool, torch.from_numpy(slot_map).to(DEV),
                                torch.from_numpy(cu).to(DEV), chunk=chunk)
    torch.cuda.synchronize()
    o = host(out)
    assert np.all(np.isfinite(o)), "non-finite output"
    if not check:
        return pool, states, o, inp
    # oracle over a mini pool: local slot i holds sequence i's state
    order = [n for n in range(N) if 0 <= slot_map[n] < num_slots]
    mini = np.stack([states[int(slot_map[n])] for n in order]) if order else None
    mini_map = np.full(N, -1, np.int32)
    for i, n in enumerate(order):
        mini_map[n] = i
    heads = None if sample is None else sorted({h for _, h in sample})
    seqs = None if sample is None else sorted({n for n, _ in sample})
    if mini is None:
        mini = np.zeros((1, Hv, D, D), np.float32)
    ref_pool, o_ref = O.chunk_prefill(mini, mini_map, cu, inp["q"], inp["k"], inp["v"], inp["a"], inp["b"], A_log,
                                      dt_bias, heads=heads, seqs=seqs)
    got_pool = host(pool)
    pairs = sample if sample is not None else [(n, h) for n in range(N) for h in range(Hv)]
    for n, h in pairs:
        sl = slice(int(cu[n]), int(cu[n + 1]))
        assert_close(o[sl, h], o_ref[sl, h], "f32", f"o seq {n} head {h}")
        if mini_map[n] >= 0 and cu[n + 1] > cu[n]:
            assert_close(got_pool[slot_map[n], h], ref_pool[mini_map[n], h], sdt, f"state seq {n} head {h}")
            states[int(slot_map[n])] = np.array(states[int(slot_map[n])], copy=True)
            states[int(slot_map[n])][h] = ref_pool[mini_map[n], h]
    return pool, states, o, inp


@pytest.mark.parametrize("sdt", ["f32", "bf16", "f16"])
def test_prefill_ragged_lengths(sdt):
    """Lengths 1, 63, 64, 65, 0 and 130: partial chunks, exact chunks, an empty sequence."""
    run_prefill(70, [1, 63, 64, 65, 0, 130], 2, 4, 32, sdt, a_shift=-1.0)


@pytest.mark.parametrize("in_dt", ["bf16", "f16"])
@pytest.mark.parametrize("D", [64, 128])
def test_prefill_ragged_lengths_wide_heads(D, in_dt):
    """Head dims 64 and 128 with 16-bit inputs (the k-contiguous state kernel): partial, exact and
    empty chunks, GQA with two value heads per key head."""
    run_prefill(74 + D, [1, 63, 64, 65, 0, 130], 2, 4, D, "f32", in_dt=in_dt, a_shift=-1.0)


@pytest.mark.parametrize("in_dt,D", [("bf16", 128), ("bf16", 64), ("f16", 128), ("f32", 32)])
def test_prefill_chunk_size_invariance(in_dt, D):
    """The chunked form is exact for any chunk length: chunks of 16, 32 and 64 tokens over lengths
    around each size (1, 15, 16, 17, 33, 64, 65, 130; partial and exact chunks of every size) and
    slow decay give the oracle's outputs and states at the fp32 bar, and the same results as each
    other (at 64 with 16-bit inputs and D = 64 / 128 the k-contiguous state kernels run, at 16 and
    32 the LDS-staged one)."""
    lengths = [1, 15, 16, 17, 33, 64, 65, 130]
    outs, pools = [], []
    for chunk in (16, 32, 64):
        pool, states, o, inp = run_prefill(120 + D, lengths, 2, 4, D, "f32", in_dt=in_dt, a_shift=-3.0, chunk=chunk)
        outs.append(o)
        pools.append(host(pool))
    slots = gen.slot_permutation(120 + D, len(lengths) + 3)[:len(lengths)]
    for i in (0, 1):
        assert_close(outs[i], outs[2], "f32", f"outputs, chunks of {16 * 2 ** i} against 64")
        assert_close(pools[i][slots], pools[2][slots], "f32", f"states, chunks of {16 * 2 ** i} against 64")


@pytest.mark.parametrize("Hk,Hv", [(4, 4), (1, 3), (2, 8), (1, 5)])
@pytest.mark.parametrize("D", [64, 128])
def test_prefill_gqa_ratios(Hk, Hv, D):
    """1, 3, 4 and 5 value heads per key head: the chunk kernel forms a key head's products once and
    scales them per value head, staging the gates of two value heads at a time."""
    run_prefill(91 + D + Hv, [70, 129, 1], Hk, Hv, D, "f32", a_shift=-1.0)


@pytest.mark.parametrize("D", [16, 64, 128])
def test_prefill_head_dims(D):
    run_prefill(71 + D, [100, 37, 192], 1, 2, D, "f32")


def test_prefill_fp32_inputs_slow_decay():
    """fp32 inputs and slow decay (a - 6): the state carries across many chunks."""
    run_prefill(72, [700, 129], 2, 2, 64, "f32", in_dt="f32", a_shift=-6.0)


def run_split(cid, lengths, Hk, Hv, D, sdt, num_slots, sample=None, a_shift=0.0):
    """One call over the whole sequences against two calls (the first 55% of each sequence, then the
    rest) on a copy of the pool: outputs and final states equal within the state dtype's bar (one
    extra rounding at the split), and the split path matches the oracle's two calls, on every
    (sequence, head) pair or on the sampled ones."""
    import torch
    import gated_deltanet_state_gdn_amd as gdn
    first, second = gen.split_lengths(lengths)
    N = len(lengths)
    slot_map = gen.slot_permutation(cid, num_slots)[:N]
    pool1, st = poisoned_pool(num_slots, Hv, D, D, sdt, [int(s) for s in slot_map], cid)
    pool2 = pool1.clone()
    cu = gen.seq_lengths_cu(lengths)
    inp = gen.token_inputs(cid, 0, (int(cu[-1]),), Hk, Hv, D, D, "bf16", a_shift)
    A_log, dt_bias = gen.head_params(cid, Hv)
    args = (dev(A_log), dev(dt_bias))
    sm = torch.from_numpy(slot_map).to(DEV)
    say(f"prefill two-call split: one call, lengths {list(lengths)} Hk={Hk} Hv={Hv} D={D} state={sdt}")
    o_one = gdn.gdn_chunk_prefill(dev(inp["q"]), dev(inp["k"]), dev(inp["v"]), dev(inp["a"]), dev(inp["b"]), *args,
                                  pool1, sm, torch.from_numpy(cu).to(DEV))
    o_two = torch.empty_like(o_one)
    off = [0] * N
    parts = []
    for part in (first, second):
        idx = np.concatenate([np.arange(cu[n] + off[n], cu[n] + off[n] + part[n]) for n in range(N)])
        parts.append((part, idx))
        sub = {k: v[idx] for k, v in inp.items()}
        say(f"prefill two-call split: part {part}")
        o_p = gdn.gdn_chunk_prefill(dev(sub["q"]), dev(sub["k"]), dev(sub["v"]), dev(sub["a"]), dev(sub["b"]),
                                    *args, pool2, sm, torch.from_numpy(gen.seq_lengths_cu(part)).to(DEV))
        o_two[torch.from_numpy(idx).to(DEV)] = o_p
        off = [o_ + p for o_, p in zip(off, part)]
    torch.cuda.synchronize()
    otol = "f32" if sdt == "f32" else "bf16"
    o_two_h, o_one_h = host(o_two), host(o_one)
    assert np.all(np.isfinite(o_two_h)), "non-finite output"
    assert_close(o_two_h, o_one_h, otol, "two calls vs one call: outputs")
    assert_close(host(pool2)[slot_map], host(pool1)[slot_map], sdt, "two calls vs one call: final states")
    # the split path against the oracle's two calls (rounding to the state dtype at the split)
    # (one oracle run per sampled pair, so only those pairs are computed)
    groups = [(None, None)] if sample is None else [([n], [h]) for n, h in sample]
    ref = np.stack([st[i] for i in range(N)])
    ref_o = np.zeros((int(cu[-1]), Hv, D))
    for seqs, heads in groups:
        for part, idx in parts:
            sub = {k: v[idx] for k, v in inp.items()}
            ref, o_p = O.chunk_prefill(ref, np.arange(N), gen.seq_lengths_cu(part), sub["q"], sub["k"], sub["v"],
                                       sub["a"], sub["b"], A_log, dt_bias, heads=heads, seqs=seqs)
            if seqs is None:
                ref_o[idx] = o_p
            else:
                mask = (idx >= cu[seqs[0]]) & (idx < cu[seqs[0] + 1])
                ref_o[idx[mask], heads[0]] = o_p[mask, heads[0]]
    got_pool = host(pool2)
    pairs = sample if sample is not None else [(n, h) for n in range(N) for h in range(Hv)]
    for n, h in pairs:
        sl = slice(int(cu[n]), int(cu[n + 1]))
        assert_close(o_two_h[sl, h], ref_o[sl, h], otol, f"split outputs vs oracle, seq {n} head {h}")
        assert_close(got_pool[slot_map[n], h], ref[n, h], sdt, f"split state vs oracle, seq {n} head {h}")


@pytest.mark.parametrize("sdt", ["f32", "bf16", "f16"])
def test_prefill_two_call_split_equals_one_call(sdt):
    """First 55% of each sequence, then the rest, equals one call: the state is carried exactly
    (one extra rounding at the split for a 16-bit state); every (sequence, head) checked."""
    run_split(73, [300, 129, 64], 2, 4, 64, sdt, 6, a_shift=-3.0)


@pytest.mark.parametrize("sdt", ["f32", "bf16", "f16"])
def test_prefill_two_call_split_workload(sdt):
    """The split at the full workload: 4 packed sequences of 1024, 3000, 8192, 8192 tokens split at
    55% (563/461, 1650/1350, 4505/3687, 4505/3687), 16 key / 32 value heads, 128 x 128 states
    read from slots.  Two calls equal one call on every element; sampled (sequence, head) pairs
    against the oracle."""
    cfg = gen.WORKLOADS["prefill"]
    s = cfg.shape
    sample = [(0, 3), (1, 30), (2, 0), (3, 19)]
    run_split(31, cfg.extra["lengths"], s.Hk, s.Hv, s.dk, sdt, cfg.num_slots, sample=sample)


def test_prefill_padded_sequence():
    """slot -1: zero outputs, nothing written; the other sequences are unaffected."""
    import torch
    slot_map = np.int32([2, -1, 0])
    pool, states, o, inp = run_prefill(74, [70, 50, 10], 1, 2, 16, "f32", num_slots=4, slot_map=slot_map)
    assert np.all(o[70:120] == 0)
    del torch, states, inp


@pytest.mark.parametrize("sdt", ["bf16", "f16"])
def test_prefill_wide_heads_16bit_states_with_padding(sdt):
    """Head dim 128, bf16 inputs, 16-bit states (rounded once per call), ragged lengths and a
    padded sequence: zero outputs for it, and the others against the oracle."""
    slot_map = np.int32([3, -1, 0, 5])
    pool, states, o, inp = run_prefill(76, [130, 40, 64, 1], 2, 4, 128, sdt, num_slots=6, slot_map=slot_map)
    assert np.all(o[130:170] == 0)


@pytest.mark.parametrize("sdt", ["f32", "bf16", "f16"])
def test_prefill_workload_sampled(sdt):
    """Full-size workload: 4 packed sequences of 1024, 3000, 8192, 8192 tokens, 16 key / 32 value
    heads, 128 x 128 states read from slots; sampled (sequence, head) pairs against the oracle."""
    cfg = gen.WORKLOADS["prefill"]
    s = cfg.shape
    lengths = cfg.extra["lengths"]
    sample = [(0, 0), (1, 31), (2, 17), (3, 6)]
    run_prefill(3, lengths, s.Hk, s.Hv, s.dk, sdt, num_slots=cfg.num_slots, sample=sample)
