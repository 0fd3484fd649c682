"""Pins of the CPU oracle against facts that do not come from the oracle itself.

Each test fixes one part of the oracle so that a plausible mistake in it (a
dropped term, a wrong sign or index, a transposed operand, a wrong rounding)
fails: a hand-worked closed form, an unrolled matrix-product brute force,
algebraic identities of the delta rule, library rounding routines, and
structural properties of the drivers.
"""
import json
import math
import os
from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle as O
from workloads import gen

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


# ---------------------------------------------------------------- worked example
def test_worked_example_dk2_closed_form():
    """dk = dv = 2, S0 = I, k = e1, v = (2, 3), g = ln 1/2, beta = 1/2, q = (1, 1).

    By hand: exp(g) S0 = I/2; S^T k = (1/2, 0); v - S^T k = (3/2, 3);
    delta = beta (v - S^T k) = (3/4, 3/2); S1 = I/2 + e1 delta^T =
    [[5/4, 3/2], [0, 1/2]]; S1^T q = (5/4, 2); o = 2**-1/2 (5/4, 2).
    The gate inputs a = -dt_bias, A_log = 0, b = 0 give softplus(0) = ln 2,
    g = -ln 2 and beta = 1/2.
    """
    F = Fraction
    S1 = np.array([[F(5, 4), F(3, 2)], [F(0), F(1, 2)]], dtype=object).astype(np.float64)
    o = np.array([1.25, 2.0]) / math.sqrt(2.0)
    g, beta = O.gates(np.float32([0.3]), np.float32([0.0]), np.float32([0.0]), np.float32([-0.3]))
    assert g[0] == pytest.approx(-math.log(2.0), rel=1e-15)
    assert beta[0] == 0.5
    S, out = O.gdn_token(np.eye(2), np.array([1.0, 1.0]), np.array([1.0, 0.0]),
                         np.array([2.0, 3.0]), g[0], beta[0], 2 ** -0.5)
    np.testing.assert_allclose(S, S1, rtol=1e-15, atol=1e-15)
    np.testing.assert_allclose(out, o, rtol=1e-15)
    # the decode driver gives the same numbers through slots, gates and the dk**-0.5 default
    pool = np.eye(2, dtype=np.float32)[None, None]
    pool2, o2 = O.decode_step(pool, [0], np.float32([[[1, 1]]]), np.float32([[[1, 0]]]),
                              np.float32([[[2, 3]]]), np.float32([[0.3]]), np.float32([[0.0]]),
                              np.float32([0.0]), np.float32([-0.3]))
    np.testing.assert_allclose(o2[0, 0], o, rtol=1e-7)
    np.testing.assert_allclose(pool2[0, 0], S1, rtol=1e-7)


# ---------------------------------------------------------------- brute force
def _brute_force(S0, q, k, v, g, beta, scale):
    """Unrolled product form: S_t = A_t...A_1 S0 + sum_i A_t...A_{i+1} beta_i k_i v_i^T,
    A_i = exp(g_i) (I - beta_i k_i k_i^T); o_t = scale S_t^T q_t (float64)."""
    T, dk = k.shape
    I = np.eye(dk)
    A = [math.exp(g[i]) * (I - beta[i] * np.outer(k[i], k[i])) for i in range(T)]
    outs, states = [], []
    for t in range(T):
        # A_t ... A_0, built left-multiplying
        Pall = I.copy()
        for i in range(t + 1):
            Pall = A[i] @ Pall
        St = Pall @ S0
        for i in range(t + 1):
            Pi = I.copy()
            for j in range(i + 1, t + 1):
                Pi = A[j] @ Pi
            St = St + Pi @ (beta[i] * np.outer(k[i], v[i]))
        states.append(St)
        outs.append(scale * St.T @ q[t])
    return np.array(outs), states


def test_brute_force_tiny_config():
    """The token loop equals the unrolled product form on the tiny workload."""
    cfg = gen.WORKLOADS["tiny"]
    sh = cfg.shape
    A_log, dt_bias = gen.head_params(0, sh.Hv)
    pool = gen.pool_slots(0, range(cfg.num_slots), sh.Hv, sh.dk, sh.dv, "f32")
    steps = [gen.token_inputs(0, s, (sh.B,), sh.Hk, sh.Hv, sh.dk, sh.dv, "f32") for s in range(cfg.steps)]
    slot_map = cfg.extra["slot_map"]
    ratio = sh.Hv // sh.Hk
    scale = sh.dk ** -0.5
    for bi, slot in enumerate(slot_map):
        for h in range(sh.Hv):
            hk = h // ratio
            q = np.stack([O.widen(s["q"][bi, hk]) for s in steps])
            k = np.stack([O.widen(s["k"][bi, hk]) for s in steps])
            v = np.stack([O.widen(s["v"][bi, h]) for s in steps])
            ab = [O.gates(s["a"][bi, h], s["b"][bi, h], A_log[h], dt_bias[h]) for s in steps]
            g = np.array([x[0] for x in ab])
            beta = np.array([x[1] for x in ab])
            S0 = O.widen(pool[slot, h])
            o_bf, st_bf = _brute_force(S0, q, k, v, g, beta, scale)
            o_loop, S_loop = O.ref_gdn(S0, q, k, v, g, beta, scale)
            np.testing.assert_allclose(o_loop, o_bf, rtol=1e-12, atol=1e-13)
            np.testing.assert_allclose(S_loop, st_bf[-1], rtol=1e-12, atol=1e-13)


def test_decode_driver_matches_brute_force_over_steps():
    """Eight decode steps through slots (f32 pool) track the unrolled form within f32 rounding."""
    cfg = gen.WORKLOADS["tiny"]
    sh = cfg.shape
    A_log, dt_bias = gen.head_params(0, sh.Hv)
    pool0 = gen.pool_slots(0, range(cfg.num_slots), sh.Hv, sh.dk, sh.dv, "f32")
    slot_map = np.int32(cfg.extra["slot_map"])
    pool = pool0
    outs = []
    steps = [gen.token_inputs(0, s, (sh.B,), sh.Hk, sh.Hv, sh.dk, sh.dv, "f32") for s in range(cfg.steps)]
    for s in steps:
        pool, o = O.decode_step(pool, slot_map, s["q"], s["k"], s["v"], s["a"], s["b"], A_log, dt_bias)
        outs.append(o)
    # untouched slots are bit-identical
    for slot in set(range(cfg.num_slots)) - set(slot_map.tolist()):
        assert np.array_equal(pool[slot].view(np.uint32), pool0[slot].view(np.uint32))
    ratio = sh.Hv // sh.Hk
    for bi, slot in enumerate(slot_map):
        for h in range(sh.Hv):
            hk = h // ratio
            q = np.stack([O.widen(s["q"][bi, hk]) for s in steps])
            k = np.stack([O.widen(s["k"][bi, hk]) for s in steps])
            v = np.stack([O.widen(s["v"][bi, h]) for s in steps])
            gb = [O.gates(s["a"][bi, h], s["b"][bi, h], A_log[h], dt_bias[h]) for s in steps]
            o_bf, st = _brute_force(O.widen(pool0[slot, h]), q, k, v,
                                    [x[0] for x in gb], [x[1] for x in gb], sh.dk ** -0.5)
            np.testing.assert_allclose(np.stack([o[bi, h] for o in outs]), o_bf, rtol=1e-5, atol=1e-6)
            np.testing.assert_allclose(O.widen(pool[slot, h]), st[-1], rtol=1e-5, atol=1e-6)


# ---------------------------------------------------------------- identities
def test_delta_rule_write_property():
    """beta = 1 and |k| = 1: the updated state maps k exactly onto v (S_new^T k = v)."""
    r = np.random.default_rng(7)
    S = r.standard_normal((16, 12))
    k = r.standard_normal(16)
    k /= np.linalg.norm(k)
    v = r.standard_normal(12)
    for g in (0.0, -0.7, -5.0):
        Sn = O.decay_update(S, k, v, g, 1.0)
        np.testing.assert_allclose(Sn.T @ k, v, rtol=0, atol=1e-13)


def test_gate_special_points():
    assert O.softplus(0.0) == pytest.approx(math.log(2.0), rel=1e-16)
    assert O.sigmoid(0.0) == 0.5
    for x in (-30.0, -3.0, -0.5, 0.25, 2.0, 20.0):
        assert O.softplus(x) == pytest.approx(math.log1p(math.exp(x)), rel=1e-14)
        assert O.sigmoid(x) == pytest.approx(1.0 / (1.0 + math.exp(-x)), rel=1e-15)
    assert O.softplus(800.0) == 800.0          # no overflow for large arguments
    assert O.softplus(-800.0) == 0.0
    assert O.sigmoid(-800.0) == 0.0 and O.sigmoid(800.0) == 1.0
    # sign convention: g <= 0 is a decay, and a larger A_log decays faster
    g1, _ = O.gates(np.float32([0.5]), np.float32([0]), np.float32([0.1]), np.float32([0.0]))
    g2, _ = O.gates(np.float32([0.5]), np.float32([0]), np.float32([1.1]), np.float32([0.0]))
    assert g2[0] < g1[0] < 0


def test_identity_token_leaves_state_bit_identical():
    """a = -200 gives g = -0 (exp(g) = 1) and b = -200 gives beta ~ 0: the state is unchanged
    bit for bit and the output is scale * S0^T q."""
    r = np.random.default_rng(3)
    S0 = r.standard_normal((8, 8)) * 0.1
    g, beta = O.gates(np.float32([-200]), np.float32([-200]), np.float32([1.0]), np.float32([0.5]))
    assert math.exp(g[0]) == 1.0 and beta[0] < 1e-80
    q, k, v = r.standard_normal(8), r.standard_normal(8), r.standard_normal(8)
    S, o = O.gdn_token(S0, q, k, v, g[0], beta[0], 0.25)
    assert np.array_equal(S, S0)
    np.testing.assert_allclose(o, 0.25 * S0.T @ q, rtol=1e-15)


def test_full_decay_keeps_only_new_outer_product():
    """a = +200 with A_log = 3 gives g ~ -4000, exp(g) = 0: S_new = beta k v^T; b = +200 gives beta = 1."""
    r = np.random.default_rng(4)
    S0 = r.standard_normal((8, 6))
    g, beta = O.gates(np.float32([200]), np.float32([200]), np.float32([3.0]), np.float32([0.0]))
    assert math.exp(g[0]) == 0.0 and beta[0] == 1.0
    k, v = r.standard_normal(8), r.standard_normal(6)
    S = O.decay_update(S0, k, v, g[0], beta[0])
    np.testing.assert_allclose(S, np.outer(k, v), rtol=1e-15)


# ---------------------------------------------------------------- rounding helpers
def _f32_from_halves(hi, lo):
    return ((hi.astype(np.uint32) << 16) | np.uint32(lo)).view(np.float32)


def test_bf16_rounding_matches_torch_all_patterns():
    hi = np.arange(1 << 16, dtype=np.uint32)
    for lo in (0x0000, 0x0001, 0x7FFF, 0x8000, 0x8001, 0xFFFF):
        x = _f32_from_halves(hi, lo)
        x = x[np.isfinite(x)]
        ours = O.to_storage(x.astype(np.float64), "bf16")
        ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
        fin = np.isfinite(O.widen(ref))      # torch overflows to inf like we do
        assert np.array_equal(ours[fin], ref[fin]), f"lo={lo:#x}"
        assert np.array_equal(np.isinf(O.widen(ours)), ~fin)


def test_f16_rounding_matches_numpy_and_ties():
    h = np.arange(1 << 16, dtype=np.uint16).view(np.float16)
    h = h[np.isfinite(h)].astype(np.float64)
    h = np.unique(h)
    mids = (h[:-1] + h[1:]) / 2                      # exact ties (f32-representable)
    xs = np.concatenate([h, mids, np.nextafter(mids.astype(np.float32), np.float32(np.inf)).astype(np.float64),
                         np.nextafter(mids.astype(np.float32), np.float32(-np.inf)).astype(np.float64)])
    xs = xs[np.abs(xs) < 65520]
    ours = O.to_storage(xs, "f16")
    ref = xs.astype(np.float32).astype(np.float16)
    assert np.array_equal(ours.view(np.uint16), ref.view(np.uint16))


def test_f32_rounding_matches_numpy():
    r = np.random.default_rng(11)
    x = r.standard_normal(200000) * np.exp2(r.integers(-140, 120, 200000))
    f = x.astype(np.float32).astype(np.float64)
    up = np.nextafter(f.astype(np.float32), np.float32(np.inf)).astype(np.float64)
    ties = (f + up) / 2
    xs = np.concatenate([x, ties])
    xs = xs[np.isfinite(xs)]
    assert np.array_equal(O.to_storage(xs, "f32").view(np.uint32), xs.astype(np.float32).view(np.uint32))


# ---------------------------------------------------------------- GQA mapping
def test_value_heads_read_contiguous_key_groups():
    """Hv = 4, Hk = 2: with q of key head 1 set to zero, value heads 2 and 3 output zero and
    heads 0 and 1 do not (contiguous groups h // 2; an interleaved h % 2 mapping fails)."""
    sh = gen.DecodeShape(1, 2, 4, 8, 8)
    inp = gen.token_inputs(99, 0, (1,), sh.Hk, sh.Hv, sh.dk, sh.dv, "f32")
    inp["q"][0, 1] = 0.0
    A_log, dt_bias = gen.head_params(99, sh.Hv)
    pool = gen.pool_slots(99, [0], sh.Hv, sh.dk, sh.dv, "f32")
    _, o = O.decode_step(pool, [0], inp["q"], inp["k"], inp["v"], inp["a"], inp["b"], A_log, dt_bias)
    assert np.all(o[0, 2:] == 0.0)
    assert np.all(np.abs(o[0, :2]).max(axis=1) > 1e-3)


# ---------------------------------------------------------------- drivers
def test_padded_rows_touch_nothing():
    sh = gen.DecodeShape(3, 1, 2, 8, 8)
    inp = gen.token_inputs(5, 0, (3,), sh.Hk, sh.Hv, sh.dk, sh.dv, "f32")
    A_log, dt_bias = gen.head_params(5, sh.Hv)
    pool = gen.pool_slots(5, range(2), sh.Hv, sh.dk, sh.dv, "bf16")
    pool2, o = O.decode_step(pool, [-1, 1, 2], inp["q"], inp["k"], inp["v"], inp["a"], inp["b"], A_log, dt_bias)
    assert np.all(o[0] == 0) and np.all(o[2] == 0) and np.any(o[1] != 0)
    assert np.array_equal(pool2[0], pool[0]) and not np.array_equal(pool2[1], pool[1])


def _decode_loop(pool, slot, q, k, v, a, b, A_log, dt_bias):
    outs = []
    for t in range(q.shape[0]):
        pool, o = O.decode_step(pool, [slot], q[t:t + 1], k[t:t + 1], v[t:t + 1], a[t:t + 1], b[t:t + 1],
                                A_log, dt_bias)
        outs.append(o[0])
    return pool, np.stack(outs)


@pytest.mark.parametrize("sdt", ["f32", "bf16", "f16"])
def test_prefill_per_token_writeback_equals_decode_loop(sdt):
    """Prefill with a write point after every token is, token for token, the decode loop;
    packing several sequences (one of length 0) must not mix them."""
    sh = gen.DecodeShape(3, 1, 2, 8, 8)
    lens = [5, 0, 7]
    cu = gen.seq_lengths_cu(lens)
    inp = gen.token_inputs(6, 0, (cu[-1],), sh.Hk, sh.Hv, sh.dk, sh.dv, "bf16", a_shift=-3.0)
    A_log, dt_bias = gen.head_params(6, sh.Hv)
    pool = gen.pool_slots(6, range(4), sh.Hv, sh.dk, sh.dv, sdt)
    slots = [2, 1, 0]
    pool_p, o_p = O.chunk_prefill(pool, slots, cu, inp["q"], inp["k"], inp["v"], inp["a"], inp["b"],
                                  A_log, dt_bias, write_interval=1)
    ref_pool = pool
    for n, slot in enumerate(slots):
        lo, hi = cu[n], cu[n + 1]
        if hi == lo:
            continue
        sl = slice(lo, hi)
        ref_pool, o = _decode_loop(ref_pool, slot, inp["q"][sl], inp["k"][sl], inp["v"][sl], inp["a"][sl],
                                   inp["b"][sl], A_log, dt_bias)
        np.testing.assert_array_equal(o_p[sl], o)
    assert np.array_equal(pool_p, ref_pool)
    assert np.array_equal(pool_p[1], pool[1]) and np.array_equal(pool_p[3], pool[3])


@pytest.mark.parametrize("sdt", ["f32", "bf16"])
def test_prefill_two_call_split(sdt):
    """Two calls (first 55%, then the rest) equal one call whose write points are the split and
    the end; with an f32 state the split costs one f32 rounding (<= 1e-6 relative)."""
    sh = gen.DecodeShape(2, 1, 2, 8, 8)
    lens = [40, 23]
    first, second = gen.split_lengths(lens)
    A_log, dt_bias = gen.head_params(8, sh.Hv)
    pool = gen.pool_slots(8, range(2), sh.Hv, sh.dk, sh.dv, sdt)
    inp = gen.token_inputs(8, 0, (sum(lens),), sh.Hk, sh.Hv, sh.dk, sh.dv, "bf16", a_shift=-4.0)
    cu = gen.seq_lengths_cu(lens)
    one_pool, one_o = O.chunk_prefill(pool, [0, 1], cu, inp["q"], inp["k"], inp["v"], inp["a"], inp["b"],
                                      A_log, dt_bias)

    def part(sel_lens, offs):
        idx = np.concatenate([np.arange(cu[n] + offs[n], cu[n] + offs[n] + sel_lens[n]) for n in range(2)])
        return {k: v[idx] for k, v in inp.items()}, gen.seq_lengths_cu(sel_lens), idx

    p1, cu1, i1 = part(first, [0, 0])
    p2, cu2, i2 = part(second, first)
    mid_pool, o1 = O.chunk_prefill(pool, [0, 1], cu1, p1["q"], p1["k"], p1["v"], p1["a"], p1["b"], A_log, dt_bias)
    two_pool, o2 = O.chunk_prefill(mid_pool, [0, 1], cu2, p2["q"], p2["k"], p2["v"], p2["a"], p2["b"],
                                   A_log, dt_bias)
    two_o = np.zeros_like(one_o)
    two_o[i1] = o1
    two_o[i2] = o2
    tol = dict(f32=dict(rtol=1e-6, atol=1e-7), bf16=dict(rtol=0, atol=1e-2))[sdt]
    np.testing.assert_allclose(two_o, one_o, **tol)
    np.testing.assert_allclose(O.widen(two_pool), O.widen(one_pool), **tol)
    # exact form of the split: the per-sequence token loop with a rounding at the split point
    ratio = 2
    for n in range(2):
        for h in range(sh.Hv):
            sl = slice(cu[n], cu[n + 1])
            g, beta = O.gates(inp["a"][sl, h], inp["b"][sl, h], A_log[h], dt_bias[h])
            o, S = O.ref_gdn(O.widen(pool[n, h]), O.widen(inp["q"][sl, h // ratio]),
                             O.widen(inp["k"][sl, h // ratio]), O.widen(inp["v"][sl, h]), g, beta,
                             sh.dk ** -0.5, sdt, write_points=[first[n] - 1])
            np.testing.assert_array_equal(two_o[sl, h], o)
            assert np.array_equal(two_pool[n, h], O.to_storage(S, sdt))


# ---------------------------------------------------------------- replay
def _replay_setup(L, sdt, B=2, Hv=2, Hk=1, d=8, num_slots=3, cid=21):
    A_log, dt_bias = gen.head_params(cid, Hv)
    ckpt = gen.pool_slots(cid, range(num_slots), Hv, d, d, sdt)
    ring = O.new_ring(num_slots, Hv, L, d, d, "bf16")
    return A_log, dt_bias, ckpt, ring


def test_ring_schedule_golden():
    """start/count, fold steps and written ring indices follow the hand-worked schedules."""
    spec = json.load(open(os.path.join(GOLDEN, "ring_schedule_L4.json")))
    L = spec["L"]
    for sched in spec["schedules"]:
        A_log, dt_bias, ckpt, ring = _replay_setup(L, "f32", B=1, Hv=1, num_slots=1)
        for step, st in enumerate(sched["steps"]):
            T = st["T"]
            inp = gen.token_inputs(22, step, (1, T), 1, 1, 8, 8, "bf16")
            ck2, ring2, _ = O.replay_decode(ckpt, ring, [0], inp["q"], inp["k"], inp["v"], inp["a"], inp["b"],
                                            A_log, dt_bias)
            assert (not np.array_equal(ck2, ckpt)) == st["fold"], (sched["name"], step)
            assert [int(ring2.start[0, 0]), int(ring2.count[0, 0])] == st["after_step"]
            for t, j in enumerate(st["written"]):
                assert np.array_equal(ring2.k[0, 0, j], inp["k"][0, t, 0])
                assert np.array_equal(ring2.v[0, 0, j], inp["v"][0, t, 0])
            ring = O.replay_rollback(ring2, [0], [st["r"]])
            ckpt = ck2
            assert [int(ring.start[0, 0]), int(ring.count[0, 0])] == st["after_rollback"]


@pytest.mark.parametrize("sdt", ["f32", "bf16", "f16"])
def test_replay_L1_equals_decode(sdt):
    """L = 1 folds every step, so its rounding points are those of decode (gates stored in f32
    in the ring are the only difference)."""
    A_log, dt_bias, ckpt, ring = _replay_setup(1, sdt)
    pool = ckpt
    slots = [2, 0]
    for step in range(6):
        inp = gen.token_inputs(23, step, (2, 1), 1, 2, 8, 8, "bf16", a_shift=-3.0)
        ckpt, ring, o_r = O.replay_decode(ckpt, ring, slots, inp["q"], inp["k"], inp["v"], inp["a"], inp["b"],
                                          A_log, dt_bias)
        pool, o_d = O.decode_step(pool, slots, inp["q"][:, 0], inp["k"][:, 0], inp["v"][:, 0], inp["a"][:, 0],
                                  inp["b"][:, 0], A_log, dt_bias)
        np.testing.assert_allclose(o_r[:, 0], o_d, rtol=1e-5, atol=1e-6)
    ckpt, ring = O.replay_flush(ckpt, ring, slots)
    tol = 1e-6 if sdt == "f32" else 1e-2
    np.testing.assert_allclose(O.widen(ckpt), O.widen(pool), rtol=0, atol=tol)


def test_replay_f32_checkpoint_equals_decode_over_folds():
    """An f32 checkpoint with L = 4 over 17 steps (4 folds) tracks f32 decode within 1e-5."""
    A_log, dt_bias, ckpt, ring = _replay_setup(4, "f32")
    pool = ckpt
    slots = [1, 2]
    for step in range(17):
        inp = gen.token_inputs(24, step, (2, 1), 1, 2, 8, 8, "bf16", a_shift=-4.0)
        ckpt, ring, o_r = O.replay_decode(ckpt, ring, slots, inp["q"], inp["k"], inp["v"], inp["a"], inp["b"],
                                          A_log, dt_bias)
        pool, o_d = O.decode_step(pool, slots, inp["q"][:, 0], inp["k"][:, 0], inp["v"][:, 0], inp["a"][:, 0],
                                  inp["b"][:, 0], A_log, dt_bias)
        np.testing.assert_allclose(o_r[:, 0], o_d, rtol=1e-5, atol=1e-5)
    ckpt, ring = O.replay_flush(ckpt, ring, slots)
    np.testing.assert_allclose(O.widen(ckpt), O.widen(pool), rtol=1e-5, atol=1e-5)
    assert np.all(ring.count == 0)


def test_replay_spec_window_and_rollback():
    """Window position t reads the state after t+1 window tokens; after rolling back r and
    flushing, the checkpoint equals decode over the accepted tokens only."""
    A_log, dt_bias, ckpt, ring = _replay_setup(16, "f32")
    pool = ckpt
    slots = [0, 1]
    T = 5
    for step in range(4):
        inp = gen.token_inputs(25, step, (2, T), 1, 2, 8, 8, "bf16", a_shift=-4.0)
        r = gen.rejected_counts(25, step, 2, T - 1)
        ckpt, ring, o_r = O.replay_decode(ckpt, ring, slots, inp["q"], inp["k"], inp["v"], inp["a"], inp["b"],
                                          A_log, dt_bias)
        # window positions from a snapshot of the standard decode
        snap = pool
        for t in range(T):
            snap, o_d = O.decode_step(snap, slots, inp["q"][:, t], inp["k"][:, t], inp["v"][:, t],
                                      inp["a"][:, t], inp["b"][:, t], A_log, dt_bias)
            np.testing.assert_allclose(o_r[:, t], o_d, rtol=1e-5, atol=1e-5)
        ring = O.replay_rollback(ring, slots, r)
        # advance the standard decode over the accepted tokens of each sequence only
        for bi, slot in enumerate(slots):
            for t in range(T - int(r[bi])):
                pool, _ = O.decode_step(pool, [slot], inp["q"][bi:bi + 1, t], inp["k"][bi:bi + 1, t],
                                        inp["v"][bi:bi + 1, t], inp["a"][bi:bi + 1, t], inp["b"][bi:bi + 1, t],
                                        A_log, dt_bias)
    ckpt, ring = O.replay_flush(ckpt, ring, slots)
    np.testing.assert_allclose(O.widen(ckpt[slots]), O.widen(pool[slots]), rtol=1e-5, atol=1e-5)


def test_spec_decode_chain_equals_sequential_decode():
    """Keeping a state per window position: outputs equal T decode steps (f32 states within
    one f32 rounding), every destination slot holds the rounded state of its position."""
    sh = gen.DecodeShape(2, 1, 2, 8, 8)
    T = 4
    A_log, dt_bias = gen.head_params(26, sh.Hv)
    pool = gen.pool_slots(26, range(12), sh.Hv, sh.dk, sh.dv, "f32")
    inp = gen.token_inputs(26, 0, (2, T), 1, 2, 8, 8, "bf16", a_shift=-4.0)
    src = np.int32([0, 1])
    dst = np.int32([[2, 3, 4, 5], [6, 7, 8, 9]])
    pool2, o = O.spec_decode(pool, src, dst, inp["q"], inp["k"], inp["v"], inp["a"], inp["b"], A_log, dt_bias)
    ref = pool
    for t in range(T):
        ref, o_d = O.decode_step(ref, src, inp["q"][:, t], inp["k"][:, t], inp["v"][:, t], inp["a"][:, t],
                                 inp["b"][:, t], A_log, dt_bias)
        np.testing.assert_allclose(o[:, t], o_d, rtol=1e-6, atol=1e-7)
        for bi in range(2):
            np.testing.assert_allclose(O.widen(pool2[dst[bi, t]]), O.widen(ref[src[bi]]), rtol=1e-6, atol=1e-7)
    assert np.array_equal(pool2[:2], pool[:2]) and np.array_equal(pool2[10:], pool[10:])


def test_copy_state_blocks_worked_example():
    """Whole slots move byte for byte; out-of-range jobs are skipped per tensor; sources are the
    pre-call contents (a chain 0 -> 1, 1 -> 2 moves the old slot 1, not the new one)."""
    a = np.arange(4 * 3, dtype=np.int32).reshape(4, 3)          # slots 0..3
    b = np.arange(2 * 2, dtype=np.uint16).reshape(2, 2) + 100   # slots 0..1 only
    out_a, out_b = O.copy_state_blocks([a, b], [0, 1, 3], [1, 2, 0])
    assert out_a.tolist() == [[9, 10, 11], [0, 1, 2], [3, 4, 5], [9, 10, 11]]
    # in b, only the job 0 -> 1 is in range (slots 2 and 3 do not exist)
    assert out_b.tolist() == [[100, 101], [100, 101]]
    # inputs are not modified
    assert a.tolist()[1] == [3, 4, 5] and b.tolist()[1] == [102, 103]


def test_copy_state_blocks_keeps_bit_patterns():
    """NaN payloads and signed zeros survive the copy (it is a byte copy, not a value copy)."""
    x = np.array([[np.nan, -0.0], [1.0, 2.0]], np.float32)
    x.view(np.uint32)[0, 0] = 0x7FC0DEAD
    (y,) = O.copy_state_blocks([x], [0], [1])
    assert np.array_equal(y.view(np.uint32)[1], x.view(np.uint32)[0])


def test_replay_dual_master_tracks_f32_checkpoint_and_reads_the_copy():
    """Dual-precision checkpoint over 17 steps of L = 4 (4 folds):
    - the master follows the plain f32-checkpoint replay bit for bit (the copy never feeds back);
    - after every step the copy equals the master rounded once to bf16 (numpy-independent
      rounding checked against torch's bfloat16 cast);
    - on steps without a fold the outputs equal a plain replay whose checkpoint is the copy;
    - outputs stay within bf16 reach of the f32-checkpoint outputs."""
    import torch
    A_log, dt_bias, master, ring = _replay_setup(4, "f32")
    ref_ckpt, ref_ring = master, ring
    slots = [1, 2]
    copy = np.zeros(master.shape, np.uint16)
    master, copy, ring = O.replay_flush_dual(master, copy, ring, slots)
    for step in range(17):
        inp = gen.token_inputs(24, step, (2, 1), 1, 2, 8, 8, "bf16", a_shift=-4.0)
        args = (slots, inp["q"], inp["k"], inp["v"], inp["a"], inp["b"], A_log, dt_bias)
        folds = int(ring.count[slots[0], 0]) + 1 > ring.L
        _, _, o_copy = O.replay_decode(copy, ring, *args)
        master, copy, ring, o = O.replay_decode_dual(master, copy, ring, *args)
        ref_ckpt, ref_ring, o_ref = O.replay_decode(ref_ckpt, ref_ring, *args)
        assert np.array_equal(master, ref_ckpt)
        t = torch.from_numpy(master[slots].astype(np.float32)).to(torch.bfloat16)
        assert np.array_equal(copy[slots], t.view(torch.int16).numpy().view(np.uint16))
        if not folds:
            np.testing.assert_array_equal(o, o_copy)
        np.testing.assert_allclose(o, o_ref, rtol=0, atol=2e-2)
    # a dual flush folds what is left and refreshes the copy; on an empty ring it only refreshes
    master, copy, ring = O.replay_flush_dual(master, copy, ring, slots)
    assert np.all(ring.count[slots] == 0)
    blank = np.zeros_like(copy)
    master2, copy2, _ = O.replay_flush_dual(master, blank, ring, slots)
    assert np.array_equal(master2, master) and np.array_equal(copy2[slots], copy[slots])
