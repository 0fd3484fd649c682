"""Pins of the Mamba2 oracle (CPU): a hand-worked token, the unrolled closed form, group
mapping, and the replay identities (L = 1 equals decode; an f32 checkpoint over folds equals
decode; window positions and rollback)."""
import math

import numpy as np

import oracle as O
from workloads import gen


def test_hand_worked_token():
    """d = n = 2, S0 = diag(1, 2), x = (1, -1), B = (1, 2), C = (3, 1), dt = dt_bias = 0
    (dt' = ln 2), A_log = 0 (A = -1, so exp(g) = 1/2), D = 1/2:
    S1 = S0 / 2 + ln2 x B^T, y = S1 C + x / 2 = (2 + 5 ln 2, 1/2 - 5 ln 2)."""
    ln2 = math.log(2.0)
    pool = np.array([[[[1.0, 0.0], [0.0, 2.0]]]], np.float32)           # [1 slot, 1 head, 2, 2]
    x = np.array([[[1.0, -1.0]]], np.float32)
    Bm = np.array([[[1.0, 2.0]]], np.float32)
    Cm = np.array([[[3.0, 1.0]]], np.float32)
    dt = np.zeros((1, 1), np.float32)
    zero, half = np.zeros(1, np.float32), np.full(1, 0.5, np.float32)
    pool2, y = O.mamba2_decode_step(pool, [0], x, Bm, Cm, dt, zero, zero, half)
    S1 = np.array([[0.5 + ln2, 2 * ln2], [-ln2, 1.0 - 2 * ln2]])
    np.testing.assert_allclose(O.widen(pool2[0, 0]), S1, rtol=1e-7)
    np.testing.assert_allclose(y[0, 0], [2.0 + 5 * ln2, 0.5 - 5 * ln2], rtol=1e-12)


def test_token_loop_equals_unrolled_sum():
    """S_T = e^{G_T} S0 + sum_j e^{G_T - G_j} dt'_j x_j B_j^T, with G the prefix sums of g."""
    rg = np.random.default_rng(7)
    d, n, T = 5, 7, 9
    S0 = rg.standard_normal((d, n))
    x, Bv, Cv = rg.standard_normal((T, d)), rg.standard_normal((T, n)), rg.standard_normal((T, n))
    g, dtp = -rg.uniform(0, 1, T), rg.uniform(0, 0.5, T)
    S = S0.copy()
    for t in range(T):
        S, y = O.m2_token(S, x[t], Bv[t], Cv[t], g[t], dtp[t], 0.3)
        np.testing.assert_allclose(y, S @ Cv[t] + 0.3 * x[t], rtol=1e-12)
    G = np.cumsum(g)
    ref = math.exp(G[-1]) * S0 + sum(math.exp(G[-1] - G[j]) * dtp[j] * np.outer(x[j], Bv[j]) for j in range(T))
    np.testing.assert_allclose(S, ref, rtol=1e-12, atol=1e-12)


def test_gates_follow_the_softplus_form():
    g, dtp = O.m2_gates(np.float32([0.0, 40.0, -40.0]), np.float32([0.0, math.log(4.0), 0.0]),
                        np.float32([0.0, 0.0, 0.0]))
    np.testing.assert_allclose(dtp, [math.log(2.0), 40.0, math.log1p(math.exp(-40.0))], rtol=1e-12)
    np.testing.assert_allclose(g, -np.array([1.0, 4.0, 1.0]) * dtp, rtol=1e-7)  # A_log is stored in float32


def test_heads_read_contiguous_groups():
    """Zeroing C of group 1 (heads 2, 3 of 4 heads in 2 groups) leaves y = D x for exactly those heads."""
    H, G, d, n = 4, 2, 4, 6
    A_log, dt_bias, Dk = gen.m2_params(31, H)
    pool = gen.pool_slots(31, [0], H, d, n, "f32")
    inp = gen.m2_inputs(31, 0, (1,), H, G, d, n, "f32")
    inp["Cm"][:, 1] = 0
    _, y = O.mamba2_decode_step(pool, [0], inp["x"], inp["Bm"], inp["Cm"], inp["dt"], A_log, dt_bias, Dk)
    for h in range(H):
        skip = Dk[h] * O.widen(inp["x"][0, h])
        if h >= 2:
            np.testing.assert_allclose(y[0, h], skip, rtol=1e-12)
        else:
            assert np.abs(y[0, h] - skip).max() > 1e-3


def _setup(L, sdt, H=4, G=2, d=8, n=16, slots=3, cid=32):
    A_log, dt_bias, Dk = gen.m2_params(cid, H)
    ckpt = gen.pool_slots(cid, range(slots), H, d, n, sdt)
    ring = O.new_m2_ring(slots, H, G, L, d, n, "bf16")
    return A_log, dt_bias, Dk, ckpt, ring


def test_replay_L1_equals_decode():
    for sdt in ("f32", "bf16", "f16"):
        A_log, dt_bias, Dk, ckpt, ring = _setup(1, sdt)
        pool, slots = ckpt, [2, 0]
        for step in range(6):
            inp = gen.m2_inputs(32, step, (2, 1), 4, 2, 8, 16, "bf16", dt_shift=1.0)
            ckpt, ring, y_r = O.mamba2_replay_decode(ckpt, ring, slots, inp["x"], inp["Bm"], inp["Cm"], inp["dt"],
                                                     A_log, dt_bias, Dk)
            pool, y_d = O.mamba2_decode_step(pool, slots, inp["x"][:, 0], inp["Bm"][:, 0], inp["Cm"][:, 0],
                                             inp["dt"][:, 0], A_log, dt_bias, Dk)
            # the ring keeps g and dt' in float32: agreement to float32 resolution
            np.testing.assert_allclose(y_r[:, 0], y_d, rtol=1e-6, atol=1e-6)
        ckpt, ring = O.mamba2_replay_flush(ckpt, ring, slots)
        tol = 1e-6 if sdt == "f32" else 1e-2
        np.testing.assert_allclose(O.widen(ckpt[slots]), O.widen(pool[slots]), rtol=0, atol=tol)


def test_replay_f32_checkpoint_over_folds_equals_decode():
    A_log, dt_bias, Dk, ckpt, ring = _setup(4, "f32")
    pool, slots = ckpt, [1, 2]
    for step in range(15):
        inp = gen.m2_inputs(33, step, (2, 1), 4, 2, 8, 16, "bf16")
        ckpt, ring, y_r = O.mamba2_replay_decode(ckpt, ring, slots, inp["x"], inp["Bm"], inp["Cm"], inp["dt"],
                                                 A_log, dt_bias, Dk)
        pool, y_d = O.mamba2_decode_step(pool, slots, inp["x"][:, 0], inp["Bm"][:, 0], inp["Cm"][:, 0],
                                         inp["dt"][:, 0], A_log, dt_bias, Dk)
        np.testing.assert_allclose(y_r[:, 0], y_d, rtol=1e-5, atol=1e-6)
        # pointers: a fold every 4 steps, count cycles 1..4
        assert list(ring.count[slots]) == [step % 4 + 1] * 2
    ckpt, ring = O.mamba2_replay_flush(ckpt, ring, slots)
    np.testing.assert_allclose(O.widen(ckpt[slots]), O.widen(pool[slots]), rtol=1e-5, atol=1e-6)
    assert np.all(ring.count == 0)


def test_replay_window_and_rollback():
    """Window position t equals t + 1 decode steps from the checkpoint; after rolling back r and
    flushing, the checkpoint equals decode over the accepted tokens only."""
    A_log, dt_bias, Dk, ckpt, ring = _setup(8, "f32")
    pool, slots, T = ckpt, [0, 2], 3
    for step in range(4):
        inp = gen.m2_inputs(34, step, (2, T), 4, 2, 8, 16, "bf16")
        ckpt, ring, y = O.mamba2_replay_decode(ckpt, ring, slots, inp["x"], inp["Bm"], inp["Cm"], inp["dt"],
                                               A_log, dt_bias, Dk)
        snap = pool
        for t in range(T):
            snap, y_d = O.mamba2_decode_step(snap, slots, inp["x"][:, t], inp["Bm"][:, t], inp["Cm"][:, t],
                                             inp["dt"][:, t], A_log, dt_bias, Dk)
            np.testing.assert_allclose(y[:, t], y_d, rtol=1e-5, atol=1e-6)
        r = gen.rejected_counts(34, step, 2, 2)
        ring = O.mamba2_replay_rollback(ring, slots, r)
        for bi, slot in enumerate(slots):
            for t in range(T - int(r[bi])):
                pool, _ = O.mamba2_decode_step(pool, [slot], inp["x"][bi:bi + 1, t], inp["Bm"][bi:bi + 1, t],
                                               inp["Cm"][bi:bi + 1, t], inp["dt"][bi:bi + 1, t], A_log, dt_bias, Dk)
    ckpt, ring = O.mamba2_replay_flush(ckpt, ring, slots)
    np.testing.assert_allclose(O.widen(ckpt[slots]), O.widen(pool[slots]), rtol=1e-5, atol=1e-6)


def test_padded_rows_touch_nothing():
    A_log, dt_bias, Dk, ckpt, ring = _setup(4, "bf16")
    inp = gen.m2_inputs(35, 0, (2, 1), 4, 2, 8, 16, "bf16")
    ck2, ring2, y = O.mamba2_replay_decode(ckpt, ring, [-1, 7], inp["x"], inp["Bm"], inp["Cm"], inp["dt"],
                                           A_log, dt_bias, Dk)
    assert np.array_equal(ck2, ckpt) and np.all(ring2.count == 0) and np.all(y == 0)
    p2, y2 = O.mamba2_decode_step(ckpt, [-1, 3], inp["x"][:, 0], inp["Bm"][:, 0], inp["Cm"][:, 0], inp["dt"][:, 0],
                                  A_log, dt_bias, Dk)
    assert np.array_equal(p2, ckpt) and np.all(y2 == 0)
