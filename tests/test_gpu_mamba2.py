"""GPU parity of the Mamba2 entry points (decode, replay decode, flush, rollback) against the oracle.

Ring pointers and the live x / B entries must match bit for bit; stored g and dt' within FP32
transcendental error; outputs and states within the state-dtype tolerance.
"""
import numpy as np
import pytest

import oracle as O
from workloads import gen

from gpu_util import DEV, assert_close, dev, host, poisoned_pool, require_gpu, say, torch_dtype

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    require_gpu()


def _tdt(name):
    return torch_dtype(name)


@pytest.mark.parametrize("sdt", ["f32", "bf16", "f16"])
@pytest.mark.parametrize("d,n", [(16, 16), (64, 128), (128, 64), (16, 128)])
def test_mamba2_decode_parity(sdt, d, n):
    """9 sequences x 4 heads in 2 groups, 3 steps, bf16 inputs, one padded row; every element."""
    import torch
    import gated_deltanet_state_gdn_amd as gdn
    cid, B, H, G, num_slots = 70 + d + n, 9, 4, 2, 16
    slot_map = gen.slot_permutation(cid, num_slots)[:B].copy()
    slot_map[5] = -1
    valid = [int(s) for s in slot_map if s >= 0]
    pool_d, states = poisoned_pool(num_slots, H, d, n, sdt, valid, cid)
    ref = states
    ref_map = np.array([valid.index(int(s)) if s >= 0 else -1 for s in slot_map], np.int32)
    A_log, dt_bias, Dk = gen.m2_params(cid, H)
    P = [dev(t) for t in (A_log, dt_bias, Dk)]
    sm = torch.from_numpy(slot_map).to(DEV)
    for step in range(3):
        inp = gen.m2_inputs(cid, step, (B,), H, G, d, n, "bf16")
        say(f"mamba2 decode d={d} n={n} state={sdt} step={step}")
        y = gdn.gdn_mamba2_decode_step(dev(inp["x"]), dev(inp["Bm"]), dev(inp["Cm"]), dev(inp["dt"]), *P, pool_d, sm)
        torch.cuda.synchronize()
        ref, y_ref = O.mamba2_decode_step(ref, ref_map, inp["x"], inp["Bm"], inp["Cm"], inp["dt"], A_log, dt_bias,
                                          Dk)
        assert_close(host(y), y_ref, sdt, f"y step {step}")
    got = host(pool_d)
    for i, s in enumerate(valid):
        assert_close(got[s], ref[i], sdt, f"state slot {s}")


@pytest.mark.parametrize("in_dt", ["bf16", "f32", "f16"])
def test_mamba2_decode_full_heads_padded_rows(in_dt):
    """The benchmark layer's heads (128 of 64 x 128 in 8 groups, fp32 state) at B = 40: 5120
    workgroups of the one-shot kernel, with padded rows (-1 and past the pool) spread through
    the batch, two of them back to back; 2 steps, every element."""
    import torch
    import gated_deltanet_state_gdn_amd as gdn
    lay = gen.M2_LAYER
    cid, B, H, G, d, n, num_slots = 81, 40, lay["H"], lay["G"], lay["d"], lay["n"], 48
    slot_map = gen.slot_permutation(cid, num_slots)[:B].copy()
    slot_map[[2, 11, 12, 39]] = [-1, num_slots, -4, num_slots + 5]
    valid = [int(s) for s in slot_map if 0 <= s < num_slots]
    pool_d, states = poisoned_pool(num_slots, H, d, n, "f32", valid, cid)
    ref = states
    ref_map = np.array([valid.index(int(s)) if 0 <= s < num_slots else -1 for s in slot_map], np.int32)
    A_log, dt_bias, Dk = gen.m2_params(cid, H)
    P = [dev(t) for t in (A_log, dt_bias, Dk)]
    sm = torch.from_numpy(slot_map).to(DEV)
    for step in range(2):
        inp = gen.m2_inputs(cid, step, (B,), H, G, d, n, in_dt)
        say(f"mamba2 decode B={B} H={H} in={in_dt} step={step}")
        y = gdn.gdn_mamba2_decode_step(dev(inp["x"]), dev(inp["Bm"]), dev(inp["Cm"]), dev(inp["dt"]), *P, pool_d, sm)
        torch.cuda.synchronize()
        ref, y_ref = O.mamba2_decode_step(ref, ref_map, inp["x"], inp["Bm"], inp["Cm"], inp["dt"], A_log, dt_bias,
                                          Dk)
        assert_close(host(y), y_ref, "f32", f"y step {step}")
    got = host(pool_d)
    for i, s in enumerate(valid):
        assert_close(got[s], ref[i], "f32", f"state slot {s}")


class M2Case:
    def __init__(self, cid, B, H, G, d, n, L, sdt, num_slots, sample=None, in_dt="bf16"):
        import torch
        import gated_deltanet_state_gdn_amd as gdn
        self.cid, self.B, self.H, self.G, self.d, self.n, self.L, self.sdt = cid, B, H, G, d, n, L, sdt
        self.in_dt = in_dt
        self.slot_map = gen.slot_permutation(cid, num_slots)[:B]
        self.ckpt_d, states = poisoned_pool(num_slots, H, d, n, sdt, [int(s) for s in self.slot_map], cid)
        self.ring_d = gdn.new_m2_ring(num_slots, H, G, L, d, n, _tdt(in_dt), DEV)
        self.rows = list(range(B)) if sample is None else list(sample)
        self.ref_ckpt = states[self.rows]
        self.ref_ring = O.new_m2_ring(len(self.rows), H, G, L, d, n, in_dt)
        self.ref_map = np.arange(len(self.rows), dtype=np.int32)
        self.A_log, self.dt_bias, self.Dk = gen.m2_params(cid, H)
        self.P = [dev(t) for t in (self.A_log, self.dt_bias, self.Dk)]
        self.slot_d = torch.from_numpy(self.slot_map).to(DEV)

    def step(self, step, T, dt_shift=0.0):
        import torch
        import gated_deltanet_state_gdn_amd as gdn
        inp = gen.m2_inputs(self.cid, step, (self.B, T), self.H, self.G, self.d, self.n, self.in_dt, dt_shift)
        say(f"mamba2 replay cid={self.cid} B={self.B} d={self.d} n={self.n} L={self.L} T={T} ckpt={self.sdt} "
            f"step={step}")
        y = gdn.gdn_mamba2_replay_decode(dev(inp["x"]), dev(inp["Bm"]), dev(inp["Cm"]), dev(inp["dt"]), *self.P,
                                         self.ckpt_d, self.slot_d, self.ring_d)
        torch.cuda.synchronize()
        sub = {k: v[self.rows] for k, v in inp.items()}
        self.ref_ckpt, self.ref_ring, y_ref = O.mamba2_replay_decode(
            self.ref_ckpt, self.ref_ring, self.ref_map, sub["x"], sub["Bm"], sub["Cm"], sub["dt"], self.A_log,
            self.dt_bias, self.Dk)
        yh = host(y)
        assert np.all(np.isfinite(yh)), "non-finite output"
        assert_close(yh[self.rows], y_ref, "f32" if self.sdt == "f32" else "bf16", f"y step {step}")

    def rollback(self, step, r):
        import torch
        import gated_deltanet_state_gdn_amd as gdn
        say(f"mamba2 rollback cid={self.cid} step={step}")
        gdn.gdn_mamba2_replay_rollback(self.slot_d, torch.from_numpy(r).to(DEV), self.ring_d)
        torch.cuda.synchronize()
        self.ref_ring = O.mamba2_replay_rollback(self.ref_ring, self.ref_map, r[self.rows])

    def flush(self):
        import torch
        import gated_deltanet_state_gdn_amd as gdn
        say(f"mamba2 flush cid={self.cid}")
        gdn.gdn_mamba2_replay_flush(self.ckpt_d, self.slot_d, self.ring_d)
        torch.cuda.synchronize()
        self.ref_ckpt, self.ref_ring = O.mamba2_replay_flush(self.ref_ckpt, self.ref_ring, self.ref_map)

    def check_state(self, what):
        import torch
        slots = torch.as_tensor(self.slot_map[self.rows].astype(np.int64), device=DEV)
        assert_close(host(self.ckpt_d[slots]), self.ref_ckpt, self.sdt, f"{what}: checkpoint")
        st, cnt = host(self.ring_d.start[slots]), host(self.ring_d.count[slots])
        assert np.array_equal(st, self.ref_ring.start), f"{what}: ring start"
        assert np.array_equal(cnt, self.ref_ring.count), f"{what}: ring count"
        rx, rB = host(self.ring_d.x[slots]), host(self.ring_d.Bm[slots])
        rg, rd = host(self.ring_d.g[slots]), host(self.ring_d.dtp[slots])
        for i in range(len(self.rows)):
            live = [(int(st[i]) + e) % self.L for e in range(int(cnt[i]))]
            if not live:
                continue
            assert np.array_equal(rx[i][:, live], self.ref_ring.x[i][:, live]), f"{what}: ring x"
            assert np.array_equal(rB[i][:, live], self.ref_ring.Bm[i][:, live]), f"{what}: ring B"
            np.testing.assert_allclose(rg[i][:, live], self.ref_ring.g[i][:, live], rtol=1e-5, atol=1e-8)
            np.testing.assert_allclose(rd[i][:, live], self.ref_ring.dtp[i][:, live], rtol=1e-5, atol=1e-8)


@pytest.mark.parametrize("sdt", ["f32", "bf16"])
@pytest.mark.parametrize("d,n", [(16, 16), (64, 128)])
def test_mamba2_replay_standard_decode_with_folds(sdt, d, n):
    """T = 1, L = 4, 11 steps (folds at steps 4 and 8), every row checked, then a flush."""
    c = M2Case(80 + d, 5, 4, 2, d, n, 4, sdt, 8)
    for step in range(11):
        c.step(step, 1, dt_shift=1.0)
        c.check_state(f"step {step}")
    c.flush()
    c.check_state("flush")


def test_mamba2_replay_windows_with_rollback():
    """T = 3 windows on L = 8 with seeded rejections, 8 heads in 2 groups; then a flush."""
    c = M2Case(90, 6, 8, 2, 16, 64, 8, "f32", 10)
    for step in range(7):
        c.step(step, 3, dt_shift=1.0)
        c.check_state(f"step {step}")
        c.rollback(step, gen.rejected_counts(90, step, c.B, 2))
        c.check_state(f"rollback {step}")
    c.flush()
    c.check_state("flush")


@pytest.mark.parametrize("in_dt", ["f32", "f16"])
def test_mamba2_replay_input_dtypes(in_dt):
    c = M2Case(95, 4, 4, 1, 64, 16, 6, "f32", 6, in_dt=in_dt)
    for step in range(8):
        c.step(step, 2, dt_shift=1.0)
        c.check_state(f"step {step}")
    c.flush()
    c.check_state("flush")


def test_mamba2_replay_padded_row():
    import torch
    import gated_deltanet_state_gdn_amd as gdn
    c = M2Case(97, 3, 4, 2, 16, 16, 4, "f32", 6)
    c.slot_map = c.slot_map.copy()
    c.slot_map[1] = -1
    c.slot_d = torch.from_numpy(c.slot_map).to(DEV)
    inp = gen.m2_inputs(97, 0, (3, 1), 4, 2, 16, 16, "bf16")
    y = gdn.gdn_mamba2_replay_decode(dev(inp["x"]), dev(inp["Bm"]), dev(inp["Cm"]), dev(inp["dt"]), *c.P, c.ckpt_d,
                                     c.slot_d, c.ring_d)
    torch.cuda.synchronize()
    assert np.all(host(y)[1] == 0)


def test_mamba2_replay_full_layer_sampled():
    """The benchmark layer (128 heads of 64 x 128 in 8 groups, fp32 checkpoint, L = 16) at B = 128
    (a 640 MiB pool), over a fold, sampled rows checked."""
    lay = gen.M2_LAYER
    c = M2Case(5, 128, lay["H"], lay["G"], lay["d"], lay["n"], 16, "f32", 160, sample=[0, 77, 127])
    for step in range(18):
        c.step(step, 1)
        if step in (15, 16, 17):
            c.check_state(f"step {step}")


def test_mamba2_replay_B512_sampled():
    """The benchmark row's shape: B = 512 of the 128-head layer (64 x 128 fp32 checkpoints in a
    600-slot pool), L = 16, 18 steps over a fold, sampled rows spread over the batch."""
    lay = gen.M2_LAYER
    c = M2Case(6, 512, lay["H"], lay["G"], lay["d"], lay["n"], 16, "f32", 600, sample=[0, 200, 511])
    for step in range(18):
        c.step(step, 1)
        if step in (0, 15, 16, 17):
            c.check_state(f"step {step}")


def test_mamba2_decode_B512_sampled():
    """The benchmark row's decode: B = 512 of the 128-head layer, fp32 state, 3 steps; sampled rows
    against the oracle, every output finite."""
    import torch
    import gated_deltanet_state_gdn_amd as gdn
    lay = gen.M2_LAYER
    cid, B, H, G, d, n, num_slots = 7, 512, lay["H"], lay["G"], lay["d"], lay["n"], 600
    rows = [0, 300, 511]
    slot_map = gen.slot_permutation(cid, num_slots)[:B]
    pool_d, states = poisoned_pool(num_slots, H, d, n, "f32", [int(s) for s in slot_map], cid)
    ref = states[rows]
    A_log, dt_bias, Dk = gen.m2_params(cid, H)
    P = [dev(t) for t in (A_log, dt_bias, Dk)]
    sm = torch.from_numpy(slot_map).to(DEV)
    for step in range(3):
        inp = gen.m2_inputs(cid, step, (B,), H, G, d, n, "bf16")
        say(f"mamba2 decode B={B} step={step}")
        y = gdn.gdn_mamba2_decode_step(dev(inp["x"]), dev(inp["Bm"]), dev(inp["Cm"]), dev(inp["dt"]), *P, pool_d, sm)
        torch.cuda.synchronize()
        sub = {k: v[rows] for k, v in inp.items()}
        ref, y_ref = O.mamba2_decode_step(ref, np.arange(len(rows), dtype=np.int32), sub["x"], sub["Bm"], sub["Cm"],
                                          sub["dt"], A_log, dt_bias, Dk)
        yh = host(y)
        assert np.all(np.isfinite(yh)), "non-finite output"
        assert_close(yh[rows], y_ref, "f32", f"y step {step}")
    got = host(pool_d)
    for i, r in enumerate(rows):
        assert_close(got[int(slot_map[r])], ref[i], "f32", f"state row {r}")
