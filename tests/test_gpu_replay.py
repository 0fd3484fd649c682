"""GPU parity of the ReplaySSM-style entry points (gdn_replay_decode, gdn_replay_flush,
gdn_replay_rollback) against the CPU oracle.

Ring pointers (start, count) and the live k / v entries must match bit for
bit; stored gates within FP32 transcendental error; outputs and checkpoints
within the state-dtype tolerance.
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


class ReplayCase:
    """copy_dt selects the dual-precision checkpoint: sdt must be f32 (the master) and the read
    copy of dtype copy_dt starts as poison, filled by an initial dual flush."""

    def __init__(self, cid, B, Hk, Hv, D, L, sdt, num_slots, sample=None, in_dt="bf16", copy_dt=None):
        import torch
        import gated_deltanet_state_gdn_amd as gdn
        self.cid, self.B, self.Hk, self.Hv, self.D, self.L, self.sdt = cid, B, Hk, Hv, D, L, sdt
        self.copy_dt = copy_dt
        self.num_slots, self.in_dt = num_slots, in_dt
        self.slot_map = gen.slot_permutation(cid, num_slots)[:B]
        self.ckpt_d, states = poisoned_pool(num_slots, Hv, D, D, sdt, [int(s) for s in self.slot_map], cid)
        self.ring_d = gdn.new_ring(num_slots, Hk, Hv, L, D, D, {"bf16": torch.bfloat16, "f32": torch.float32,
                                                               "f16": torch.float16}[in_dt], DEV)
        self.rows = list(range(B)) if sample is None else list(sample)
        # oracle: mini pool / ring over the sampled rows' slots, local slot i = sample row i
        self.ref_ckpt = states[self.rows]
        self.ref_ring = O.new_ring(len(self.rows), Hv, L, D, D, in_dt)
        self.ref_map = np.arange(len(self.rows), dtype=np.int32)
        self.A_log, self.dt_bias = gen.head_params(cid, Hv)
        self.A_d, self.dt_d = dev(self.A_log), dev(self.dt_bias)
        self.slot_d = torch.from_numpy(self.slot_map).to(DEV)
        self.copy_d = self.ref_copy = None
        self.exact_copy_steps = 0
        if copy_dt is not None:
            assert sdt == "f32"
            self.copy_d, _ = poisoned_pool(num_slots, Hv, D, D, copy_dt, [], cid)
            self.ref_copy = np.zeros(self.ref_ckpt.shape, {"bf16": np.uint16, "f16": np.float16}[copy_dt])
            self.flush()

    def step(self, step, T, a_shift=0.0):
        import torch
        import gated_deltanet_state_gdn_amd as gdn
        inp = gen.token_inputs(self.cid, step, (self.B, T), self.Hk, self.Hv, self.D, self.D, self.in_dt, a_shift)
        copy_exact = False
        if self.copy_dt is not None:
            # While the read copies of the sampled slots equal the oracle's bit for bit (always before
            # the first fold: both round the same fp32 master), outputs differ only by fp32 against
            # float64 arithmetic and take the fp32 bar.  After a fold the GPU's fp32 fold may land on
            # the other side of a 16-bit rounding boundary than the float64 one, and then the 16-bit bar
            # applies.
            slots = torch.as_tensor(self.slot_map[self.rows].astype(np.int64), device=DEV)
            copy_exact = np.array_equal(host(self.copy_d[slots]).view(np.uint16), self.ref_copy.view(np.uint16))
        say(f"replay cid={self.cid} B={self.B} D={self.D} L={self.L} T={T} ckpt={self.sdt} "
            f"copy={self.copy_dt} step={step}")
        out = gdn.gdn_replay_decode(dev(inp["q"]), dev(inp["k"]), dev(inp["v"]), dev(inp["a"]), dev(inp["b"]),
                                    self.A_d, self.dt_d, self.ckpt_d, self.slot_d, self.ring_d,
                                    read_copy=self.copy_d)
        torch.cuda.synchronize()
        sub = {k: v[self.rows] for k, v in inp.items()}
        args = (self.ref_map, sub["q"], sub["k"], sub["v"], sub["a"], sub["b"], self.A_log, self.dt_bias)
        if self.copy_dt is None:
            self.ref_ckpt, self.ref_ring, o_ref = O.replay_decode(self.ref_ckpt, self.ref_ring, *args)
        else:
            self.ref_ckpt, self.ref_copy, self.ref_ring, o_ref = O.replay_decode_dual(
                self.ref_ckpt, self.ref_copy, self.ref_ring, *args)
        o = host(out)
        self.last_out = o
        assert np.all(np.isfinite(o)), "non-finite output"
        tol = "f32" if self.sdt == "f32" and (self.copy_dt is None or copy_exact) else "bf16"
        assert_close(o[self.rows], o_ref, tol, f"o step {step}")
        self.exact_copy_steps += int(copy_exact)
        return inp

    def rollback(self, step, r):
        import torch
        import gated_deltanet_state_gdn_amd as gdn
        say(f"replay rollback cid={self.cid} step={step}")
        gdn.gdn_replay_rollback(self.slot_d, torch.from_numpy(r).to(DEV), self.ring_d, self.Hk, self.D)
        torch.cuda.synchronize()
        self.ref_ring = O.replay_rollback(self.ref_ring, self.ref_map, r[self.rows])

    def flush(self):
        import torch
        import gated_deltanet_state_gdn_amd as gdn
        say(f"replay flush cid={self.cid} copy={self.copy_dt}")
        gdn.gdn_replay_flush(self.ckpt_d, self.slot_d, self.ring_d, self.Hk, read_copy=self.copy_d)
        torch.cuda.synchronize()
        if self.copy_dt is None:
            self.ref_ckpt, self.ref_ring = O.replay_flush(self.ref_ckpt, self.ref_ring, self.ref_map)
        else:
            self.ref_ckpt, self.ref_copy, self.ref_ring = O.replay_flush_dual(self.ref_ckpt, self.ref_copy,
                                                                               self.ref_ring, self.ref_map)

    def check_state(self, what):
        import torch
        slots = torch.as_tensor(self.slot_map[self.rows].astype(np.int64), device=DEV)
        ck = host(self.ckpt_d[slots])
        assert_close(ck, self.ref_ckpt, self.sdt, f"{what}: checkpoint")
        if self.copy_dt is not None:
            assert_close(host(self.copy_d[slots]), self.ref_copy, self.copy_dt, f"{what}: read copy")
        # one pointer pair per slot on the GPU; the oracle keeps one per (slot, head), all equal
        st1, cnt1 = host(self.ring_d.start[slots]), host(self.ring_d.count[slots])
        st = np.repeat(st1[:, None], self.Hv, axis=1)
        cnt = np.repeat(cnt1[:, None], self.Hv, axis=1)
        assert np.array_equal(st, self.ref_ring.start), f"{what}: ring start"
        assert np.array_equal(cnt, self.ref_ring.count), f"{what}: ring count"
        rk, rv = host(self.ring_d.k[slots]), host(self.ring_d.v[slots])
        rg, rb = host(self.ring_d.g[slots]), host(self.ring_d.beta[slots])
        L = self.L
        for i in range(len(self.rows)):
            for h in range(self.Hv):
                live = [(int(st[i, h]) + e) % L for e in range(int(cnt[i, h]))]
                if not live:
                    continue
                # keys are kept once per key head (the oracle keeps them per value head)
                assert np.array_equal(rk[i, h // (self.Hv // self.Hk), live], self.ref_ring.k[i, h, live]), \
                    f"{what}: ring k"
                assert np.array_equal(rv[i, h, live], self.ref_ring.v[i, h, live]), f"{what}: ring v"
                np.testing.assert_allclose(rg[i, h, live], self.ref_ring.g[i, h, live], rtol=1e-5, atol=1e-8)
                np.testing.assert_allclose(rb[i, h, live], self.ref_ring.beta[i, h, live], rtol=1e-5, atol=1e-8)


@pytest.mark.parametrize("sdt", ["f32", "bf16"])
@pytest.mark.parametrize("D", [16, 128])
def test_replay_standard_decode_with_folds(sdt, D):
    """T = 1, L = 4, 11 steps (folds at steps 5 and 9), every row checked, then a flush."""
    c = ReplayCase(30 + D, 5, 1, 2, D, 4, sdt, 8)
    for step in range(11):
        c.step(step, 1, a_shift=-2.0)
        c.check_state(f"step {step}")
    c.flush()
    c.check_state("flush")


@pytest.mark.parametrize("D", [64, 128])
def test_replay_strong_decay_folds(D):
    """Strong decay (a + 6) on L = 16: within one fold the running decay of the tile drops far
    below 2^-64 and is folded into it; every row checked after each fold and the flush."""
    c = ReplayCase(61 + D, 4, 1, 2, D, 16, "f32", 6)
    for step in range(34):
        c.step(step, 1, a_shift=6.0)
        if step % 16 in (0, 15):
            c.check_state(f"step {step}")
    c.flush()
    c.check_state("flush")


@pytest.mark.parametrize("sdt,in_dt", [("f16", "bf16"), ("bf16", "f16"), ("f32", "f32")])
@pytest.mark.parametrize("D", [64, 128])
def test_replay_full_ring_folds(sdt, in_dt, D):
    """L = 16 (the fold's matrix form, every ring entry live): fp16 / bf16 / fp32 checkpoints with
    16-bit and fp32 inputs, T = 1 for 17 steps then windows of 3 with rollback, over folds."""
    c = ReplayCase(70 + D, 3, 1, 2, D, 16, sdt, 5, in_dt=in_dt)
    for step in range(17):
        c.step(step, 1, a_shift=-1.0)
        if step in (0, 15, 16):
            c.check_state(f"step {step}")
    for step in range(17, 23):
        c.step(step, 3, a_shift=-1.0)
        c.check_state(f"step {step}")
        c.rollback(step, gen.rejected_counts(70, step, c.B, 2))
    c.flush()
    c.check_state("flush")


@pytest.mark.parametrize("D", [64, 128])
def test_replay_long_windows(D):
    """L = 16 with windows of 16 (the whole ring, a fold before every step), 7 and 9, with
    rollback between them; bf16 inputs, fp32 checkpoint."""
    c = ReplayCase(80 + D, 3, 1, 2, D, 16, "f32", 5)
    for step, T in enumerate([16, 7, 9, 16, 5, 7]):
        c.step(step, T, a_shift=-1.0)
        c.check_state(f"step {step} T={T}")
        if step in (1, 4):
            c.rollback(step, gen.rejected_counts(80, step, c.B, 3))
            c.check_state(f"rollback {step}")
    c.flush()
    c.check_state("flush")


@pytest.mark.parametrize("sdt", ["f32", "bf16"])
def test_replay_spec_windows_with_rollback(sdt):
    """T = 3 windows on L = 8 with seeded rejections; then a flush."""
    c = ReplayCase(40, 6, 2, 4, 32, 8, sdt, 10)
    for step in range(7):
        c.step(step, 3, a_shift=-2.0)
        c.check_state(f"step {step}")
        c.rollback(step, gen.rejected_counts(40, step, c.B, 2))
        c.check_state(f"rollback {step}")
    c.flush()
    c.check_state("flush")


@pytest.mark.parametrize("in_dt", ["f32", "f16"])
@pytest.mark.parametrize("D", [16, 64])
def test_replay_input_dtypes(in_dt, D):
    """fp32 and fp16 inputs (rings of the same dtype), L = 6, windows of 2 with rollback, over folds."""
    c = ReplayCase(45 + D, 4, 1, 2, D, 6, "f32", 6, in_dt=in_dt)
    for step in range(7):
        c.step(step, 2, a_shift=-2.0)
        c.check_state(f"step {step}")
        c.rollback(step, gen.rejected_counts(45, step, c.B, 1))
    c.flush()
    c.check_state("flush")


def test_replay_L1_matches_decode_on_gpu():
    """L = 1 folds every step: outputs and checkpoint equal the decode kernel's."""
    import torch
    import gated_deltanet_state_gdn_amd as gdn
    c = ReplayCase(50, 4, 1, 2, 64, 1, "bf16", 6)
    pool_d = c.ckpt_d.clone()
    for step in range(5):
        inp = c.step(step, 1, a_shift=-2.0)
        o_dec = gdn.gdn_decode_step(dev(inp["q"][:, 0]), dev(inp["k"][:, 0]), dev(inp["v"][:, 0]),
                                    dev(inp["a"][:, 0]), dev(inp["b"][:, 0]), c.A_d, c.dt_d, pool_d, c.slot_d)
        torch.cuda.synchronize()
    c.flush()
    sl = c.slot_map.astype(np.int64)
    assert_close(host(c.ckpt_d)[sl], host(pool_d)[sl], "bf16", "checkpoint vs decode pool")
    del o_dec


def test_replay_layer_f32_sampled_over_a_fold():
    """Full-size layer: B = 512, 128 x 128 fp32 checkpoints, L = 16, 20 steps (fold at 17)."""
    cfg = gen.WORKLOADS["replay"]
    s = cfg.shape
    c = ReplayCase(4, s.B, s.Hk, s.Hv, s.dk, cfg.extra["L"], "f32", cfg.num_slots, sample=[0, 211, 511])
    for step in range(20):
        c.step(step, 1)
        if step in (0, 15, 16, 19):
            c.check_state(f"step {step}")


def test_replay_layer_bf16_spec_sampled():
    """Full-size layer, bf16 checkpoints, verify windows of T = 5 with rollback of 0..4 tokens."""
    cfg = gen.WORKLOADS["replay"]
    s = cfg.shape
    c = ReplayCase(41, s.B, s.Hk, s.Hv, s.dk, cfg.extra["L"], "bf16", cfg.num_slots, sample=[3, 300])
    T = cfg.extra["T_spec"]
    for step in range(8):
        c.step(step, T)
        c.rollback(step, gen.rejected_counts(41, step, s.B, T - 1))
    c.check_state("after spec steps")
    c.flush()
    c.check_state("flush")


@pytest.mark.parametrize("T,D,sdt", [(1, 128, "f32"), (3, 128, "f32"), (5, 128, "f32"), (7, 128, "f32"),
                                     (1, 64, "bf16")])
def test_replay_persistent_stream_padded_rows(T, D, sdt):
    """80 rows x 32 value heads (2560 units, about ten per workgroup of the persistent stream) with
    padded rows spread through the walk, windows of T tokens over enough steps to cross folds.
    fp32 128 x 128 checkpoints with T <= 5 take the persistent stream, T = 7 and the 64 x 64 bf16
    checkpoints the one-shot one; all of them the fused fold (its stream lists and appends).
    Padded rows read as zero outputs, the others match the oracle."""
    import torch
    c = ReplayCase(44 + T + (D != 128), 80, 16, 32, D, 16, sdt, 96, sample=[0, 5, 41, 78])
    pad = [3, 17, 40, 79]
    sm = c.slot_map.copy()
    sm[pad] = [-1, 96, -7, 200]
    c.slot_d = torch.from_numpy(sm).to(DEV)
    for step in range(18 if T == 1 else 8):
        c.step(step, T)
        assert np.all(c.last_out[pad] == 0), f"padded rows, step {step}"
    c.check_state("after a fold")


def test_replay_padded_rows():
    import torch
    import gated_deltanet_state_gdn_amd as gdn
    c = ReplayCase(60, 3, 1, 2, 16, 4, "f32", 4)
    c.slot_d = torch.tensor([-1, int(c.slot_map[1]), 4], dtype=torch.int32, device=DEV)
    before = host(c.ckpt_d)
    inp = gen.token_inputs(60, 0, (3, 2), 1, 2, 16, 16, "bf16")
    out = gdn.gdn_replay_decode(dev(inp["q"]), dev(inp["k"]), dev(inp["v"]), dev(inp["a"]), dev(inp["b"]), c.A_d,
                                c.dt_d, c.ckpt_d, c.slot_d, c.ring_d)
    torch.cuda.synchronize()
    o = host(out)
    assert np.all(o[0] == 0) and np.all(o[2] == 0) and np.any(o[1] != 0)
    cnt = host(c.ring_d.count)
    assert int(cnt[int(c.slot_map[1])]) == 2
    assert cnt.sum() == 2
    assert np.array_equal(host(c.ckpt_d).view(np.uint32), before.view(np.uint32))  # no fold, nothing written


@pytest.mark.parametrize("copy_dt", ["bf16", "f16"])
@pytest.mark.parametrize("D", [16, 128])
def test_replay_dual_precision_checkpoint(copy_dt, D):
    """fp32 master + 16-bit read copy: T = 1 on L = 4 over three folds, then a window of 3 with
    rollback, then a flush; master, copy, ring and outputs checked every step."""
    c = ReplayCase(60 + D, 5, 1, 2, D, 4, "f32", 8, copy_dt=copy_dt)
    c.check_state("initial flush")
    for step in range(13):
        c.step(step, 1, a_shift=-2.0)
        c.check_state(f"step {step}")
    c.step(13, 3, a_shift=-2.0)
    c.check_state("window")
    c.rollback(13, gen.rejected_counts(60, 13, c.B, 2))
    c.flush()
    c.check_state("flush")


def test_replay_dual_full_size_sampled():
    """B = 512, 32 value heads, 128 x 128 fp32 master with a bf16 read copy, L = 16, over a fold;
    the 16 steps before the fold read a copy equal to the oracle's and meet the fp32 bar."""
    c = ReplayCase(4, 512, 16, 32, 128, 16, "f32", 1024, sample=[0, 255, 511], copy_dt="bf16")
    for step in range(18):
        c.step(step, 1)
        if step in (15, 16, 17):
            c.check_state(f"step {step}")
    assert c.exact_copy_steps >= 16


@pytest.mark.parametrize("sdt", ["f32", "bf16"])
def test_replay_layer_staggered_rings(sdt):
    """The steady serving layout at full size: B = 512, 128 x 128 checkpoints, L = 16.  Sixteen
    one-token steps fill every ring, then a seeded rollback of 0..15 entries per row leaves
    staggered counts, so rows fold on different steps; 20 more steps cross each row's fold.
    Sampled rows with different counts are checked against the oracle throughout."""
    cfg = gen.WORKLOADS["replay"]
    s = cfg.shape
    L = cfg.extra["L"]
    r = gen.rejected_counts(14, 0, s.B, L - 1)
    # rows whose counts after the rollback differ: 16, 15, 9, 1 live entries (or what the draw gives)
    rows = sorted({int(np.argmin(r)), int(np.argmax(r)), 7, 300, 511})
    c = ReplayCase(14, s.B, s.Hk, s.Hv, s.dk, L, sdt, cfg.num_slots, sample=rows)
    for step in range(L):
        c.step(step, 1)
    c.rollback(L, r)
    c.check_state("staggered counts")
    assert len(set(int(x) for x in c.ref_ring.count[:, 0])) > 1
    for step in range(L + 1, 2 * L + 5):
        c.step(step, 1)
        if step % 4 == 0:
            c.check_state(f"step {step}")
    c.check_state("end")


@pytest.mark.parametrize("D", [16, 32, 64])
def test_replay_more_sequences_than_one_fold_plan_window(D):
    """4100 sequences: the fold kernels list the folding sequences in windows of 4096, so the
    last four sit in a second window.  Each fold kernel (rows at D = 16, columns at 32, MFMA at
    64) runs aligned folds, then staggered ones after a seeded rollback; sampled rows on both
    sides of the window boundary are checked against the oracle."""
    B, L = 4100, 4
    r = gen.rejected_counts(15, 0, B, L - 1)
    rows = [0, 1, 2047, 4095, 4096, 4097, 4099]
    c = ReplayCase(15, B, 1, 1, D, L, "f32", B + 16, sample=rows)
    for step in range(2 * L):  # every ring folds at step L and is full again after step 2 L - 1
        c.step(step, 1)
    c.check_state("aligned fold")
    c.rollback(2 * L, r)  # counts 1..4
    for step in range(2 * L + 1, 4 * L + 1):
        c.step(step, 1)
    c.check_state("staggered folds")


def test_replay_on_a_side_stream_with_internal_workspace():
    """A call on a stream other than the current one, with the workspace and output allocated by
    the binding: equal, bit for bit, to the same steps on the current stream."""
    import torch
    import gated_deltanet_state_gdn_amd as gdn
    outs = []
    for side in (False, True):
        c = ReplayCase(90, 6, 2, 4, 64, 4, "f32", 8)
        s = torch.cuda.Stream() if side else None
        res = []
        for step in range(6):
            inp = gen.token_inputs(90, step, (6, 1), 2, 4, 64, 64, "bf16")
            args = [dev(inp[x]) for x in "qkvab"]
            torch.cuda.synchronize()
            say(f"replay side stream={side} step={step}")
            if s is not None:
                s.wait_stream(torch.cuda.current_stream())
            o = gdn.gdn_replay_decode(*args, c.A_d, c.dt_d, c.ckpt_d, c.slot_d, c.ring_d, stream=s)
            if s is not None:
                torch.cuda.current_stream().wait_stream(s)
            res.append(o)
        torch.cuda.synchronize()
        outs.append([host(o) for o in res])
    for a, b in zip(*outs):
        assert np.array_equal(a.view(np.uint32), b.view(np.uint32))
