"""GPU parity of gdn_decode_step against the CPU oracle (same seeded inputs).

Small cases compare every output and every touched state element; the
full-size layer (B up to 512, 16 key / 32 value heads, 128 x 128 states)
compares sampled sequences, which the oracle computes one by one, plus
properties of the rest (finite outputs, untouched slots bit-identical).
"""
import numpy as np
import pytest

import oracle as O
from workloads import gen

from gpu_util import (DEV, TOL, assert_close, assert_poison_kept, dev, host, poisoned_pool, require_gpu, say,
                      torch_dtype)

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    require_gpu()


def run_decode(cid, B, Hk, Hv, D, sdt, in_dt, steps, num_slots, slot_map, sample=None, a_shift=0.0,
               out_dt="f32", check_every=1):
    import torch
    import gated_deltanet_state_gdn_amd as gdn
    slot_map = np.asarray(slot_map, np.int32)
    valid = [int(s) for s in slot_map if 0 <= s < num_slots]
    pool_d, states = poisoned_pool(num_slots, Hv, D, D, sdt, valid, cid)
    rows = list(range(B)) if sample is None else list(sample)
    # oracle state: a mini pool holding the sampled rows' slots
    loc = {s: i for i, s in enumerate(valid)}
    mini_rows = [r for r in rows if 0 <= slot_map[r] < num_slots]
    ref_pool = states[[loc[int(slot_map[r])] for r in mini_rows]] if mini_rows else states[:0]
    ref_map = np.full(len(rows), -1, np.int32)
    for i, r in enumerate(rows):
        if r in mini_rows:
            ref_map[i] = mini_rows.index(r)
    A_log, dt_bias = gen.head_params(cid, Hv)
    A_d, dt_d = dev(A_log), dev(dt_bias)
    slot_d = torch.from_numpy(slot_map).to(DEV)
    out = torch.empty((B, Hv, D), dtype=torch_dtype(out_dt), device=DEV)
    for step in range(steps):
        inp = gen.token_inputs(cid, step, (B,), Hk, Hv, D, D, in_dt, a_shift)
        say(f"decode cid={cid} B={B} Hk={Hk} Hv={Hv} D={D} state={sdt} in={in_dt} step={step}")
        gdn.gdn_decode_step(dev(inp["q"]), dev(inp["k"]), dev(inp["v"]), dev(inp["a"]), dev(inp["b"]), A_d, dt_d,
                            pool_d, slot_d, out=out)
        torch.cuda.synchronize()
        sub = {k: v[rows] for k, v in inp.items()}
        ref_pool, o_ref = O.decode_step(ref_pool, ref_map, sub["q"], sub["k"], sub["v"], sub["a"], sub["b"],
                                        A_log, dt_bias)
        if step % check_every == 0 or step == steps - 1:
            o = host(out)
            assert np.all(np.isfinite(O.widen(o))), "non-finite output"
            # outputs share the state dtype's bar (a bf16 output, or a rounded state, is a bf16-level result)
            assert_close(o[rows], o_ref, sdt if out_dt == "f32" else "bf16", f"o step {step}")
    got = host(pool_d)
    for i, r in enumerate(rows):
        s = int(slot_map[r])
        if 0 <= s < num_slots:
            assert_close(got[s], ref_pool[ref_map[i]], sdt, f"state slot {s}")
    untouched = sorted(set(range(num_slots)) - set(valid))
    assert_poison_kept(pool_d, untouched[:64], sdt)
    return got


def test_decode_tiny_recurrence():
    """2 sequences, 2 heads, 16 x 16 fp32 state, 8 steps, slots [3, 1] of a 4-slot pool."""
    cfg = gen.WORKLOADS["tiny"]
    s = cfg.shape
    run_decode(0, s.B, s.Hk, s.Hv, s.dk, "f32", "f32", cfg.steps, cfg.num_slots, cfg.extra["slot_map"])


@pytest.mark.parametrize("sdt", ["f32", "bf16", "f16"])
@pytest.mark.parametrize("D", [16, 32, 64, 128])
def test_decode_full_parity(sdt, D):
    """Every output and state element: 37 sequences x 4 value heads (2 key heads), 3 steps."""
    B, num_slots = 37, 48
    slot_map = gen.slot_permutation(100 + D, num_slots)[:B]
    run_decode(100 + D, B, 2, 4, D, sdt, "bf16", 3, num_slots, slot_map)


def test_decode_layer_f32_64_steps_sampled():
    """Full-size layer: B = 256, 16/32 heads, 128 x 128 fp32 states in a 1024-slot pool, 64 steps."""
    cfg = gen.WORKLOADS["decode_f32"]
    s = cfg.shape
    slot_map = gen.slot_permutation(1, cfg.num_slots)[:s.B]
    run_decode(1, s.B, s.Hk, s.Hv, s.dk, "f32", "bf16", cfg.steps, cfg.num_slots, slot_map,
               sample=[0, 1, 31, 97, 128, 129, 200, 254, 255], check_every=8)


def test_decode_layer_f32_B512_sampled():
    """The fp32 layer at B = 512 (16384 tiles, 64 per workgroup of the persistent kernel), 16 steps,
    sampled rows spread over the batch."""
    cfg = gen.WORKLOADS["decode_f32"]
    s = cfg.shape
    B = 512
    slot_map = gen.slot_permutation(11, cfg.num_slots)[:B]
    run_decode(11, B, s.Hk, s.Hv, s.dk, "f32", "bf16", 16, cfg.num_slots, slot_map,
               sample=[0, 1, 63, 64, 255, 256, 300, 449, 510, 511], check_every=5)


@pytest.mark.parametrize("B", [256, 512])
def test_decode_layer_f32_every_row(B):
    """Every output and every state element of the fp32 layer at B = 256 and 512 (the persistent
    kernel's launches of the headline and the large-batch row), over two steps."""
    cfg = gen.WORKLOADS["decode_f32"]
    s = cfg.shape
    slot_map = gen.slot_permutation(13, cfg.num_slots)[:B]
    run_decode(13, B, s.Hk, s.Hv, s.dk, "f32", "bf16", 2, cfg.num_slots, slot_map)


@pytest.mark.parametrize("sdt", ["bf16", "f16"])
@pytest.mark.parametrize("B", [1, 64, 256, 512])
def test_decode_layer_lowp_sampled(sdt, B):
    """bf16 / fp16 states, FP32 math, one rounding per step, B in {1, 64, 256, 512}."""
    cfg = gen.WORKLOADS["decode_lowp"]
    s = cfg.shape
    slot_map = gen.slot_permutation(2, cfg.num_slots)[:B]
    sample = sorted({0, B // 3, B - 1})
    run_decode(2, B, s.Hk, s.Hv, s.dk, sdt, "bf16", 8, cfg.num_slots, slot_map, sample=sample, check_every=4)


@pytest.mark.parametrize("sdt", ["f32", "bf16", "f16"])
def test_decode_slow_decay_state_carry(sdt):
    """a shifted by -6 (exp(g) close to 1): 32 steps of carried state and repeated rounding."""
    B, num_slots = 9, 12
    run_decode(7, B, 2, 4, 64, sdt, "bf16", 32, num_slots, gen.slot_permutation(7, num_slots)[:B], a_shift=-6.0,
               check_every=4)


def test_decode_padded_rows_and_bf16_output():
    """Slots -1 and >= num_slots are padding (zero output, nothing touched); bf16 outputs."""
    B, num_slots = 6, 8
    slot_map = np.int32([5, -1, 2, 8, 7, -7])
    got = run_decode(8, B, 1, 2, 32, "f32", "bf16", 2, num_slots, slot_map, out_dt="bf16")
    del got


@pytest.mark.parametrize("in_dt", ["bf16", "f32", "f16"])
def test_decode_persistent_walk_with_padded_rows(in_dt):
    """fp32 128 x 128 states: 80 rows x 32 value heads = 2560 tiles, about ten per workgroup of the
    persistent kernel (each input dtype is its own instantiation), with padded rows (-1 and past
    the pool) spread through the walk, two of them back to back, so live tiles sit on both sides
    of padded ones within a workgroup's walk."""
    B, num_slots = 80, 96
    slot_map = gen.slot_permutation(12, num_slots)[:B].copy()
    slot_map[[3, 17, 18, 40, 79]] = [-1, num_slots, -2, -5, num_slots + 3]
    run_decode(12, B, 16, 32, 128, "f32", in_dt, 3, num_slots, slot_map, out_dt="bf16")


def test_decode_one_shot_16bit_walk_with_padded_rows():
    """The same 2560-tile launch with bf16 states, which the one-shot kernel serves (one workgroup
    per tile), with the same padded rows."""
    B, num_slots = 80, 96
    slot_map = gen.slot_permutation(12, num_slots)[:B].copy()
    slot_map[[3, 17, 18, 40, 79]] = [-1, num_slots, -2, -5, num_slots + 3]
    run_decode(12, B, 16, 32, 128, "bf16", "bf16", 2, num_slots, slot_map, out_dt="bf16")


def test_decode_identity_token_keeps_state_bit_identical():
    """a = b = -200: exp(g) = 1 and beta = 0 in FP32, so the written state equals the read state
    bit for bit (also through bf16 storage) and o = scale S^T q."""
    import torch
    import gated_deltanet_state_gdn_amd as gdn
    B, Hk, Hv, D = 4, 2, 4, 128
    for sdt in ("f32", "bf16", "f16"):
        pool_d, states = poisoned_pool(4, Hv, D, D, sdt, [0, 1, 2, 3], 9)
        inp = gen.token_inputs(9, 0, (B,), Hk, Hv, D, D, "bf16")
        a = gen.store(np.full((B, Hv), -200.0, np.float32), "bf16")
        A_log, dt_bias = gen.head_params(9, Hv)
        slot = torch.arange(B, dtype=torch.int32, device=DEV)
        say(f"decode identity token state={sdt}")
        out = gdn.gdn_decode_step(dev(inp["q"]), dev(inp["k"]), dev(inp["v"]), dev(a), dev(a), dev(A_log),
                                  dev(dt_bias), pool_d, slot)
        torch.cuda.synchronize()
        assert np.array_equal(host(pool_d), states)
        ref = np.einsum("bhkv,bhk->bhv", O.widen(states), np.repeat(O.widen(inp["q"]), 2, axis=1)) * D ** -0.5
        np.testing.assert_allclose(host(out), ref, rtol=1e-5, atol=1e-6)


def test_decode_zero_batch_is_a_no_op():
    import torch
    import gated_deltanet_state_gdn_amd as gdn
    pool_d, states = poisoned_pool(2, 2, 16, 16, "f32", [0, 1], 10)
    e = torch.empty((0, 1, 16), dtype=torch.float32, device=DEV)
    ev = torch.empty((0, 2, 16), dtype=torch.float32, device=DEV)
    ea = torch.empty((0, 2), dtype=torch.float32, device=DEV)
    A_log, dt_bias = gen.head_params(10, 2)
    gdn.gdn_decode_step(e, e, ev, ea, ea, dev(A_log), dev(dt_bias), pool_d,
                        torch.empty(0, dtype=torch.int32, device=DEV))
    torch.cuda.synchronize()
    assert np.array_equal(host(pool_d), states)
