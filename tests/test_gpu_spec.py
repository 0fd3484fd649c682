"""GPU parity of gdn_spec_decode (one full state per window position) against the oracle.

Small cases compare every output and every destination state; the full-size
window (512 sequences, 32 value heads, 128 x 128 fp32 states, 5 positions)
compares sampled sequences, which the oracle computes one by one, and checks
that the other rows' destinations were written and untouched slots kept.
"""
import numpy as np
import pytest

import oracle as O
from workloads import gen

from gpu_util import DEV, POISON, assert_close, assert_poison_kept, dev, host, require_gpu, say, torch_dtype

pytestmark = pytest.mark.gpu

CID = 4  # the speculative-window workload's seeds


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    require_gpu()


def _device_pool(num_slots, Hv, D, sdt, src_rows, states):
    """Device pool filled with the poison pattern, the listed slots holding `states`."""
    import torch
    if sdt == "f32":
        pool = torch.empty((num_slots, Hv, D, D), dtype=torch.int32, device=DEV)
        pool.fill_(int(POISON["f32"].view(np.int32)))
        pool = pool.view(torch.float32)
    else:
        pool = torch.empty((num_slots, Hv, D, D), dtype=torch.int16, device=DEV)
        pool.fill_(int(POISON[sdt].view(np.int16)))
        pool = pool.view(torch_dtype(sdt))
    if len(src_rows):
        idx = torch.as_tensor(np.asarray(src_rows, np.int64), device=DEV)
        pool.index_copy_(0, idx, dev(states))
    return pool


def run_spec(B, T, Hk, Hv, D, sdt, in_dt, num_slots, src, dst, sample=None, out_dt="f32", a_shift=0.0):
    import torch
    import gated_deltanet_state_gdn_amd as gdn
    src = np.asarray(src, np.int32)
    dst = np.asarray(dst, np.int32).reshape(B, T)
    ok = lambda s: 0 <= s < num_slots  # noqa: E731
    src_valid = [int(s) for s in src if ok(s)]
    states = gen.pool_slots(CID, src_valid, Hv, D, D, sdt)
    pool_d = _device_pool(num_slots, Hv, D, sdt, src_valid, states)
    A_log, dt_bias = gen.head_params(CID, Hv)
    inp = gen.token_inputs(CID, 0, (B, T), Hk, Hv, D, D, in_dt, a_shift)
    out = torch.empty((B, T, Hv, D), dtype=torch_dtype(out_dt), device=DEV)
    say(f"spec B={B} T={T} Hk={Hk} Hv={Hv} D={D} state={sdt} in={in_dt} out={out_dt}")
    gdn.gdn_spec_decode(dev(inp["q"]), dev(inp["k"]), dev(inp["v"]), dev(inp["a"]), dev(inp["b"]), dev(A_log),
                        dev(dt_bias), pool_d, torch.from_numpy(src).to(DEV), torch.from_numpy(dst).to(DEV), out=out)
    torch.cuda.synchronize()

    rows = list(range(B)) if sample is None else list(sample)
    # oracle on a mini pool: per sampled row its source, then its destinations
    loc = {s: i for i, s in enumerate(src_valid)}
    mini, m_src, m_dst = [], np.full(len(rows), -1, np.int32), np.full((len(rows), T), -1, np.int32)
    for i, r in enumerate(rows):
        if ok(src[r]):
            m_src[i] = len(mini)
            mini.append(states[loc[int(src[r])]])
        for t in range(T):
            if ok(src[r]) and ok(dst[r, t]):
                m_dst[i, t] = len(mini)
                mini.append(np.zeros_like(states[0]) if len(states) else None)
    ref_pool = np.stack(mini) if mini else states[:0]
    sub = {k: v[rows] for k, v in inp.items()}
    ref_pool, o_ref = O.spec_decode(ref_pool, m_src, m_dst, sub["q"], sub["k"], sub["v"], sub["a"], sub["b"],
                                    A_log, dt_bias)
    o = host(out)
    assert np.all(np.isfinite(O.widen(o[rows]))), "non-finite output"
    assert_close(o[rows], o_ref, sdt if out_dt == "f32" else "bf16", "o")
    written = [int(dst[r, t]) for r in rows for t in range(T) if ok(src[r]) and ok(dst[r, t])]
    got = host(pool_d.index_select(0, torch.as_tensor(np.asarray(written or [0], np.int64), device=DEV)))
    j = 0
    for i, r in enumerate(rows):
        for t in range(T):
            if m_dst[i, t] >= 0:
                assert_close(got[j], ref_pool[m_dst[i, t]], sdt, f"row {r} position {t} slot {int(dst[r, t])}")
                j += 1
    # sources are only read; slots nobody names keep the poison
    if src_valid:
        src_back = host(pool_d.index_select(0, torch.as_tensor(np.asarray(src_valid[:8], np.int64), device=DEV)))
        assert np.array_equal(src_back.view(np.uint8), states[:8].view(np.uint8)), "a source slot was modified"
    # a padded row writes nothing, its destinations included
    pad_dst = [int(dst[r, t]) for r in range(B) if not ok(src[r]) for t in range(T) if ok(dst[r, t])]
    assert_poison_kept(pool_d, pad_dst, sdt)
    named = set(src_valid) | {int(s) for s in dst.ravel() if ok(s)}
    untouched = sorted(set(range(num_slots)) - named)
    assert_poison_kept(pool_d, untouched[:64], sdt)
    return o


def _layout(B, T, num_slots, seed):
    """Distinct source and destination slots drawn from a seeded permutation of the pool."""
    perm = np.random.default_rng(seed).permutation(num_slots).astype(np.int32)
    return perm[:B].copy(), perm[B:B + B * T].reshape(B, T).copy()


def test_spec_tiny():
    """2 sequences, 2 heads, 16 x 16 fp32 state, 3 positions; one destination skipped."""
    src = [3, 1]
    dst = [[0, 5, 6], [7, -1, 2]]
    run_spec(2, 3, 2, 2, 16, "f32", "f32", 8, src, dst)


@pytest.mark.parametrize("sdt", ["f32", "bf16", "f16"])
@pytest.mark.parametrize("D", [16, 64, 128])
def test_spec_parity(sdt, D):
    """9 sequences x 4 value heads (2 key heads), 5 positions, bf16 inputs; a padded row and a skipped write."""
    B, T, num_slots = 9, 5, 64
    src, dst = _layout(B, T, num_slots, 11 + D)
    src[4] = -1          # padded row: zero outputs, its destinations untouched
    dst[2, 3] = -1       # one skipped write
    o = run_spec(B, T, 2, 4, D, sdt, "bf16", num_slots, src, dst)
    assert np.all(O.widen(o[4]) == 0.0)


@pytest.mark.parametrize("in_dt", ["f32", "f16"])
def test_spec_input_dtypes(in_dt):
    B, T, num_slots = 6, 4, 40
    src, dst = _layout(B, T, num_slots, 5)
    run_spec(B, T, 2, 4, 32, "f32", in_dt, num_slots, src, dst)


def test_spec_long_window_bf16_out():
    """16 positions, slow decay (a shifted down), bf16 output."""
    B, T, num_slots = 4, 16, 80
    src, dst = _layout(B, T, num_slots, 7)
    run_spec(B, T, 1, 2, 64, "bf16", "bf16", num_slots, src, dst, out_dt="bf16", a_shift=-4.0)


@pytest.mark.parametrize("sdt", ["f32", "bf16"])
def test_spec_full_size_sampled(sdt):
    """512 sequences, 16 key / 32 value heads, 128 x 128 states, 5 positions: 3072 slots.  With
    bf16 states the 2.7 GB of destination tiles take the non-temporal store path."""
    B, T = 512, 5
    num_slots = B * (T + 1)
    src, dst = _layout(B, T, num_slots, 23)
    run_spec(B, T, 16, 32, 128, sdt, "bf16", num_slots, src, dst, sample=[0, 137, 511])
