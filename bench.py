#!/usr/bin/env python3
"""GDN recurrent-state update benchmark on one MI355X.

Headline: single-token decode of a 16-key-head / 32-value-head layer with
128 x 128 fp32 states, B = 256 sequences (state pool of 1024 slots, bf16
q/k/v/a/b, bf16 outputs); a step is one gdn_decode_step (every decode row
of the hot path: slot lookup, gates, state read + decay, delta, rank-1
update + output, rounded write-back).  `value` is the algorithmic state-update
bandwidth in GB/s (1 GB = 1e9 B) with inputs resident in HBM; tokens/s and
the fraction of the 8 TB/s HBM peak are reported beside it.

Also measured in the same run (under "rows"): bf16/fp16-state decode, the
ReplaySSM-style replay decode (ring of 16, standard and 5-token verify
windows), the speculative window that keeps one state per position (the
baseline replay replaces) and the chunked prefill of 4 packed sequences, each with its own
roofline object.  Inputs are seeded synthetic data (workloads/gen.py).

python bench.py [--gpus 1] [--steps K] [--warmup W] [--only ROW] [--no-rows] [--no-cpu]
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0        # MI355X HBM3E
FP32_MFMA_PEAK_TFS = 157.3   # MI355X dense fp32 matrix
METRIC = "GDN decode state-update GB/s + tokens/s, % of HBM peak (B=256,H=32,128×128)"
HK, HV, D = 16, 32, 128
NUM_SLOTS = 1024
SB = {"f32": 4, "bf16": 2, "f16": 2}
CSRC = os.path.join(ROOT, "gated_deltanet_state_gdn_amd", "csrc")
TRAFFIC = os.path.join(ROOT, "profiles", "traffic.json")


def log(*a):
    print(*a, file=sys.stderr, flush=True)


# ------------------------------------------------------------------ byte / flop models
def decode_bytes(B, sdt, ib=2, ob=2, Hk=HK, Hv=HV, d=D):
    """Algorithmic bytes of one decode step: state read + write, inputs, gates, slot map, outputs."""
    state = 2 * B * Hv * d * d * SB[sdt]
    inputs = B * (2 * Hk * d + Hv * d + 2 * Hv) * ib + 2 * Hv * 4 + B * 4
    return state + inputs + B * Hv * d * ob


def replay_entry_bytes(ib=2, Hk=HK, Hv=HV, d=D):
    """One ring entry of one sequence: k per key head, v per value head, g and beta per value head."""
    return (Hk * d + Hv * d) * ib + 2 * Hv * 4


def replay_step_bytes(B, sdt, n_before, T, L, ib=2, ob=2, Hk=HK, Hv=HV, d=D, copy_dt=None):
    """Algorithmic bytes of one replay step of T tokens when every sequence holds n_before entries.
    With copy_dt (dual-precision checkpoint) outputs read the copy and a fold also writes it."""
    fold = n_before + T > L
    tile = B * Hv * d * d
    if copy_dt is None:
        state = tile * SB[sdt] * (2 if fold else 1)
    else:
        state = tile * SB[copy_dt] + (tile * (2 * SB[sdt] + SB[copy_dt]) if fold else 0)
    entries = B * n_before * replay_entry_bytes(ib, Hk, Hv, d)       # committed entries read
    appended = B * T * replay_entry_bytes(ib, Hk, Hv, d)             # new entries written
    inputs = B * T * (2 * Hk * d + Hv * d + 2 * Hv) * ib + 2 * Hv * 4 + B * 4 + 2 * B * 4
    return state + entries + appended + inputs + B * T * Hv * d * ob


def replay_rows_step_bytes(counts, sdt, T, L, copy_dt=None):
    """replay_step_bytes for rows that hold different numbers of entries (the gate parameters,
    read once per step, are counted once)."""
    head = 2 * HV * 4
    return head + sum(replay_step_bytes(1, sdt, int(n), T, L, copy_dt=copy_dt) - head for n in counts)


def spec_bytes(B, sdt, T, ib=2, ob=2, Hk=HK, Hv=HV, d=D):
    """Algorithmic bytes of one speculative window that keeps every state: the source read once, T
    destination states written, inputs, gates, slot tables and outputs."""
    state = B * Hv * d * d * SB[sdt] * (1 + T)
    inputs = B * T * (2 * Hk * d + Hv * d + 2 * Hv) * ib + 2 * Hv * 4 + B * (1 + T) * 4
    return state + inputs + B * T * Hv * d * ob


def prefill_bytes(lengths, sdt, ib=2, ob=2, Hk=HK, Hv=HV, d=D):
    T, N = sum(lengths), len(lengths)
    return (T * (2 * Hk * d + Hv * d + 2 * Hv) * ib + T * Hv * d * ob + 2 * N * Hv * d * d * SB[sdt]
            + 2 * Hv * 4 + (2 * N + 1) * 4)


def prefill_flops(lengths, Hv=HV, d=D, C=64):
    """FLOPs of the chunked form as this library computes it: per (chunk, value head) K K^T, Q K^T,
    T R and P U (2 C^2 d each) and [K; Q] S, K~^T U (2 C d^2 each, three).  U = T R with
    R = diag(beta)(V - diag(e^gamma) K S) replaces W = T diag(beta e^gamma) K, W S and
    U' = T diag(beta) V, one C^2 d product fewer than the textbook count below."""
    chunks = sum((n + C - 1) // C for n in lengths)
    per = 4 * 2 * C * C * d + 3 * 2 * C * d * d
    state_kernel = 2 * 2 * C * C * d + 3 * 2 * C * d * d
    return chunks * Hv * per, chunks * Hv * state_kernel


def prefill_flops_method(lengths, Hv=HV, d=D, C=64):
    """The method's chunked-form work per token and value head: K K^T, the two WY factors
    W = T diag(beta e^gamma) K and U' = T diag(beta) V, Q K^T and (M o Q K^T) U (2 C d each per
    token), W S, Q S and K~^T U (2 d^2 each), and the triangular inverse (C^2 / 3): 181.6 kFLOP
    per token per value head at C = 64, d = 128."""
    return sum(lengths) * Hv * (5 * 2 * C * d + 3 * 2 * d * d + C * C // 3)


def counters_for(key, sources):
    """The whole counter record (traffic and MFMA counters) if taken on the current kernel sources."""
    try:
        with open(TRAFFIC) as f:
            t = json.load(f).get(key)
    except (OSError, ValueError):
        return None
    if not t or t.get("source_sha256") != kernel_sources_sha(sources):
        return None
    return t


# ------------------------------------------------------------------ timing helpers
def kernel_sources_sha(names):
    h = hashlib.sha256()
    for n in names:
        with open(os.path.join(CSRC, n), "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def traffic_for(key, sources):
    """Counter-measured HBM bytes per launch, if taken on the current kernel sources."""
    try:
        with open(TRAFFIC) as f:
            t = json.load(f).get(key)
    except (OSError, ValueError):
        return None
    if not t or t.get("source_sha256") != kernel_sources_sha(sources):
        return None
    return t.get("bytes_per_launch")


def timed_launches(torch, fn, n_launch, warmup):
    """Run fn(i) for i in [0, warmup + n): warmup untimed calls, then n timed back to back.

    One event pair on the launch stream brackets the n calls, with a
    synchronize on both sides; the mean launch time is the span over n.  No
    events sit between the calls: an event pair around every call leaves the
    GPU idle for about 10 us between kernels (kernel trace: back to back
    without them, 10 us apart with them)."""
    for i in range(warmup):
        fn(i)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    e0.record()
    for i in range(n_launch):
        fn(warmup + i)
    e1.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    span = e0.elapsed_time(e1)
    return dict(mean_launch_ms=span / n_launch, span_ms=span, wall_s=wall)


def roofline_bw(bytes_per_launch, mean_launch_ms, traffic):
    gbs = bytes_per_launch / (mean_launch_ms * 1e-3) / 1e9
    return {"bound": "hbm", "achieved": round(gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
            "frac": round(gbs / HBM_PEAK_GBS, 4), "traffic": traffic}


# ------------------------------------------------------------------ workloads
def make_pool(torch, gen, cid, slots, sdt, device):
    import numpy as np
    pool = torch.zeros((NUM_SLOTS, HV, D, D), dtype={"f32": torch.float32, "bf16": torch.bfloat16,
                                                      "f16": torch.float16}[sdt], device=device)
    chunk = 64
    for i in range(0, len(slots), chunk):
        sl = list(slots[i:i + chunk])
        pool[torch.as_tensor(np.asarray(sl, np.int64), device=device)] = gen.to_torch(
            gen.pool_slots(cid, sl, HV, D, D, sdt), device)
    return pool


def bench_decode(torch, gdn, gen, B, sdt, steps, warmup, cid=1):
    dev = "cuda"
    slot_map = gen.slot_permutation(cid, NUM_SLOTS)[:B]
    pool = make_pool(torch, gen, cid, slot_map, sdt, dev)
    A_log, dt_bias = gen.head_params(cid, HV)
    A_d, dt_d = gen.to_torch(A_log, dev), gen.to_torch(dt_bias, dev)
    sm = torch.from_numpy(slot_map).to(dev)
    ins = []
    for s in range(warmup + steps):
        inp = gen.token_inputs(cid, s, (B,), HK, HV, D, D, "bf16")
        ins.append([gen.to_torch(inp[x], dev) for x in "qkvab"])
    out = torch.empty((B, HV, D), dtype=torch.bfloat16, device=dev)

    def fn(i):
        q, k, v, a, b = ins[i % len(ins)]
        gdn.gdn_decode_step(q, k, v, a, b, A_d, dt_d, pool, sm, out=out)

    t = timed_launches(torch, fn, steps, warmup)
    nbytes = decode_bytes(B, sdt)
    ms = t["span_ms"] / steps
    res = {
        "B": B, "state": sdt, "ms_per_step": round(ms, 5), "mean_launch_us": round(t["mean_launch_ms"] * 1e3, 2),
        "GB_per_s": round(nbytes / (ms * 1e-3) / 1e9, 1), "tokens_per_s": round(B / (ms * 1e-3), 1),
        "bytes_per_step": nbytes,
        "working_set_MiB": round(B * HV * D * D * SB[sdt] / 2 ** 20, 1),
    }
    src = ["gdn_decode.hip", "gdn_device.h"]
    res["roofline"] = roofline_bw(nbytes, t["mean_launch_ms"], traffic_for(f"decode_{sdt}_B{B}", src))
    if res["working_set_MiB"] <= 256:
        res["note"] = "state working set fits the 256 MB Infinity Cache: cache-assisted, not an HBM-only figure"
    del pool, ins
    torch.cuda.empty_cache()
    return res


def bench_replay(torch, gdn, gen, B, sdt, T, cycles, L=16, cid=4, copy_dt=None, staggered=False):
    """Aligned rings (every sequence starts empty): 1 untimed cycle, then `cycles` timed cycles.
    copy_dt selects the dual-precision checkpoint (sdt is then the f32 master).  staggered: the
    steady serving layout; L one-token steps fill every ring, then a seeded rollback of 0..L-1
    entries per row leaves the rows' counts spread over 1..L, so each step folds about 1/L of the
    rows (untimed setup, then the same warm-up and timed cycles)."""
    import numpy as np
    dev = "cuda"
    steps_per_cycle = L // T if T > 1 else L
    slot_map = gen.slot_permutation(cid, NUM_SLOTS)[:B]
    ckpt = make_pool(torch, gen, cid, slot_map, sdt, dev)
    ring = gdn.new_ring(NUM_SLOTS, HK, HV, L, D, D, torch.bfloat16, dev)
    copy = None
    if copy_dt is not None:
        copy = torch.empty((NUM_SLOTS, HV, D, D), dtype={"bf16": torch.bfloat16, "f16": torch.float16}[copy_dt],
                           device=dev)
        gdn.gdn_replay_flush(ckpt, torch.from_numpy(slot_map).to(dev), ring, HK, read_copy=copy)
    A_log, dt_bias = gen.head_params(cid, HV)
    A_d, dt_d = gen.to_torch(A_log, dev), gen.to_torch(dt_bias, dev)
    sm = torch.from_numpy(slot_map).to(dev)
    n_in = steps_per_cycle * 2  # inputs are reused across cycles
    ins = []
    for s in range(n_in):
        inp = gen.token_inputs(cid, s, (B, T), HK, HV, D, D, "bf16")
        ins.append([gen.to_torch(inp[x], dev) for x in "qkvab"])
    out = torch.empty((B, T, HV, D), dtype=torch.bfloat16, device=dev)
    ws = torch.empty(gdn.gdn_replay_workspace_bytes(HK, HV, D, D, B, T), dtype=torch.uint8, device=dev)
    warm = steps_per_cycle
    n = cycles * steps_per_cycle
    cnt = np.zeros(B, np.int64)  # every row's committed entries before the next step

    def fn(i):
        q, k, v, a, b = ins[i % n_in]
        gdn.gdn_replay_decode(q, k, v, a, b, A_d, dt_d, ckpt, sm, ring, out=out, workspace=ws, read_copy=copy)

    if staggered:
        for i in range(L):  # fill every ring with one-token steps
            q, k, v, a, b = ins[i % n_in]
            gdn.gdn_replay_decode(q[:, :1].contiguous(), k[:, :1].contiguous(), v[:, :1].contiguous(),
                                  a[:, :1].contiguous(), b[:, :1].contiguous(), A_d, dt_d, ckpt, sm, ring,
                                  out=out[:, :1].contiguous(), workspace=ws, read_copy=copy)
        r = gen.rejected_counts(cid, 0, B, L - 1)
        gdn.gdn_replay_rollback(sm, torch.from_numpy(r).to(dev), ring, HK, D)
        torch.cuda.synchronize()
        cnt = L - r.astype(np.int64)
        got = ring.count[torch.from_numpy(slot_map.astype(np.int64)).to(dev)].cpu().numpy()
        assert np.array_equal(got, cnt), "staggered ring counts"
    t = timed_launches(torch, fn, n, warm)
    # byte model follows the (deterministic) per-row counts of the schedule
    nbytes = 0
    for i in range(warm + n):
        b_i = replay_rows_step_bytes(cnt, sdt, T, L, copy_dt=copy_dt)
        cnt = np.where(cnt + T > L, 0, cnt) + T
        if i >= warm:
            nbytes += b_i
    ms = t["span_ms"] / n
    res = {
        "B": B, "ckpt": sdt if copy_dt is None else f"{sdt} master + {copy_dt} read copy", "L": L, "T": T,
        "rings": "staggered (counts spread over 1..L by a seeded rollback after a full ring)" if staggered
                 else "aligned (every row starts empty)",
        "ms_per_step": round(ms, 5),
        "mean_launch_us": round(t["mean_launch_ms"] * 1e3, 2),
        "GB_per_s": round(nbytes / n / (ms * 1e-3) / 1e9, 1), "tokens_per_s": round(B * T / (ms * 1e-3), 1),
        "bytes_per_step_avg": nbytes // n,
        "vs_decode_bytes": round(nbytes / n / (T * decode_bytes(B, sdt)), 3),
    }
    src = ["gdn_replay.hip", "gdn_device.h"]
    key = f"replay_{sdt}_B{B}_T{T}" if copy_dt is None else f"replay_dual_{copy_dt}_B{B}_T{T}"
    key += "_staggered" if staggered else ""
    res["roofline"] = roofline_bw(nbytes / n, t["mean_launch_ms"], traffic_for(key, src))
    del ckpt, ring, ins, ws, copy
    torch.cuda.empty_cache()
    return res


def bench_spec(torch, gdn, gen, B, sdt, T, reps, cid=4):
    """Speculative window of T tokens keeping one state per position (source + T destinations per row)."""
    import numpy as np
    dev = "cuda"
    num_slots = B * (T + 1)
    perm = gen.slot_permutation(cid, num_slots)
    src, dst = perm[:B].copy(), perm[B:].reshape(B, T).copy()
    pool = torch.zeros((num_slots, HV, D, D), dtype={"f32": torch.float32, "bf16": torch.bfloat16,
                                                     "f16": torch.float16}[sdt], device=dev)
    for i in range(0, B, 64):
        sl = src[i:i + 64]
        pool[torch.as_tensor(sl.astype(np.int64), device=dev)] = gen.to_torch(
            gen.pool_slots(cid, sl, HV, D, D, sdt), dev)
    A_log, dt_bias = gen.head_params(cid, HV)
    A_d, dt_d = gen.to_torch(A_log, dev), gen.to_torch(dt_bias, dev)
    src_d, dst_d = torch.from_numpy(src).to(dev), torch.from_numpy(dst).to(dev)
    ins = []
    for s in range(2):
        inp = gen.token_inputs(cid, s, (B, T), HK, HV, D, D, "bf16")
        ins.append([gen.to_torch(inp[x], dev) for x in "qkvab"])
    out = torch.empty((B, T, HV, D), dtype=torch.bfloat16, device=dev)

    def fn(i):
        q, k, v, a, b = ins[i % 2]
        gdn.gdn_spec_decode(q, k, v, a, b, A_d, dt_d, pool, src_d, dst_d, out=out)

    t = timed_launches(torch, fn, reps, 2)
    nbytes = spec_bytes(B, sdt, T)
    ms = t["span_ms"] / reps
    res = {
        "B": B, "state": sdt, "T": T, "ms_per_step": round(ms, 5), "mean_launch_us": round(t["mean_launch_ms"] * 1e3, 2),
        "GB_per_s": round(nbytes / (ms * 1e-3) / 1e9, 1), "tokens_per_s": round(B * T / (ms * 1e-3), 1),
        "bytes_per_step": nbytes, "state_MiB": round(num_slots * HV * D * D * SB[sdt] / 2 ** 20, 1),
    }
    src_files = ["gdn_spec.hip", "gdn_device.h"]
    res["roofline"] = roofline_bw(nbytes, t["mean_launch_ms"], traffic_for(f"spec_{sdt}_B{B}_T{T}", src_files))
    del pool, ins, out
    torch.cuda.empty_cache()
    return res


def bench_prefill(torch, gdn, gen, sdt, reps, cid=3):
    import numpy as np
    dev = "cuda"
    lengths = gen.WORKLOADS["prefill"].extra["lengths"]
    N = len(lengths)
    cu = gen.seq_lengths_cu(lengths)
    slot_map = gen.slot_permutation(cid, 16)[:N]
    pool = torch.zeros((16, HV, D, D), dtype={"f32": torch.float32, "bf16": torch.bfloat16}[sdt], device=dev)
    pool[torch.as_tensor(slot_map.astype(np.int64), device=dev)] = gen.to_torch(
        gen.pool_slots(cid, slot_map, HV, D, D, sdt), dev)
    inp = gen.token_inputs(cid, 0, (int(cu[-1]),), HK, HV, D, D, "bf16")
    A_log, dt_bias = gen.head_params(cid, HV)
    args = [gen.to_torch(inp[x], dev) for x in "qkvab"] + [gen.to_torch(A_log, dev), gen.to_torch(dt_bias, dev)]
    sm, cu_d = torch.from_numpy(slot_map).to(dev), torch.from_numpy(cu).to(dev)
    out = torch.empty((int(cu[-1]), HV, D), dtype=torch.bfloat16, device=dev)
    ws = torch.empty(gdn.gdn_chunk_prefill_workspace_bytes(HK, HV, D, D, N, int(cu[-1])), dtype=torch.uint8,
                     device=dev)

    def fn(i):
        gdn.gdn_chunk_prefill(*args, pool, sm, cu_d, out=out, workspace=ws)

    t = timed_launches(torch, fn, reps, 2)
    nbytes = prefill_bytes(lengths, sdt)
    flops_lib, flops_state = prefill_flops(lengths)
    flops = prefill_flops_method(lengths)
    ms = t["span_ms"] / reps
    tf = flops / (ms * 1e-3) / 1e12
    rec = counters_for(f"prefill_{sdt}", ["gdn_prefill.hip", "gdn_device.h"])
    res = {
        "lengths": lengths, "state": sdt, "ms_per_call": round(ms, 4), "tokens_per_s": round(sum(lengths) / (ms * 1e-3)),
        "GB_per_s": round(nbytes / (ms * 1e-3) / 1e9, 1), "bytes_per_call": nbytes, "flops_per_call": flops,
        "flops_as_computed": flops_lib,
        "roofline": {"bound": "mfma", "achieved": round(tf, 2), "peak": FP32_MFMA_PEAK_TFS, "unit": "TFLOP/s",
                     "frac": round(tf / FP32_MFMA_PEAK_TFS, 4), "traffic": rec["bytes_per_launch"] if rec else None,
                     "scope": "whole call (chunk kernel + state kernel); the method's chunked-form FLOPs "
                              "(181.6 kFLOP per token per value head); fp32-accurate products, those with a key "
                              "or query operand run as three-term bf16 splits; against the fp32 MFMA peak"},
        "workspace_MiB": round(ws.numel() / 2 ** 20, 1),
    }
    if rec and "mfma" in rec:
        m = rec["mfma"]
        # time the issued MFMA instructions would take at their own peaks, against the measured call
        at_peak_us = (m["bf16_flops"] / 2.5e15 + m["f32_flops"] / (FP32_MFMA_PEAK_TFS * 1e12)) * 1e6
        res["mfma_counters"] = dict(m, issued_mix_at_peak_us=round(at_peak_us, 1),
                                    issued_mix_utilisation=round(at_peak_us / (ms * 1e3), 4))
    del pool, ws, out, args
    torch.cuda.empty_cache()
    return res


def m2_state_bytes(sdt, H, d, n):
    return H * d * n * SB[sdt]


def m2_decode_bytes(B, sdt, H, G, d, n, ib=2, ob=2):
    """Algorithmic bytes of one Mamba2 decode step: state read + write, x, B, C, dt, outputs."""
    return (2 * B * m2_state_bytes(sdt, H, d, n) + B * (H * d + 2 * G * n + H) * ib + 3 * H * 4 + B * 4
            + B * H * d * ob)


def m2_replay_step_bytes(B, sdt, n_before, T, L, H, G, d, n, ib=2, ob=2):
    """Algorithmic bytes of one Mamba2 replay step of T tokens with n_before committed entries."""
    fold = n_before + T > L
    state = B * m2_state_bytes(sdt, H, d, n) * (2 if fold else 1)
    entry = (H * d + G * n) * ib + 2 * H * 4  # x per head, B per group, g and dt' per head
    live = 0 if fold else n_before
    read_fold = n_before * entry if fold else 0
    return (state + B * (live * entry + read_fold) + B * T * entry
            + B * T * (H * d + 2 * G * n + H) * ib + 3 * H * 4 + 3 * B * 4 + B * T * H * d * ob)


def bench_mamba2(torch, gdn, gen, B, sdt, mode, T=1, L=16, cycles=2, steps=16, cid=5):
    """Mamba2 layer (gen.M2_LAYER): standard decode (mode "decode") or replay (mode "replay")."""
    import numpy as np
    dev = "cuda"
    lay = gen.M2_LAYER
    H, G, d, n = lay["H"], lay["G"], lay["d"], lay["n"]
    num_slots = 2 * B
    slot_map = gen.slot_permutation(cid, num_slots)[:B]
    pool = torch.zeros((num_slots, H, d, n), dtype={"f32": torch.float32, "bf16": torch.bfloat16,
                                                     "f16": torch.float16}[sdt], device=dev)
    for i in range(0, B, 32):
        sl = slot_map[i:i + 32]
        pool[torch.as_tensor(sl.astype(np.int64), device=dev)] = gen.to_torch(gen.pool_slots(cid, sl, H, d, n, sdt),
                                                                              dev)
    A_log, dt_bias, Dk = gen.m2_params(cid, H)
    Pm = [gen.to_torch(t, dev) for t in (A_log, dt_bias, Dk)]
    sm = torch.from_numpy(slot_map).to(dev)
    lead = (B,) if mode == "decode" else (B, T)
    ins = []
    for s in range(4):
        inp = gen.m2_inputs(cid, s, lead, H, G, d, n, "bf16")
        ins.append([gen.to_torch(inp[x], dev) for x in ("x", "Bm", "Cm", "dt")])
    out = torch.empty(lead + (H, d), dtype=torch.bfloat16, device=dev)
    if mode == "decode":
        def fn(i):
            x, Bm, Cm, dt = ins[i % 4]
            gdn.gdn_mamba2_decode_step(x, Bm, Cm, dt, *Pm, pool, sm, out=out)
        t = timed_launches(torch, fn, steps, 3)
        n_steps, nbytes = steps, steps * m2_decode_bytes(B, sdt, H, G, d, n)
        src = ["gdn_mamba2.hip", "gdn_device.h"]
    else:
        ring = gdn.new_m2_ring(num_slots, H, G, L, d, n, torch.bfloat16, dev)
        per_cycle = L // T if T > 1 else L

        def fn(i):
            x, Bm, Cm, dt = ins[i % 4]
            gdn.gdn_mamba2_replay_decode(x, Bm, Cm, dt, *Pm, pool, sm, ring, out=out)
        t = timed_launches(torch, fn, cycles * per_cycle, per_cycle)
        n_steps, nbytes, cnt = cycles * per_cycle, 0, 0
        for i in range((cycles + 1) * per_cycle):
            b_i = m2_replay_step_bytes(B, sdt, cnt, T, L, H, G, d, n)
            cnt = (0 if cnt + T > L else cnt) + T
            if i >= per_cycle:
                nbytes += b_i
        src = ["gdn_mamba2.hip", "gdn_device.h"]
        del ring
    ms = t["span_ms"] / n_steps
    res = {"B": B, "state": sdt, "mode": mode, "T": T if mode != "decode" else 1, "L": L if mode != "decode" else None,
           "layer": f"H={H} G={G} headdim={d} dstate={n}", "ms_per_step": round(ms, 5),
           "GB_per_s": round(nbytes / n_steps / (ms * 1e-3) / 1e9, 1),
           "tokens_per_s": round(B * (T if mode != "decode" else 1) / (ms * 1e-3), 1),
           "bytes_per_step_avg": nbytes // n_steps}
    res["roofline"] = roofline_bw(nbytes / n_steps, t["mean_launch_ms"], traffic_for(f"m2_{mode}_{sdt}_B{B}", src))
    del pool, ins, out
    torch.cuda.empty_cache()
    return res


def bench_copy_blocks(torch, gdn, reps=8, P=16, slots=64, jobs=32):
    """Prefix-caching state-block copy: `jobs` slot copies in each of P layer-state tensors of
    [slots, 32, 128, 128] fp32 (2 MiB slots)."""
    import numpy as np
    dev = "cuda"
    tensors = [torch.empty((slots, HV, D, D), dtype=torch.float32, device=dev).normal_() for _ in range(P)]
    perm = np.random.default_rng(48109).permutation(slots).astype(np.int32)
    src_d = torch.from_numpy(perm[:jobs].copy()).to(dev)
    dst_d = torch.from_numpy(perm[jobs:2 * jobs].copy()).to(dev)
    table = gdn.make_state_table(tensors, dev)
    t = timed_launches(torch, lambda i: gdn.gdn_copy_state_blocks(tensors, src_d, dst_d, table=table), reps, 2)
    slot_bytes = HV * D * D * 4
    nbytes = 2 * jobs * P * slot_bytes + P * 24 + 2 * jobs * 4
    ms = t["span_ms"] / reps
    res = {"P": P, "jobs": jobs, "slot_MiB": slot_bytes / 2 ** 20, "ms_per_call": round(ms, 4),
           "GB_per_s": round(nbytes / (ms * 1e-3) / 1e9, 1), "bytes_per_call": nbytes,
           "roofline": roofline_bw(nbytes, t["mean_launch_ms"], traffic_for("blockcopy", ["gdn_copy.hip", "gdn_device.h"]))}
    del tensors
    torch.cuda.empty_cache()
    return res


def bench_copy(torch, nbytes=1 << 30, reps=4):
    """A plain device-to-device copy of known size (the counter calibration for HBM traffic)."""
    src = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
    dst = torch.empty_like(src)
    t = timed_launches(torch, lambda i: dst.copy_(src), reps, 2)
    res = {"bytes_read_per_launch": nbytes, "bytes_written_per_launch": nbytes,
           "GB_per_s": round(2 * nbytes / (t["mean_launch_ms"] * 1e-3) / 1e9, 1)}
    del src, dst
    torch.cuda.empty_cache()
    return res


# ------------------------------------------------------------------ CPU oracle baseline
# The plain oracle (float64 numpy, token by token) on the host cores, in four legs: the headline
# decode layer (fp32 state), the same layer with a bf16 state, the chunked-prefill workload and
# one 16-step replay cycle.  Each leg is a bounded sample of its workload, split over a pool of
# worker processes (one BLAS thread each).  Inputs are generated once in the parent; the pool is
# forked after that and before the GPU is first touched, so the workers share the inputs
# copy-on-write and never hold a GPU context.
CPU_MAX_WORKERS = 16           # the host share of one GPU on the benchmark boxes
_CPU = {}                      # leg inputs, inherited by the forked workers


def _cpu_worker_init():
    try:
        from threadpoolctl import threadpool_limits
        threadpool_limits(limits=1)
    except Exception:  # pragma: no cover - threadpoolctl is present in this image
        pass


def _cpu_task(task):
    """One share of a leg; returns the oracle's compute seconds."""
    import numpy as np
    import oracle as O
    kind, idx = task
    d = _CPU[kind]
    t0 = time.perf_counter()
    if kind.startswith("decode"):
        rows = d["shares"][idx]
        pool = d["states"][rows]
        local = np.arange(len(rows))
        for inp in d["inputs"]:
            pool, _ = O.decode_step(pool, local, *(inp[x][rows] for x in "qkvab"), d["A_log"], d["dt_bias"])
    elif kind == "prefill":
        n, heads = d["shares"][idx]
        lo, hi = int(d["cu"][n]), int(d["cu"][n + 1])
        inp = {x: d["inputs"][x][lo:hi] for x in "qkvab"}
        O.chunk_prefill(d["states"][n:n + 1], [0], [0, hi - lo], *(inp[x] for x in "qkvab"), d["A_log"],
                        d["dt_bias"], heads=heads)
    elif kind == "replay":
        rows = d["shares"][idx]
        ck = d["states"][rows]
        ring = O.new_ring(len(rows), HV, d["L"], D, D)
        local = np.arange(len(rows))
        for inp in d["inputs"]:
            ck, ring, _ = O.replay_decode(ck, ring, local, *(inp[x][rows] for x in "qkvab"), d["A_log"],
                                          d["dt_bias"])
    return time.perf_counter() - t0


def cpu_prepare(gen, cores):
    """Generate the inputs of the four legs (before the worker pool is forked)."""
    import numpy as np
    B, steps = 256, 8
    for kind, sdt, cid in (("decode_f32", "f32", 1), ("decode_bf16", "bf16", 2)):
        slot_map = gen.slot_permutation(cid, NUM_SLOTS)[:B]
        A_log, dt_bias = gen.head_params(cid, HV)
        _CPU[kind] = dict(states=gen.pool_slots(cid, slot_map, HV, D, D, sdt), A_log=A_log, dt_bias=dt_bias,
                          inputs=[gen.token_inputs(cid, s, (B,), HK, HV, D, D, "bf16") for s in range(steps)],
                          shares=np.array_split(np.arange(B), cores), B=B, steps=steps, sdt=sdt)
    lengths = gen.WORKLOADS["prefill"].extra["lengths"]
    cu = gen.seq_lengths_cu(lengths)
    slot_map = gen.slot_permutation(3, 16)[:len(lengths)]
    A_log, dt_bias = gen.head_params(3, HV)
    # sample: all 32 heads of the 1024- and 3000-token sequences (one share per (sequence, 4 heads))
    shares = [(n, list(range(h, h + 4))) for n in (0, 1) for h in range(0, HV, 4)]
    _CPU["prefill"] = dict(states=gen.pool_slots(3, slot_map, HV, D, D, "f32"), A_log=A_log, dt_bias=dt_bias,
                           inputs=gen.token_inputs(3, 0, (int(cu[-1]),), HK, HV, D, D, "bf16"), cu=cu,
                           shares=shares, head_tokens=sum(4 * lengths[n] for n, _ in shares), lengths=lengths)
    Br, L = 32, 16
    slot_map = gen.slot_permutation(4, NUM_SLOTS)[:Br]
    A_log, dt_bias = gen.head_params(4, HV)
    _CPU["replay"] = dict(states=gen.pool_slots(4, slot_map, HV, D, D, "f32"), A_log=A_log, dt_bias=dt_bias,
                          inputs=[gen.token_inputs(4, s, (Br, 1), HK, HV, D, D, "bf16") for s in range(L)],
                          shares=np.array_split(np.arange(Br), cores), B=Br, L=L)


def cpu_baseline(pool, cores):
    """Time the four legs on the worker pool; tokens/s and GB/s use the GPU rows' byte models."""
    legs = {}
    for kind in ("decode_f32", "decode_bf16", "prefill", "replay"):
        d = _CPU[kind]
        tasks = [(kind, i) for i in range(len(d["shares"]))]
        t0 = time.perf_counter()
        busy = sum(pool.map(_cpu_task, tasks, chunksize=1))
        wall = time.perf_counter() - t0
        if kind.startswith("decode"):
            tok = d["B"] * d["steps"] / wall
            legs[kind] = {"tokens_per_s": round(tok, 1), "GB_per_s": round(tok * decode_bytes(1, d["sdt"]) / 1e9, 4),
                          "sample": f"B={d['B']} rows x 32 value heads x {d['steps']} decode steps, "
                                    f"{d['sdt']} state", "wall_s": round(wall, 2), "busy_s": round(busy, 1)}
        elif kind == "prefill":
            tok = d["head_tokens"] / HV / wall  # whole-layer tokens (all 32 heads) per second
            per_tok = prefill_bytes(d["lengths"], "f32") / sum(d["lengths"])
            legs[kind] = {"tokens_per_s": round(tok, 1), "GB_per_s": round(tok * per_tok / 1e9, 4),
                          "sample": "every value head of the 1024- and 3000-token sequences of the 4-sequence "
                                    "workload, one call, fp32 state", "wall_s": round(wall, 2),
                          "busy_s": round(busy, 1)}
        else:
            L = d["L"]
            cyc = sum(replay_step_bytes(1, "f32", n, 1, L) for n in range(L))  # one row, one 16-step cycle
            tok = d["B"] * L / wall
            legs[kind] = {"tokens_per_s": round(tok, 1), "GB_per_s": round(tok * cyc / L / 1e9, 4),
                          "sample": f"B={d['B']} rows x 32 value heads, one 16-step fold cycle (T=1, L=16), "
                                    "fp32 checkpoint", "wall_s": round(wall, 2), "busy_s": round(busy, 1)}
    head = legs["decode_f32"]
    return {"value": head["GB_per_s"], "unit": "GB/s", "cores": cores, "kind": "oracle",
            "tokens_per_s": head["tokens_per_s"],
            "sample": f"plain oracle (float64 numpy, token by token) on {cores} worker processes, one BLAS thread "
                      f"each; value: {head['sample']} of the headline layer", "legs": legs}


# ------------------------------------------------------------------ main
def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=64)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--only", default=None, help="comma-separated rows only: decode_<dt>_B<n> | replay_<dt>_T<t>[_staggered] | replay_dual_<dt>_T<t> | "
                                                    "spec_<dt>_T<t> | mamba2_<decode|replay>_<dt>[_T<t>] | prefill_<dt> | blockcopy | copy")
    ap.add_argument("--no-rows", action="store_true", help="headline only")
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only: this library has no multi-GPU path (asked for --gpus {args.gpus}); "
              "the per-(sequence, head) units would shard across GPUs without any exchange",
              file=sys.stderr)
        sys.exit(2)

    import torch
    import gated_deltanet_state_gdn_amd as gdn
    from workloads import gen
    cpu_pool = None
    if not args.no_cpu and not args.only:
        # before any GPU call: the workers are forked from a process without a GPU context
        import multiprocessing as mp
        cores = min(len(os.sched_getaffinity(0)), CPU_MAX_WORKERS)
        log(f"cpu baseline: generating oracle inputs, {cores} workers")
        cpu_prepare(gen, cores)
        cpu_pool = mp.get_context("fork").Pool(cores, initializer=_cpu_worker_init)
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    gdn.lib()

    if args.only:
        for row in args.only.split(","):
            kind, *rest = row.split("_")
            if kind == "decode":
                r = bench_decode(torch, gdn, gen, int(rest[1][1:]) if len(rest) > 1 else 256, rest[0], args.steps,
                                 args.warmup)
            elif kind == "replay" and rest[0] == "dual":
                r = bench_replay(torch, gdn, gen, 512, "f32", int(rest[2][1:]) if len(rest) > 2 else 1, 2,
                                 copy_dt=rest[1])
            elif kind == "replay":
                r = bench_replay(torch, gdn, gen, 512, rest[0], int(rest[1][1:]) if len(rest) > 1 else 1, 2,
                                 staggered=rest[-1] == "staggered")
            elif kind == "spec":
                r = bench_spec(torch, gdn, gen, 512, rest[0], int(rest[1][1:]) if len(rest) > 1 else 5,
                               max(args.steps // 4, 4))
            elif kind == "prefill":
                r = bench_prefill(torch, gdn, gen, rest[0], max(args.steps // 8, 2))
            elif kind == "copy":
                r = bench_copy(torch)
            elif kind == "mamba2":
                r = bench_mamba2(torch, gdn, gen, 512, rest[1], rest[0], T=int(rest[2][1:]) if len(rest) > 2 else 1)
            elif kind == "blockcopy":
                r = bench_copy_blocks(torch, gdn)
            else:
                raise SystemExit(f"unknown row {row}")
            print(json.dumps({"row": row, **r}), flush=True)
        return

    log(f"headline: decode B=256 fp32 state, {args.warmup} warmup + {args.steps} timed steps")
    head = bench_decode(torch, gdn, gen, 256, "f32", args.steps, args.warmup)
    log(f"  {head['ms_per_step'] * 1e3:.1f} us/step, {head['GB_per_s']} GB/s")
    rows = {}
    if not args.no_rows:
        for B, dt in ((512, "f32"), (256, "bf16"), (512, "bf16"), (512, "f16"), (64, "bf16"), (1, "bf16")):
            log(f"row: decode B={B} {dt} state")
            rows[f"decode_{dt}_B{B}"] = bench_decode(torch, gdn, gen, B, dt, args.steps, args.warmup)
        for dt, T, cyc in (("f32", 1, 4), ("bf16", 1, 4), ("f32", 5, 8)):
            log(f"row: replay B=512 {dt} checkpoint T={T}")
            rows[f"replay_{dt}_B512_T{T}"] = bench_replay(torch, gdn, gen, 512, dt, T, cyc)
        for dt in ("f32", "bf16"):
            log(f"row: replay B=512 {dt} checkpoint T=1, staggered rings")
            rows[f"replay_{dt}_B512_T1_staggered"] = bench_replay(torch, gdn, gen, 512, dt, 1, 4, staggered=True)
        log("row: replay B=512 fp32 master + bf16 read copy T=1")
        rows["replay_dual_bf16_B512_T1"] = bench_replay(torch, gdn, gen, 512, "f32", 1, 4, copy_dt="bf16")
        for dt in ("f32", "bf16"):
            log(f"row: speculative window B=512 T=5 {dt} state, one state per position")
            rows[f"spec_{dt}_B512_T5"] = bench_spec(torch, gdn, gen, 512, dt, 5, 16)
        for mode in ("decode", "replay"):
            log(f"row: Mamba2 {mode} B=512 fp32 state")
            rows[f"mamba2_{mode}_f32_B512"] = bench_mamba2(torch, gdn, gen, 512, "f32", mode)
        log("row: state-block copy, 32 jobs x 16 tensors of 2 MiB slots")
        rows["state_block_copy"] = bench_copy_blocks(torch, gdn)
        for dt in ("f32", "bf16"):
            log(f"row: chunked prefill {dt} state")
            rows[f"prefill_{dt}"] = bench_prefill(torch, gdn, gen, dt, 8)
    cpu = None
    if cpu_pool is not None:
        log("cpu baseline: oracle legs")
        cpu = cpu_baseline(cpu_pool, cores)
        cpu_pool.close()
        cpu_pool.join()

    ms = head["ms_per_step"]
    line = {
        "metric": METRIC, "value": head["GB_per_s"], "unit": "GB/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": ms, "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "f32", "data": "synthetic (seeded workloads/gen.py)",
        "tokens_per_s": head["tokens_per_s"], "hbm_peak_frac": round(head["GB_per_s"] / HBM_PEAK_GBS, 4),
        "config": {"workload": "gdn_decode_step: B=256 sequences, 16 key / 32 value heads, dk=dv=128, fp32 state "
                               "in a 1024-slot pool, bf16 q/k/v/a/b, bf16 out, one token per step",
                   "B": 256, "Hk": HK, "Hv": HV, "dk": D, "dv": D, "state_dtype": "f32",
                   "bytes_per_step": head["bytes_per_step"]},
        "roofline": dict(head["roofline"], kernel="gdn_decode_persist_kernel<f32,128>",
                         mean_launch_us=head["mean_launch_us"]),
        "cpu_baseline": cpu,
        "rows": rows,
    }
    print(json.dumps(line))


if __name__ == "__main__":
    main()
