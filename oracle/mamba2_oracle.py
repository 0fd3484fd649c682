"""CPU oracle for the Mamba2 selective-state decode and its ReplaySSM form.

TEST INFRASTRUCTURE.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import this module.  The library
under test never imports it, and it imports nothing from the library.

Plain definition, token by token, float64 numpy; nothing blocked or reordered.

Sources:
  [ReplaySSM] AREX feed article on ReplaySSM.  "Bottleneck": decode reads and
              writes the whole (nheads, d, n) state every step.  "Cache inputs,
              not state": a checkpoint S0 plus a ring of the latest
              state-building inputs, folded into S0 every L steps; other steps
              compute outputs from S0 and the ring; the read-out vector (C for
              Mamba2) is taken from the current activations and never cached;
              rollback of rejected drafts moves the ring pointer.  "Numbers":
              the 1.55x / 1.67x per-step figures were measured on Mamba2 with
              FP32 state and a 16-entry ring.
  [Mamba2]    The selective state-space update as published by Dao and Gu
              ("Transformers are SSMs", 2024): per head, with step size
              dt' = softplus(dt + dt_bias) and scalar A = -exp(A_log),
              h <- exp(dt' A) h + dt' x B^T, y = h C + D x, where x is the
              head's input (headdim d), B and C (dstate n) are shared by the
              heads of a group and D is a per-head skip.

Readings taken where the pages are silent:
  * the state of a head is [d, n] (n fastest), as the pages' (nheads, d, n);
  * the log-decay is g = -exp(A_log) softplus(dt + dt_bias), the same gate
    form as the GDN path, and the write strength is dt' itself;
  * the optional output gate z of some Mamba2 kernels is left to the caller;
  * head h reads group h // (H / G) (contiguous groups);
  * ring pointers are per slot (every head of a slot advances together); x,
    g and dt' are stored per head, B per group;
  * the state is rounded to its storage dtype only at write points (every
    decode step; each replay fold).
"""
from __future__ import annotations

import math
from dataclasses import dataclass, replace

import numpy as np

from .gdn_oracle import _slot_ok, dtype_of, softplus, to_storage, widen

__all__ = [
    "m2_gates", "m2_token", "mamba2_decode_step", "M2Ring", "new_m2_ring", "mamba2_replay_decode",
    "mamba2_replay_flush", "mamba2_replay_rollback",
]


def m2_gates(dt, A_log, dt_bias):
    """Per (token, head): log-decay g = -exp(A_log) dt', write strength dt' = softplus(dt + dt_bias)."""
    dtp = softplus(widen(dt) + widen(dt_bias))
    return -np.exp(widen(A_log)) * dtp, dtp


def m2_token(S, x, Bv, Cv, g, dtp, Dh):
    """One token of one head: S <- exp(g) S + dt' x B^T; y = S C + D x.  S is [d, n]."""
    S = math.exp(float(g)) * S + float(dtp) * np.outer(x, Bv)
    return S, S @ Cv + float(Dh) * x


def mamba2_decode_step(pool, slot_map, x, Bm, Cm, dt, A_log, dt_bias, Dskip, heads=None):
    """One token per sequence.  pool [slots, H, d, n]; x [B, H, d]; Bm, Cm [B, G, n]; dt [B, H];
    A_log, dt_bias, Dskip [H].  Each touched state is written back rounded once.
    Returns (new pool, y [B, H, d])."""
    pool = np.array(pool, copy=True)
    sdt = dtype_of(pool)
    num_slots, H, d, n = pool.shape
    B, G = x.shape[0], Bm.shape[1]
    xf, Bf, Cf = widen(x), widen(Bm), widen(Cm)
    g, dtp = m2_gates(dt, A_log, dt_bias)
    Dk = widen(Dskip)
    y = np.zeros((B, H, d))
    for bi in range(B):
        slot = int(slot_map[bi])
        if not _slot_ok(slot, num_slots):
            continue
        for h in (range(H) if heads is None else heads):
            gr = h // (H // G)
            S, y[bi, h] = m2_token(widen(pool[slot, h]), xf[bi, h], Bf[bi, gr], Cf[bi, gr], g[bi, h], dtp[bi, h],
                                   Dk[h])
            pool[slot, h] = to_storage(S, sdt)
    return pool, y


@dataclass
class M2Ring:
    """Mamba2 ReplaySSM ring: x [slots, H, L, d] and Bm [slots, G, L, n] in the input dtype;
    g, dtp [slots, H, L] float32; start, count [slots] int32.  Live entry i sits at ring index
    (start + i) mod L.  C is never stored."""
    x: np.ndarray
    Bm: np.ndarray
    g: np.ndarray
    dtp: np.ndarray
    start: np.ndarray
    count: np.ndarray

    @property
    def L(self):
        return self.g.shape[2]

    def copy(self):
        return replace(self, **{f: np.array(getattr(self, f), copy=True)
                                for f in ("x", "Bm", "g", "dtp", "start", "count")})


def new_m2_ring(num_slots, H, G, L, d, n, in_dtype="bf16"):
    kd = {"f32": np.float32, "bf16": np.uint16, "f16": np.float16}[in_dtype]
    return M2Ring(x=np.zeros((num_slots, H, L, d), kd), Bm=np.zeros((num_slots, G, L, n), kd),
                  g=np.zeros((num_slots, H, L), np.float32), dtp=np.zeros((num_slots, H, L), np.float32),
                  start=np.zeros(num_slots, np.int32), count=np.zeros(num_slots, np.int32))


def _m2_replay_state(S0, ring, slot, h, gr, n_live):
    """S0 of head h advanced over the first n_live live entries of the slot."""
    S = np.array(S0, copy=True)
    L, st = ring.L, int(ring.start[slot])
    for i in range(n_live):
        j = (st + i) % L
        S = math.exp(float(ring.g[slot, h, j])) * S + float(ring.dtp[slot, h, j]) * np.outer(
            widen(ring.x[slot, h, j]), widen(ring.Bm[slot, gr, j]))
    return S


def _m2_fold(ckpt, ring, slot, sdt):
    """Fold every committed entry of the slot into each head's checkpoint (one rounding) and empty the ring."""
    H, G = ckpt.shape[1], ring.Bm.shape[1]
    cnt = int(ring.count[slot])
    for h in range(H):
        S = _m2_replay_state(widen(ckpt[slot, h]), ring, slot, h, h // (H // G), cnt)
        ckpt[slot, h] = to_storage(S, sdt)
    ring.start[slot] = (int(ring.start[slot]) + cnt) % ring.L
    ring.count[slot] = 0


def mamba2_replay_decode(ckpt, ring, slot_map, x, Bm, Cm, dt, A_log, dt_bias, Dskip, heads=None):
    """One replay step of T tokens per sequence.  x [B, T, H, d]; Bm, Cm [B, T, G, n]; dt [B, T, H].

    Per slot: if count + T > L, first fold all committed entries into the checkpoint; then
    append the T new entries at ring indices (start + count + t) mod L; then window position t
    outputs y = S_t C_t + D x_t, S_t the checkpoint replayed over the first count + t + 1 live
    entries (no state write).  Returns (ckpt, ring, y [B, T, H, d])."""
    ckpt = np.array(ckpt, copy=True)
    ring = ring.copy()
    sdt = dtype_of(ckpt)
    num_slots, H, d, n = ckpt.shape
    B, T, G = x.shape[0], x.shape[1], Bm.shape[2]
    L = ring.L
    if not 1 <= T <= L:
        raise ValueError("window longer than the ring")
    Cf, xf = widen(Cm), widen(x)
    g, dtp = m2_gates(dt, A_log, dt_bias)
    Dk = widen(Dskip)
    y = np.zeros((B, T, H, d))
    for bi in range(B):
        slot = int(slot_map[bi])
        if not _slot_ok(slot, num_slots):
            continue
        if int(ring.count[slot]) + T > L:
            _m2_fold(ckpt, ring, slot, sdt)
        st, cnt = int(ring.start[slot]), int(ring.count[slot])
        for t in range(T):
            j = (st + cnt + t) % L
            ring.x[slot, :, j] = x[bi, t]
            ring.Bm[slot, :, j] = Bm[bi, t]
            ring.g[slot, :, j] = g[bi, t].astype(np.float32)
            ring.dtp[slot, :, j] = dtp[bi, t].astype(np.float32)
        ring.count[slot] = cnt + T
        for h in (range(H) if heads is None else heads):
            gr = h // (H // G)
            S0 = widen(ckpt[slot, h])
            for t in range(T):
                St = _m2_replay_state(S0, ring, slot, h, gr, cnt + t + 1)
                y[bi, t, h] = St @ Cf[bi, t, gr] + Dk[h] * xf[bi, t, h]
    return ckpt, ring, y


def mamba2_replay_flush(ckpt, ring, slot_map):
    """Fold every committed entry of the mapped slots into their checkpoints."""
    ckpt = np.array(ckpt, copy=True)
    ring = ring.copy()
    sdt = dtype_of(ckpt)
    for slot in slot_map:
        if _slot_ok(slot, ckpt.shape[0]):
            _m2_fold(ckpt, ring, int(slot), sdt)
    return ckpt, ring


def mamba2_replay_rollback(ring, slot_map, num_rejected):
    """Drop the last r live entries of each mapped slot: count <- max(count - r, 0)."""
    ring = ring.copy()
    for bi, slot in enumerate(slot_map):
        if _slot_ok(slot, ring.count.shape[0]):
            ring.count[slot] = max(int(ring.count[slot]) - int(num_rejected[bi]), 0)
    return ring
