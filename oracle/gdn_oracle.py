"""CPU oracle for the Gated DeltaNet (GDN) gated-delta-rule recurrent-state update.

TEST INFRASTRUCTURE.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import this module.  The library
under test never imports it, and it imports nothing from the library.

It is the plain definition, written token by token in float64 with numpy;
nothing is blocked, chunked, fused or reordered.  The chunked prefill and the
replay decode of the library are reformulations of this same recurrence, so
this one loop is the reference for all three entry points.

Sources (cited by page title and section):
  [PR52191]   vLLM PR #52191 summary page (prhub.com.cn): "GDN state kept in
              FP16/BF16 on CPU AMX".  Implementation section, item 3 (the
              fused sigmoid-gating delta-rule decode kernel, the chunked
              inter-chunk kernel and the spec kernel, templated on the state
              type), item 4 (all math in FP32, only slot reads and writes use
              the state type, so every write-back rounds once; chunk states
              are scaled by exp(g_last)), item 5 (the reference recurrence
              simulates the state-dtype rounding once per write interval).
  [ReplaySSM] AREX feed article on ReplaySSM.  "Bottleneck" section (decode
              reads and writes the whole (nheads, d, n) state each step);
              "cache inputs, not state" section (a checkpoint S0 plus a ring
              of the latest state-building inputs, folded into S0 every L
              steps; other steps compute outputs from S0 and the ring without
              materialising the state; the read-out vector q is not cached).
  [PR48109]   vLLM PR #48109 summary page (prhub.com.cn), the XPU state
              pointer fix: its implementation section (the state-block copy
              kernel behind --mamba-cache-mode align, fed by tables of state
              base addresses) and risk section (the addresses need all 64
              bits).
  [GDN]       The gated delta rule as published by Yang, Kautz and
              Hatamizadeh ("Gated Delta Networks: Improving Mamba2 with Delta
              Rule", 2024): S_t = a_t (I - b_t k_t k_t^T) S_{t-1} + b_t k_t v_t^T
              with the read-out o_t = S_t^T q_t, in this library's dk x dv
              orientation of S.

Readings taken where the pages are silent:
  * gates: g = -exp(A_log) * softplus(a + dt_bias) (a log-decay: the pages
    scale states by exp(g)), beta = sigmoid(b) (the kernel is named after a
    fused sigmoid gating); softplus is the exact max(x,0)+log1p(exp(-|x|));
  * order inside one token: decay, then k-projection of the decayed state,
    then the rank-1 correction; the output reads the updated, unrounded
    state and is scaled by dk**-0.5;
  * value head h reads key head h // (Hv / Hk) (contiguous GQA groups);
  * the state is rounded to its storage dtype (round to nearest, ties to
    even) only at write points: every decode step, the end of each prefill
    call, and each replay fold;
  * a slot index outside [0, num_slots) marks a padded row: its outputs are
    zero and no state is touched.

Host representation of tensors (shared with ``workloads``): float32 ->
np.float32, float16 -> np.float16, bfloat16 -> np.uint16 raw bits.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, replace

import numpy as np

__all__ = [
    "round_to_format", "to_storage", "widen", "dtype_of", "softplus", "sigmoid", "gates",
    "decay_update", "readout", "gdn_token", "ref_gdn", "decode_step", "chunk_prefill",
    "Ring", "new_ring", "replay_decode", "replay_flush", "replay_rollback", "spec_decode",
    "copy_state_blocks", "replay_decode_dual", "replay_flush_dual",
]

# ---------------------------------------------------------------------------
# storage formats ([PR52191] item 4: FP32 math, narrow storage, one rounding
# per write-back)
# ---------------------------------------------------------------------------

# (stored fraction bits, exponent of the smallest normal, largest finite value)
_FORMATS = {
    "f32": (23, -126, float(np.finfo(np.float32).max)),
    "bf16": (7, -126, float.fromhex("0x1.fep127")),
    "f16": (10, -14, 65504.0),
}


def round_to_format(x, fmt: str) -> np.ndarray:
    """Round float64 values to the nearest value of ``fmt`` (ties to even).

    The exponent of the leading bit is clamped at the smallest normal
    exponent, which gives the fixed subnormal quantum below it; magnitudes
    that round above the largest finite value become infinities.  Returns
    float64 holding exactly representable values.
    """
    frac_bits, min_exp, max_finite = _FORMATS[fmt]
    x = np.asarray(x, dtype=np.float64)
    out = np.array(x, dtype=np.float64, copy=True)
    sel = np.isfinite(x) & (x != 0.0)
    xs = x[sel]
    _, e = np.frexp(xs)                       # xs = m * 2**e with 0.5 <= |m| < 1
    lead = np.maximum(e - 1, min_exp)         # exponent of the leading significant bit
    quantum = np.ldexp(1.0, lead - frac_bits)
    r = np.rint(xs / quantum) * quantum       # np.rint rounds half to even
    over = np.abs(r) > max_finite
    r[over] = np.copysign(np.inf, xs[over])
    out[sel] = r
    return out


def to_storage(x, dtype: str) -> np.ndarray:
    """float64 -> host representation of ``dtype`` (rounded once, RNE)."""
    r = round_to_format(x, dtype)
    if dtype == "f32":
        return r.astype(np.float32)
    if dtype == "f16":
        return r.astype(np.float16)
    if dtype == "bf16":
        return (r.astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)
    raise ValueError(dtype)


def dtype_of(arr: np.ndarray) -> str:
    if arr.dtype == np.float32:
        return "f32"
    if arr.dtype == np.uint16:
        return "bf16"
    if arr.dtype == np.float16:
        return "f16"
    if arr.dtype == np.float64:
        return "f64"
    raise TypeError(f"not a state/input tensor dtype: {arr.dtype}")


def widen(arr) -> np.ndarray:
    """Host representation -> float64 (exact)."""
    arr = np.asarray(arr)
    if arr.dtype == np.uint16:
        return (arr.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    return arr.astype(np.float64)


# ---------------------------------------------------------------------------
# gates ([PR52191] item 3: fused sigmoid gating; item 4: exp(g) decay)
# ---------------------------------------------------------------------------

def softplus(x):
    x = np.asarray(x, np.float64)
    with np.errstate(over="ignore"):
        return np.maximum(x, 0.0) + np.log1p(np.exp(-np.abs(x)))


def sigmoid(x):
    x = np.asarray(x, np.float64)
    with np.errstate(over="ignore"):
        return 1.0 / (1.0 + np.exp(-x))


def gates(a, b, A_log, dt_bias):
    """Per (token, value head): log-decay g = -exp(A_log) softplus(a + dt_bias), beta = sigmoid(b)."""
    a = widen(a)
    b = widen(b)
    A_log = widen(A_log)
    dt_bias = widen(dt_bias)
    g = -np.exp(A_log) * softplus(a + dt_bias)
    beta = sigmoid(b)
    return g, beta


# ---------------------------------------------------------------------------
# one token of the recurrence ([GDN]; [PR52191] item 3)
# ---------------------------------------------------------------------------

def decay_update(S, k, v, g, beta):
    """S <- exp(g) S; then S <- S + beta k (v - S^T k)^T.  S is dk x dv."""
    S = math.exp(float(g)) * S
    kv = S.T @ k
    return S + float(beta) * np.outer(k, v - kv)


def readout(S, q, scale):
    """o = scale * S^T q."""
    return float(scale) * (S.T @ q)


def gdn_token(S, q, k, v, g, beta, scale):
    S = decay_update(S, k, v, g, beta)
    return S, readout(S, q, scale)


def ref_gdn(S0, q, k, v, g, beta, scale, state_dtype="f32", write_points=()):
    """Token loop for one (sequence, value head).

    q, k: [T, dk]; v: [T, dv]; g, beta: [T].  ``write_points`` holds token
    indices after which the state is rounded to ``state_dtype`` and re-read
    ([PR52191] item 5: the reference simulates the write-back rounding).
    Returns (o [T, dv], S after the last token, unrounded).
    """
    S = np.array(S0, dtype=np.float64, copy=True)
    T = len(g)
    o = np.zeros((T, S.shape[1]))
    wp = set(int(t) for t in write_points)
    for t in range(T):
        S, o[t] = gdn_token(S, q[t], k[t], v[t], g[t], beta[t], scale)
        if t in wp:
            S = widen(to_storage(S, state_dtype))
    return o, S


def _slot_ok(slot, num_slots):
    return 0 <= int(slot) < num_slots


def _scale(dk, scale):
    return dk ** -0.5 if scale is None or scale <= 0 else float(scale)


# ---------------------------------------------------------------------------
# decode: one token per sequence, state read from and written to its slot
# ---------------------------------------------------------------------------

def decode_step(pool, slot_map, q, k, v, a, b, A_log, dt_bias, scale=None, heads=None):
    """One decode step for B sequences.

    pool [num_slots, Hv, dk, dv] (storage dtype); slot_map int [B];
    q, k [B, Hk, dk]; v [B, Hv, dv]; a, b [B, Hv]; A_log, dt_bias [Hv].
    Returns (new pool, o [B, Hv, dv] float64).  Every touched slot is rounded
    once (the step's write-back); slots not in the map are left untouched.
    """
    pool = np.array(pool, copy=True)
    sdt = dtype_of(pool)
    num_slots, Hv, dk, dv = pool.shape
    B = len(slot_map)
    Hk = q.shape[1]
    ratio = Hv // Hk
    s = _scale(dk, scale)
    qf, kf, vf = widen(q), widen(k), widen(v)
    g, beta = gates(a, b, A_log, dt_bias)
    o = np.zeros((B, Hv, dv))
    for bi in range(B):
        slot = int(slot_map[bi])
        if not _slot_ok(slot, num_slots):
            continue
        for h in (range(Hv) if heads is None else heads):
            hk = h // ratio
            S, o[bi, h] = gdn_token(widen(pool[slot, h]), qf[bi, hk], kf[bi, hk], vf[bi, h],
                                    g[bi, h], beta[bi, h], s)
            pool[slot, h] = to_storage(S, sdt)
    return pool, o


# ---------------------------------------------------------------------------
# prefill: packed variable-length sequences, state carried across calls
# ---------------------------------------------------------------------------

def chunk_prefill(pool, slot_map, cu_seqlens, q, k, v, a, b, A_log, dt_bias, scale=None,
                  write_interval=None, heads=None, seqs=None):
    """Prefill of N packed sequences (the token-by-token definition).

    cu_seqlens int [N+1]; q, k [T_total, Hk, dk]; v [T_total, Hv, dv];
    a, b [T_total, Hv].  Sequence n starts from pool[slot_map[n]] and its
    final state is written back there, rounded once at the end of the call
    (the default), or also every ``write_interval`` tokens from the call's
    start (the per-chunk write-back of [PR52191] item 4).  A zero-length
    sequence leaves its slot untouched.  Returns (new pool, o [T_total, Hv, dv]).
    """
    pool = np.array(pool, copy=True)
    sdt = dtype_of(pool)
    num_slots, Hv, dk, dv = pool.shape
    Hk = q.shape[1]
    ratio = Hv // Hk
    s = _scale(dk, scale)
    cu = [int(x) for x in cu_seqlens]
    N = len(cu) - 1
    qf, kf, vf = widen(q), widen(k), widen(v)
    g, beta = gates(a, b, A_log, dt_bias)
    o = np.zeros((qf.shape[0], Hv, dv))
    for n in (range(N) if seqs is None else seqs):
        lo, hi = cu[n], cu[n + 1]
        slot = int(slot_map[n])
        if hi <= lo or not _slot_ok(slot, num_slots):
            continue
        wp = []
        if write_interval:
            wp = [lo + j - 1 for j in range(write_interval, hi - lo, write_interval)]
        for h in (range(Hv) if heads is None else heads):
            hk = h // ratio
            S = widen(pool[slot, h])
            wpl = set(wp)
            for t in range(lo, hi):
                S, o[t, h] = gdn_token(S, qf[t, hk], kf[t, hk], vf[t, h], g[t, h], beta[t, h], s)
                if t in wpl:
                    S = widen(to_storage(S, sdt))
            pool[slot, h] = to_storage(S, sdt)
    return pool, o


# ---------------------------------------------------------------------------
# ReplaySSM-style decode ([ReplaySSM] "cache inputs, not state")
# ---------------------------------------------------------------------------

@dataclass
class Ring:
    """Per (slot, value head) ring of the last <= L state-building inputs.

    k [num_slots, Hv, L, dk] and v [num_slots, Hv, L, dv] are copies of the
    inputs in the input dtype; g, beta [num_slots, Hv, L] float32; start,
    count [num_slots, Hv] int32.  Live entry i (0 <= i < count) sits at ring
    index (start + i) mod L.  q is never cached.
    """
    k: np.ndarray
    v: np.ndarray
    g: np.ndarray
    beta: np.ndarray
    start: np.ndarray
    count: np.ndarray

    @property
    def L(self):
        return self.g.shape[2]

    def copy(self):
        return replace(self, **{f: np.array(getattr(self, f), copy=True)
                                for f in ("k", "v", "g", "beta", "start", "count")})


def new_ring(num_slots, Hv, L, dk, dv, in_dtype="bf16"):
    kd = {"f32": np.float32, "bf16": np.uint16, "f16": np.float16}[in_dtype]
    return Ring(k=np.zeros((num_slots, Hv, L, dk), kd), v=np.zeros((num_slots, Hv, L, dv), kd),
                g=np.zeros((num_slots, Hv, L), np.float32), beta=np.zeros((num_slots, Hv, L), np.float32),
                start=np.zeros((num_slots, Hv), np.int32), count=np.zeros((num_slots, Hv), np.int32))


def _replay_state(S0, ring, slot, h, n):
    """Forward replay: S0 advanced over the first n live entries of (slot, h)."""
    S = np.array(S0, copy=True)
    L = ring.L
    st = int(ring.start[slot, h])
    for i in range(n):
        j = (st + i) % L
        S = decay_update(S, widen(ring.k[slot, h, j]), widen(ring.v[slot, h, j]),
                         float(ring.g[slot, h, j]), float(ring.beta[slot, h, j]))
    return S


def _fold(ckpt, ring, slot, h, sdt):
    """Fold every committed entry into the checkpoint (one rounding) and empty the ring."""
    n = int(ring.count[slot, h])
    S = _replay_state(widen(ckpt[slot, h]), ring, slot, h, n)
    ckpt[slot, h] = to_storage(S, sdt)
    ring.start[slot, h] = (int(ring.start[slot, h]) + n) % ring.L
    ring.count[slot, h] = 0


def replay_decode(ckpt, ring, slot_map, q, k, v, a, b, A_log, dt_bias, scale=None, heads=None):
    """One replay step of T tokens per sequence (T = 1 standard, T > 1 a verify window).

    q, k [B, T, Hk, dk]; v [B, T, Hv, dv]; a, b [B, T, Hv].  For each
    (sequence, value head): if count + T > L, first fold all committed
    entries into the checkpoint; then append the T new entries at ring
    indices (start + count + t) mod L; then the output of window position t
    reads the state reached by replaying the checkpoint over the first
    count + t + 1 live entries (no state write).  Returns (ckpt, ring, o [B, T, Hv, dv]).
    """
    ckpt = np.array(ckpt, copy=True)
    ring = ring.copy()
    sdt = dtype_of(ckpt)
    num_slots, Hv, dk, dv = ckpt.shape
    B, T = q.shape[0], q.shape[1]
    Hk = q.shape[2]
    ratio = Hv // Hk
    L = ring.L
    if not 1 <= T <= L:
        raise ValueError("window longer than the ring")
    s = _scale(dk, scale)
    qf = widen(q)
    g, beta = gates(a, b, A_log, dt_bias)
    o = np.zeros((B, T, Hv, dv))
    for bi in range(B):
        slot = int(slot_map[bi])
        if not _slot_ok(slot, num_slots):
            continue
        for h in (range(Hv) if heads is None else heads):
            hk = h // ratio
            if int(ring.count[slot, h]) + T > L:
                _fold(ckpt, ring, slot, h, sdt)
            st, cnt = int(ring.start[slot, h]), int(ring.count[slot, h])
            for t in range(T):
                j = (st + cnt + t) % L
                ring.k[slot, h, j] = k[bi, t, hk]
                ring.v[slot, h, j] = v[bi, t, h]
                ring.g[slot, h, j] = np.float32(g[bi, t, h])
                ring.beta[slot, h, j] = np.float32(beta[bi, t, h])
            ring.count[slot, h] = cnt + T
            S0 = widen(ckpt[slot, h])
            for t in range(T):
                St = _replay_state(S0, ring, slot, h, cnt + t + 1)
                o[bi, t, h] = readout(St, qf[bi, t, hk], s)
    return ckpt, ring, o


def replay_flush(ckpt, ring, slot_map):
    """Fold every committed entry of the mapped slots into their checkpoints."""
    ckpt = np.array(ckpt, copy=True)
    ring = ring.copy()
    sdt = dtype_of(ckpt)
    num_slots, Hv = ckpt.shape[:2]
    for slot in slot_map:
        if _slot_ok(slot, num_slots):
            for h in range(Hv):
                _fold(ckpt, ring, int(slot), h, sdt)
    return ckpt, ring


def _refresh_copy(master, copy, slot, h):
    """The read copy holds the master rounded once to the copy's format."""
    copy[slot, h] = to_storage(widen(master[slot, h]), dtype_of(copy))


def replay_decode_dual(master, copy, ring, slot_map, q, k, v, a, b, A_log, dt_bias, scale=None, heads=None):
    """Replay step on a dual-precision checkpoint ([ReplaySSM] "cache inputs, not state", the
    closing remarks on precision: recursion on a high-precision checkpoint, reads from a
    low-precision copy).

    master: f32 checkpoint pool; copy: bf16/f16 pool of the same shape.  As replay_decode, except
    that a fold reads and writes master and then refreshes copy from it, and the window outputs
    replay from copy.  Returns (master, copy, ring, o).
    """
    master = np.array(master, copy=True)
    copy = np.array(copy, copy=True)
    if dtype_of(master) != "f32":
        raise ValueError("the master checkpoint is f32")
    ring = ring.copy()
    num_slots, Hv, dk, dv = master.shape
    B, T, Hk = q.shape[0], q.shape[1], q.shape[2]
    ratio = Hv // Hk
    L = ring.L
    if not 1 <= T <= L:
        raise ValueError("window longer than the ring")
    s = _scale(dk, scale)
    qf = widen(q)
    g, beta = gates(a, b, A_log, dt_bias)
    o = np.zeros((B, T, Hv, dv))
    for bi in range(B):
        slot = int(slot_map[bi])
        if not _slot_ok(slot, num_slots):
            continue
        for h in (range(Hv) if heads is None else heads):
            hk = h // ratio
            if int(ring.count[slot, h]) + T > L:
                _fold(master, ring, slot, h, "f32")
                _refresh_copy(master, copy, slot, h)
            st, cnt = int(ring.start[slot, h]), int(ring.count[slot, h])
            for t in range(T):
                j = (st + cnt + t) % L
                ring.k[slot, h, j] = k[bi, t, hk]
                ring.v[slot, h, j] = v[bi, t, h]
                ring.g[slot, h, j] = np.float32(g[bi, t, h])
                ring.beta[slot, h, j] = np.float32(beta[bi, t, h])
            ring.count[slot, h] = cnt + T
            S0 = widen(copy[slot, h])
            for t in range(T):
                St = _replay_state(S0, ring, slot, h, cnt + t + 1)
                o[bi, t, h] = readout(St, qf[bi, t, hk], s)
    return master, copy, ring, o


def replay_flush_dual(master, copy, ring, slot_map):
    """Fold every committed entry of the mapped slots into master and refresh copy from master
    (also for empty rings, which is how a copy is first filled)."""
    master = np.array(master, copy=True)
    copy = np.array(copy, copy=True)
    ring = ring.copy()
    num_slots, Hv = master.shape[:2]
    for slot in slot_map:
        if _slot_ok(slot, num_slots):
            for h in range(Hv):
                _fold(master, ring, int(slot), h, "f32")
                _refresh_copy(master, copy, int(slot), h)
    return master, copy, ring


def replay_rollback(ring, slot_map, num_rejected):
    """Drop the last r live entries of each mapped slot: count <- max(count - r, 0)."""
    ring = ring.copy()
    num_slots = ring.count.shape[0]
    for bi, slot in enumerate(slot_map):
        if _slot_ok(slot, num_slots):
            ring.count[slot] = np.maximum(ring.count[slot] - int(num_rejected[bi]), 0)
    return ring


# ---------------------------------------------------------------------------
# speculative decode without replay: one full state per window position
# ([ReplaySSM] "bottleneck" section: (1 + num_spec) states; [PR52191] item 3:
# the spec kernel reads a source state and writes destination states)
# ---------------------------------------------------------------------------

def spec_decode(pool, src_slots, dst_slots, q, k, v, a, b, A_log, dt_bias, scale=None, heads=None):
    """Verify a window of T tokens per sequence keeping every intermediate state.

    src_slots int [B]; dst_slots int [B, T]; q, k [B, T, Hk, dk]; v [B, T, Hv, dv];
    a, b [B, T, Hv].  Position t advances the state of position t-1 (the
    source slot for t = 0) by one token and writes it, rounded, to
    dst_slots[b, t]; its output reads the unrounded state, and the chain
    carries on from the unrounded state (stores inside one call are not
    re-read).  A destination slot outside the pool skips that write.
    Returns (new pool, o [B, T, Hv, dv]).
    """
    pool = np.array(pool, copy=True)
    sdt = dtype_of(pool)
    num_slots, Hv, dk, dv = pool.shape
    B, T, Hk = q.shape[0], q.shape[1], q.shape[2]
    ratio = Hv // Hk
    s = _scale(dk, scale)
    qf, kf, vf = widen(q), widen(k), widen(v)
    g, beta = gates(a, b, A_log, dt_bias)
    o = np.zeros((B, T, Hv, dv))
    src_pool = np.array(pool, copy=True)
    for bi in range(B):
        src = int(src_slots[bi])
        if not _slot_ok(src, num_slots):
            continue
        for h in (range(Hv) if heads is None else heads):
            hk = h // ratio
            S = widen(src_pool[src, h])
            for t in range(T):
                S, o[bi, t, h] = gdn_token(S, qf[bi, t, hk], kf[bi, t, hk], vf[bi, t, h],
                                           g[bi, t, h], beta[bi, t, h], s)
                dst = int(dst_slots[bi, t])
                if _slot_ok(dst, num_slots):
                    pool[dst, h] = to_storage(S, sdt)
    return pool, o


# ---------------------------------------------------------------------------
# state-block copy for prefix caching ([PR48109] implementation section: the
# state-copy kernel of --mamba-cache-mode align copies whole state blocks of
# every state tensor named by its pointer table)
# ---------------------------------------------------------------------------
def copy_state_blocks(tensors, src_slots, dst_slots):
    """Copy slot src_slots[j] over slot dst_slots[j] in every tensor, byte for byte.

    tensors: list of arrays [num_slots, ...] (any dtype, slots may differ per
    tensor).  A job whose source or destination is outside a tensor's slots
    is skipped for that tensor.  Sources are read from the tensors as they
    were before the call.  Returns new arrays.
    """
    out = []
    for t in tensors:
        before = np.array(t, copy=True)
        after = np.array(t, copy=True)
        n = before.shape[0]
        for s, d in zip(src_slots, dst_slots):
            s, d = int(s), int(d)
            if _slot_ok(s, n) and _slot_ok(d, n):
                after[d] = before[s]
        out.append(after)
    return out
