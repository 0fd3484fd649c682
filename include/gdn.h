/*
 * gdn.h -- C ABI of the Gated DeltaNet (GDN) recurrent-state update library
 * for AMD Instinct MI355X (gfx950).
 *
 * The operation is the gated delta rule (Yang, Kautz, Hatamizadeh, "Gated
 * Delta Networks", 2024) as run by hybrid-model decode and prefill.  With a
 * per-(sequence, value head) state S of dk x dv and, per token, a key k and
 * query q (dk), a value v (dv), a log-decay g and a write strength beta:
 *
 *     S <- exp(g) S                                  (decay)
 *     S <- S + beta k (v - S^T k)^T                  (delta-rule correction)
 *     o  = scale * S^T q                             (read-out, scale = dk^-1/2)
 *
 * with the fused sigmoid gating g = -exp(A_log[h]) * softplus(a + dt_bias[h])
 * and beta = sigmoid(b).  Sources: vLLM PR #52191 summary page (prhub.com.cn),
 * implementation section items 3-4 (decode, chunked and spec kernels templated
 * on the state type; FP32 math with the state read and written in its storage
 * type, one rounding per write-back; chunk states scaled by exp(g_last)); AREX
 * feed article on ReplaySSM, "bottleneck" and "cache inputs, not state"
 * sections (full-state read and write per decode step; checkpoint plus ring
 * of inputs folded every L steps; q never cached).
 *
 * Conventions for every entry point
 *   - All math is FP32.  The state is stored as f32, bf16 or f16 and rounded
 *     to nearest-even once per write-back.
 *   - Every pointer argument is a DEVICE pointer unless stated otherwise; the
 *     struct arguments themselves live in host memory and are read during
 *     the call only.  The caller allocates and owns every buffer; the
 *     library allocates nothing and keeps no state between calls (the one
 *     exception is the fixed device scratch of gdn_replay_decode_noalloc).
 *   - Calls only validate and enqueue work on `stream` (a hipStream_t; NULL
 *     is the default stream).  They return before the work runs.
 *   - Tensors are dense and row-major with the last dimension fastest.
 *     Inputs q, k, v, a, b share one dtype `in_dtype`; q, k, v (and ring k,
 *     v) must be 16-byte aligned (they are read with 16-byte vector loads).
 *   - State pools are [num_slots, Hv, dk, dv] (dv fastest), 16-byte aligned.
 *     Value head h reads key head h / (Hv / Hk) (contiguous groups).
 *   - A slot index outside [0, num_slots) marks a padded row: its outputs
 *     are written as zero and no state or ring entry is touched.
 *   - Slots named by one call must be distinct (not checked).
 *   - Errors: invalid arguments are rejected synchronously, before anything
 *     is enqueued, with GDN_EINVAL or GDN_EUNSUPPORTED; a failed launch gives
 *     GDN_ELAUNCH.  gdn_last_error() describes the last failure of the
 *     calling thread.  There is no silent fallback and no logging.
 *   - Supported head dims: dk == dv in {16, 32, 64, 128}; Hv % Hk == 0.
 */
#ifndef GDN_H
#define GDN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum { GDN_F32 = 0, GDN_BF16 = 1, GDN_F16 = 2 } gdn_dtype;

typedef enum {
  GDN_OK = 0,
  GDN_EINVAL = 1,       /* null pointer, bad size, misaligned buffer, bad dtype value */
  GDN_EUNSUPPORTED = 2, /* valid request outside the compiled set (head dim, chunk, ring length) */
  GDN_ELAUNCH = 3       /* the HIP runtime refused a kernel launch */
} gdn_status;

/* Layer shape.  scale <= 0 selects dk^-1/2. */
typedef struct {
  int32_t num_k_heads; /* Hk */
  int32_t num_v_heads; /* Hv, a multiple of Hk */
  int32_t dk;
  int32_t dv;
  float scale;
} gdn_dims;

/* Gate inputs.  a, b: [rows, Hv] in the call's in_dtype (rows = tokens of the
 * call); A_log, dt_bias: float32 [Hv]. */
typedef struct {
  const void* a;
  const void* b;
  const float* A_log;
  const float* dt_bias;
} gdn_gates;

/* State pool [num_slots, Hv, dk, dv] of `dtype`, 16-byte aligned. */
typedef struct {
  void* base;
  gdn_dtype dtype;
  int64_t num_slots;
} gdn_pool;

/* ReplaySSM ring of a slot, caller-allocated and separate from the checkpoint
 * pool:
 *   k    [num_slots, Hk, L, dk]  copies of the keys, in `dtype`, once per key head
 *   v    [num_slots, Hv, L, dv]  copies of the values, in `dtype`
 *   g    [num_slots, Hv, L]      float32 log-decays
 *   beta [num_slots, Hv, L]      float32 write strengths
 *   start, count [num_slots]     int32, one pair per slot for all its heads;
 *                                live entry i (0 <= i < count) of every head
 *                                sits at ring index (start + i) mod L.
 * q is never stored.  Before first use, start and count must be zero (or any
 * 0 <= start < L, 0 <= count <= L).  Every head of a slot takes the same
 * windows, folds and rollbacks, so one pointer pair serves them all and the
 * value heads of a key head find its shared key entries where they wrote
 * them. */
typedef struct {
  void* k;
  void* v;
  float* g;
  float* beta;
  int32_t* start;
  int32_t* count;
  int64_t num_slots; /* slots the ring arrays hold; equals the checkpoint pool's */
  int32_t L;         /* 1 <= L <= 64 */
  gdn_dtype dtype;   /* dtype of k and v entries; must equal the calls' in_dtype */
} gdn_ring;

/* Single-token decode for B sequences (vLLM PR #52191 page, implementation
 * item 3: the fused sigmoid-gating delta-rule update; AREX ReplaySSM article,
 * "bottleneck" section: the whole state is read and written every step).
 *   q, k     [B, Hk, dk] in_dtype
 *   v        [B, Hv, dv] in_dtype
 *   gates    a, b [B, Hv]
 *   state    pool; slot_map[b] (device int32 [B]) selects the slot of row b
 *   out      [B, Hv, dv] out_dtype; o is read from the updated state before
 *            its write-back rounding.
 * Each touched (slot, head) state is read once and written once, rounded. */
gdn_status gdn_decode_step(const gdn_dims* dims, int32_t B, const void* q, const void* k,
                           const void* v, gdn_dtype in_dtype, const gdn_gates* gates,
                           const gdn_pool* state, const int32_t* slot_map, void* out,
                           gdn_dtype out_dtype, void* stream);

/* Speculative decode keeping one full state per window position, the
 * per-draft-token baseline (vLLM PR #52191 page, implementation item 3: the
 * speculative update kernel with separate source and destination state
 * pointers; AREX ReplaySSM article, "bottleneck" section: (1 + num_spec)
 * full states written per step whether or not drafts are accepted).
 *   q, k       [B, T, Hk, dk] in_dtype
 *   v          [B, T, Hv, dv] in_dtype
 *   gates      a, b [B, T, Hv]
 *   state      pool holding both the sources and the destinations
 *   src_slots  device int32 [B]: the state row b starts from (outside the
 *              pool: padded row, zero outputs, nothing written)
 *   dst_slots  device int32 [B, T]: where the state after position t is
 *              written, rounded once (outside the pool: that write is skipped)
 *   out        [B, T, Hv, dv] out_dtype; position t reads the state after
 *              its own token, before rounding.
 * The chain between positions carries the unrounded FP32 state.  Destination
 * slots must be distinct and must not be any row's source slot in the same
 * call (not checked).  1 <= T and 4 T (3 dk + 3) bytes <= 48 KiB (T <= 31 at
 * dk = 128), else GDN_EUNSUPPORTED. */
gdn_status gdn_spec_decode(const gdn_dims* dims, int32_t B, int32_t T, const void* q, const void* k,
                           const void* v, gdn_dtype in_dtype, const gdn_gates* gates,
                           const gdn_pool* state, const int32_t* src_slots,
                           const int32_t* dst_slots, void* out, gdn_dtype out_dtype, void* stream);

/* Chunked prefill of N packed variable-length sequences (vLLM PR #52191 page,
 * implementation items 3-4: the chunked inter-chunk recurrence; chunk states
 * are scaled by exp(g_last); FP32 buffers, slot read at the start and written
 * at the end).
 *   cu_seqlens  device int32 [N+1], non-decreasing, cu_seqlens[0] = 0,
 *               cu_seqlens[N] = total_tokens
 *   q, k        [total_tokens, Hk, dk] in_dtype
 *   v           [total_tokens, Hv, dv] in_dtype
 *   gates       a, b [total_tokens, Hv]
 *   state       sequence n starts from slot slot_map[n] and its final state is
 *               written back there, rounded once per call; a zero-length
 *               sequence leaves its slot untouched.  The state is carried
 *               exactly across calls: two calls over a split sequence equal
 *               one call up to that one extra rounding.
 *   out         [total_tokens, Hv, dv] out_dtype
 *   chunk       tokens per chunk, counted from each sequence's start in this
 *               call: 16, 32 or 64 (the chunked form is exact for any chunk
 *               length; 64 runs the fastest kernels for 16-bit inputs at
 *               dk = 64 and 128), else GDN_EUNSUPPORTED.
 *   workspace   device scratch of at least gdn_chunk_prefill_workspace_bytes()
 *               bytes, 256-byte aligned, owned by the caller, not read before
 *               it is written; NULL is allowed when that size is 0.
 * A sequence longer than 2^31 - 1 tokens is rejected. */
size_t gdn_chunk_prefill_workspace_bytes(const gdn_dims* dims, int32_t N, int64_t total_tokens,
                                         int32_t chunk);
gdn_status gdn_chunk_prefill(const gdn_dims* dims, int32_t N, const int32_t* cu_seqlens,
                             int64_t total_tokens, int32_t chunk, const void* q, const void* k,
                             const void* v, gdn_dtype in_dtype, const gdn_gates* gates,
                             const gdn_pool* state, const int32_t* slot_map, void* out,
                             gdn_dtype out_dtype, void* workspace, size_t workspace_bytes,
                             void* stream);

/* ReplaySSM-style decode of a window of T tokens per sequence (AREX ReplaySSM
 * article, "cache inputs, not state": checkpoint S0 plus a ring of the last
 * inputs, folded into S0 every L steps; other steps read outputs from S0 and
 * the ring without writing the state; a verify window is evaluated in one
 * pass and rejected drafts are dropped by moving the ring pointer).
 *   q, k   [B, T, Hk, dk] in_dtype;  v [B, T, Hv, dv];  gates a, b [B, T, Hv]
 *   ckpt   checkpoint pool; slot_map[b] selects the slot of row b
 *   ring   the ring; T must satisfy 1 <= T <= ring->L
 *   out    [B, T, Hv, dv] out_dtype
 *   workspace  device scratch of at least gdn_replay_workspace_bytes() bytes,
 *          256-byte aligned, owned by the caller, not read before it is
 *          written (it carries per-unit vectors and ring-pointer records
 *          between the kernels of one call); calls that share a workspace
 *          must not overlap.
 * Per sequence: if count + T > L, every committed entry of each value head is
 * first folded into that head's checkpoint (one rounding) and the ring emptied
 * (start += count mod L, count = 0); then the T new entries are appended at
 * ring indices (start + count + t) mod L and count += T; window position t
 * outputs scale * S_t^T q_t where S_t is the checkpoint advanced over the
 * first count_before + t + 1 live entries (computed without writing it).
 * L and T are limited by a 64 KiB LDS staging budget:
 * 4 ((L+T)(2 dk + 6) + T (dk + 1) + (L+T)^2 + 3 (L+T) T) bytes (at dk = 128,
 * L = 16 allows every T <= 16). */
size_t gdn_replay_workspace_bytes(const gdn_dims* dims, int32_t B, int32_t T);
gdn_status gdn_replay_decode(const gdn_dims* dims, int32_t B, int32_t T, const void* q,
                             const void* k, const void* v, gdn_dtype in_dtype,
                             const gdn_gates* gates, const gdn_pool* ckpt,
                             const int32_t* slot_map, const gdn_ring* ring, void* out,
                             gdn_dtype out_dtype, void* workspace, size_t workspace_bytes,
                             void* stream);

/* gdn_replay_decode without a caller workspace, for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc).  The workspace is a fixed device array
 * inside the library, one per GPU, 96 MiB, held from the first call on that
 * GPU until the process ends; the call itself allocates nothing.  Arguments,
 * results and errors are those of gdn_replay_decode, plus GDN_EUNSUPPORTED
 * when gdn_replay_workspace_bytes(dims, B, T) exceeds 96 MiB (B * Hv * T <=
 * 96,790 at dv = 128, e.g. 512 rows x 32 value heads x 5-token windows), and
 * GDN_ELAUNCH if the array's device address cannot be obtained.  Every call on
 * one GPU uses the same array: calls that overlap on one GPU (on different
 * streams, or from different threads without ordering) race and give
 * undefined results. */
gdn_status gdn_replay_decode_noalloc(const gdn_dims* dims, int32_t B, int32_t T, const void* q,
                                     const void* k, const void* v, gdn_dtype in_dtype,
                                     const gdn_gates* gates, const gdn_pool* ckpt,
                                     const int32_t* slot_map, const gdn_ring* ring, void* out,
                                     gdn_dtype out_dtype, void* stream);

/* Fold every committed ring entry of the mapped slots into their checkpoints
 * (one rounding each) and empty their rings.  After it, the checkpoint is the
 * plain decode state and the other entry points may use the slot. */
gdn_status gdn_replay_flush(const gdn_dims* dims, int32_t B, const gdn_pool* ckpt,
                            const int32_t* slot_map, const gdn_ring* ring, void* stream);

/* Dual-precision checkpoint variants (AREX ReplaySSM article, "cache inputs,
 * not state" section, its closing paragraph on precision: the scheme it cites
 * recurses on a high-precision checkpoint and serves reads from a
 * low-precision copy).  `master` is the f32 checkpoint pool that every fold reads and
 * writes; `read_copy` is a bf16 or f16 pool of the same slots and shape that
 * holds master rounded once.  Each fold (count + T > L) writes the folded
 * state to master and, rounded, to read_copy; window outputs read read_copy
 * (half the bytes of an f32 checkpoint) and the ring.  Everything else is as
 * gdn_replay_decode / gdn_replay_flush.  gdn_replay_flush_dual also refreshes
 * read_copy from master for every mapped slot, whether or not its ring is
 * empty: call it once to initialise read_copy before the first step.
 * read_copy must not alias master. */
gdn_status gdn_replay_decode_dual(const gdn_dims* dims, int32_t B, int32_t T, const void* q,
                                  const void* k, const void* v, gdn_dtype in_dtype,
                                  const gdn_gates* gates, const gdn_pool* master,
                                  const gdn_pool* read_copy, const int32_t* slot_map,
                                  const gdn_ring* ring, void* out, gdn_dtype out_dtype,
                                  void* workspace, size_t workspace_bytes, void* stream);
gdn_status gdn_replay_flush_dual(const gdn_dims* dims, int32_t B, const gdn_pool* master,
                                 const gdn_pool* read_copy, const int32_t* slot_map,
                                 const gdn_ring* ring, void* stream);

/* Drop the last num_rejected[b] live entries of row b's slot (all its heads):
 * count <- max(count - r, 0), the pointer move that replaces a state
 * rollback.  num_rejected: device int32 [B]; a negative entry counts as 0. */
gdn_status gdn_replay_rollback(const gdn_dims* dims, int32_t B, const int32_t* slot_map,
                               const int32_t* num_rejected, const gdn_ring* ring, void* stream);

/* One state tensor for gdn_copy_state_blocks: slot i occupies bytes
 * [base + i * slot_bytes, base + (i + 1) * slot_bytes).  `base` is a device
 * address kept as an unsigned 64-bit value (vLLM PR #48109 page, the XPU
 * state-pointer fix: device addresses may exceed 2^63, so a signed 64-bit
 * table loses or wraps them). */
typedef struct {
  uint64_t base;
  uint64_t slot_bytes;
  uint64_t num_slots;
} gdn_state_ref;

/* State-block copy for prefix caching (vLLM PR #48109 page, implementation
 * section: the state-copy kernel of --mamba-cache-mode align, driven by
 * tables of state base addresses).  For every job j < n and every tensor
 * p < P: slot src_slots[j] of refs[p] is copied byte for byte over slot
 * dst_slots[j] of refs[p].
 *   refs            device array of P gdn_state_ref, 8-byte aligned
 *   max_slot_bytes  host value >= every refs[p].slot_bytes (sizes the grid;
 *                   at most 2^31 * 64 KiB)
 *   src_slots, dst_slots  device int32 [n]
 * A job whose source or destination is outside [0, num_slots) of a tensor
 * is skipped for that tensor.  A slot must not be both a source and a
 * destination in one call, and destinations must be distinct (not checked).
 * Any base, slot size and alignment is accepted (16-byte-aligned ones copy
 * with vector accesses).  P <= 65535 and n <= 65535. */
gdn_status gdn_copy_state_blocks(const gdn_state_ref* refs, int32_t P, uint64_t max_slot_bytes,
                                 const int32_t* src_slots, const int32_t* dst_slots, int32_t n,
                                 void* stream);

/* ------------------------------------------------------------------ Mamba2
 * The second SSM variant of the ReplaySSM article (AREX ReplaySSM article:
 * "bottleneck", "cache inputs, not state" and "numbers" sections; the
 * recurrence is Dao and Gu's selective state-space update).  Per head h of
 * group h / (H / G), with dt' = softplus(dt + dt_bias[h]) and
 * g = -exp(A_log[h]) dt':
 *     S <- exp(g) S + dt' x B^T        (S is headdim x dstate, dstate fastest)
 *     y  = S C + D[h] x
 * FP32 math; the state is rounded once per write-back. */
typedef struct {
  int32_t num_heads;  /* H */
  int32_t num_groups; /* G, divides H */
  int32_t headdim;    /* d: 16, 64 or 128 */
  int32_t dstate;     /* n: 16, 64 or 128 */
} gdn_m2_dims;

/* dt: [rows, H] in the call's in_dtype (the raw step before softplus);
 * A_log, dt_bias, D: float32 [H]. */
typedef struct {
  const void* dt;
  const float* A_log;
  const float* dt_bias;
  const float* D;
} gdn_m2_params;

/* Mamba2 ReplaySSM ring, caller-allocated:
 *   x     [num_slots, H, L, d]  copies of the head inputs, in `dtype`
 *   Bm    [num_slots, G, L, n]  copies of the group B vectors, in `dtype`
 *   g     [num_slots, H, L]     float32 log-decays
 *   dtp   [num_slots, H, L]     float32 steps dt'
 *   start, count [num_slots]    int32, shared by the slot's heads
 * C is never stored.  Before first use start and count must be zero. */
typedef struct {
  void* x;
  void* Bm;
  float* g;
  float* dtp;
  int32_t* start;
  int32_t* count;
  int64_t num_slots;
  int32_t L;       /* 1 <= L <= 64 */
  gdn_dtype dtype; /* must equal the calls' in_dtype */
} gdn_m2_ring;

/* One token for B sequences: x [B, H, d], Bm and Cm [B, G, n], dt [B, H];
 * state pool [num_slots, H, d, n]; y [B, H, d]. */
gdn_status gdn_mamba2_decode_step(const gdn_m2_dims* dims, int32_t B, const void* x, const void* Bm,
                                  const void* Cm, gdn_dtype in_dtype, const gdn_m2_params* params,
                                  const gdn_pool* state, const int32_t* slot_map, void* y,
                                  gdn_dtype out_dtype, void* stream);

/* Replay step of T tokens: x [B, T, H, d], Bm and Cm [B, T, G, n], dt
 * [B, T, H]; y [B, T, H, d].  Per slot: if count + T > L, every committed
 * entry is first folded into each head's checkpoint (one rounding) and the
 * ring emptied; then the window is appended at (start + count + t) mod L and
 * count += T; window position t outputs y computed from the checkpoint
 * advanced over the first count_before + t + 1 live entries (without writing
 * it).  x and the ring's x must be 16-byte aligned.  With HPG = H / G heads
 * per group, 4 (L n + 2 T n + T L + HPG (2 L + T L + T + T d)) bytes of
 * staging must fit 64 KiB, else GDN_EUNSUPPORTED. */
gdn_status gdn_mamba2_replay_decode(const gdn_m2_dims* dims, int32_t B, int32_t T, const void* x,
                                    const void* Bm, const void* Cm, gdn_dtype in_dtype,
                                    const gdn_m2_params* params, const gdn_pool* ckpt,
                                    const int32_t* slot_map, const gdn_m2_ring* ring, void* y,
                                    gdn_dtype out_dtype, void* stream);

/* Fold every committed entry of the mapped slots into their checkpoints. */
gdn_status gdn_mamba2_replay_flush(const gdn_m2_dims* dims, int32_t B, const gdn_pool* ckpt,
                                   const int32_t* slot_map, const gdn_m2_ring* ring, void* stream);

/* count <- max(count - num_rejected[b], 0) for row b's slot (device int32 [B]). */
gdn_status gdn_mamba2_replay_rollback(const gdn_m2_dims* dims, int32_t B, const int32_t* slot_map,
                                      const int32_t* num_rejected, const gdn_m2_ring* ring,
                                      void* stream);

/* Static description of a status code (never NULL). */
const char* gdn_status_string(gdn_status status);

/* Description of the last failure reported to the calling thread ("" if none). */
const char* gdn_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* GDN_H */
