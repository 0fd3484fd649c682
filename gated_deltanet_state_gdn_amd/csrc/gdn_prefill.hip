// Chunked GDN prefill over packed variable-length sequences.
//
// Chunk form of the gated delta rule (the chunkwise WY/UT representation of
// the Gated Delta Networks paper, restated here for this library's dk x dv
// state; vLLM PR #52191 page, implementation items 3-4: the inter-chunk
// recurrence runs its GEMMs in FP32 and scales chunk states by exp(g_last)).
// Within a chunk of C tokens t = 0..C-1 (C = 16, 32 or 64; counted from the
// sequence start of this call), with gamma_t = g_0 + ... + g_t and S the state entering the
// chunk, every token's update unrolls to
//     S_t = e^{gamma_t} S + sum_{s<=t} e^{gamma_t - gamma_s} k_s u_s^T
// where the pseudo-values u solve the unit lower-triangular system
//     (I + A) U = diag(beta) (V - diag(e^gamma) K S),
//     A_ts = beta_t e^{gamma_t - gamma_s} k_t.k_s  for s < t.
// Hence, with T = (I + A)^-1 and P_ts = e^{gamma_t - gamma_s} q_t.k_s (s <= t):
//     U      = T diag(beta) (V - diag(e^gamma) K S)
//     O      = scale (diag(e^gamma) Q S + P U)
//     S_next = e^{gamma_C} S + (diag(e^{gamma_C - gamma}) K)^T U.
// Only exp(gamma_t - gamma_s) with s <= t and exp(gamma_t) appear, so nothing
// overflows however strong the decay.  A partial last chunk is padded with
// k = q = v = 0, g = 0, beta = 0, which leaves every formula exact.
//
// Kernel 1 (chunk-parallel, one workgroup per (chunk, key head), for the key
// head's value heads): K K^T and Q K^T once, then per value head its gates,
// gamma, A and P, and T by blocked inversion (16x16 diagonal blocks by
// substitution in registers, off-diagonal blocks by MFMA products), written to
// the workspace.  Kernel 2 (sequential over chunks, one workgroup per
// (sequence, value head, 32-column dv block); each dv column of S evolves on
// its own given k, g and beta): the S-dependent products [K;Q] S, T R, P U and
// K~^T U on MFMA with the state block resident in LDS, the state read from its
// slot once and written back, rounded, once.  Kernel 2 has three variants:
// bf16 inputs at dk = 64 / 128 (the key- and query-side products on bf16 MFMA
// with the fp32 side split in three bf16 terms, fixed wave roles), f16 inputs
// at dk = 64 / 128 (the same operand layout, fp32 MFMA), and the first,
// LDS-staged fp32 design for fp32 inputs and small head dims.
#include "gdn_device.h"
#include "gdn_launch.h"

namespace gdn {

// Chunk lengths: 16, 32 or 64 tokens (a multiple of the 16-row MFMA tile).
// The k-contiguous state kernels for 16-bit inputs are written for 64; the
// LDS-staged kernel takes any of the three.
constexpr int kC = 64;
// floats per (chunk slot, head) of the workspace: T, P, gamma, beta, e^gamma, e^{gamma_C - gamma}
template <int C>
constexpr int ws_floats() { return 2 * C * C + 4 * C; }
constexpr int kWsFloats = ws_floats<kC>();

// Chunk slot of chunk c of sequence n: n + floor(cu[n] / C) + c.  It is unique
// and below N + ceil(total / C) (floor((x+l)/C) >= floor(x/C) + ceil(l/C) - 1).
__host__ __device__ inline int64_t prefill_chunk_slots(int64_t N, int64_t total, int C) {
  return N + (total + C - 1) / C;
}

size_t prefill_workspace_bytes(int N, int64_t total, int Hv, int C) {
  return (size_t)prefill_chunk_slots(N, total, C) * (size_t)Hv * (2 * (size_t)C * C + 4 * (size_t)C) * sizeof(float);
}

bool prefill_chunk_slots_fit(int N, int64_t total, int Hk, int Hv, int C) {
  const int64_t units = ((int64_t)N * Hv + 7) / 8 * 8 * 4;
  const int64_t grouped = ((int64_t)N * Hk + 7) / 8 * 8 * (Hv / Hk) * 4;
  return prefill_chunk_slots(N, total, C) <= INT32_MAX && Hv <= 65535 && units <= INT32_MAX && grouped <= INT32_MAX;
}

typedef float f32x4_t __attribute__((ext_vector_type(4)));

// acc[16x16] += A[16 x K] B[K x 16] on v_mfma_f32_16x16x4_f32.  Operand
// layout: lane l supplies A(l % 16, k0 + l / 16) and B(k0 + l / 16, l % 16);
// result element r of lane l is C(4 (l / 16) + r, l % 16).
template <int K, class FA, class FB>
__device__ __forceinline__ f32x4_t mma16(f32x4_t acc, const FA& A, const FB& B, int lane) {
  const int i = lane & 15, kk = lane >> 4;
#pragma unroll 4
  for (int k0 = 0; k0 < K; k0 += 4) acc = __builtin_amdgcn_mfma_f32_16x16x4f32(A(i, k0 + kk), B(k0 + kk, i), acc, 0, 0, 0);
  return acc;
}

__device__ __forceinline__ int acc_row(int lane, int r) { return 4 * (lane >> 4) + r; }
__device__ __forceinline__ int acc_col(int lane) { return lane & 15; }

// One 16 x 16 tile of X Y^T over D columns, X and Y packed rows in LDS (row
// stride ldw words, a multiple of 4, rows past the data zeroed).  Lane l
// supplies row l % 16 of both at the same k; 16-bit rows use the gfx950
// 16x16x32 bf16 / f16 MFMA with one 16-byte LDS read per operand and k block,
// fp32 rows the 16x16x4 f32 one.  Element r of the result is (4 (l / 16) + r, l % 16).
template <int D, int EB>
__device__ __forceinline__ f32x4_t rows_xyt(const uint32_t* X, const uint32_t* Y, int ldw, int dt, int lane) {
  const int i = lane & 15, kb = lane >> 4;
  f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
  if constexpr (EB == 2) {
    typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
    typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
#pragma unroll
    for (int s = 0; s < (D + 31) / 32; ++s) {
      const int w0 = 16 * s + 4 * kb;  // word of element 32 s + 8 kb
      const bool kv = D >= 32 || w0 < D / 2;
      const int wr = kv ? w0 : 0;
      u32x4 a = *reinterpret_cast<const u32x4*>(X + i * ldw + wr);
      u32x4 b = *reinterpret_cast<const u32x4*>(Y + i * ldw + wr);
      if (!kv) a = b = u32x4{0u, 0u, 0u, 0u};
      if (dt == GDN_BF16)
        acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a), __builtin_bit_cast(bf16x8, b),
                                                      acc, 0, 0, 0);
      else
        acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8, a), __builtin_bit_cast(f16x8, b), acc,
                                                     0, 0, 0);
    }
  } else {
#pragma unroll 8
    for (int s = 0; s < D / 4; ++s)
      acc = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(X[i * ldw + 4 * s + kb]),
                                                 __uint_as_float(Y[i * ldw + 4 * s + kb]), acc, 0, 0, 0);
  }
  return acc;
}

// Gate input element i as raw bits (EB = 4: fp32; 2: bf16 or f16), and its value.
template <int EB>
__device__ __forceinline__ uint32_t gate_bits(const void* p, int64_t i) {
  if constexpr (EB == 4) return static_cast<const uint32_t*>(p)[i];
  else return static_cast<const uint16_t*>(p)[i];
}
template <int EB>
__device__ __forceinline__ float gate_value(uint32_t x, int dt) {
  if constexpr (EB == 4) return __uint_as_float(x);
  else return dt == GDN_BF16 ? bf16_bits_to_f32(x) : f16_bits_to_f32(x);
}

// ---------------------------------------------------------------- kernel 1
// One workgroup per (chunk slot, key head) for its R = Hv / Hk value heads:
// the key and query rows are loaded and K K^T, Q K^T formed once, then each
// value head scales them by its own gates and inverts its own (I + A).  The
// gate inputs of the first two value heads load with the rows, so at R <= 2 the
// workgroup waits on memory once; further heads load theirs two at a time.
template <int D, int EB, int C>
__global__ void __launch_bounds__(256) gdn_prefill_chunk_kernel(const PrefillArgs p, float* __restrict__ ws) {
  static_assert(C == 16 || C == 32 || C == 64, "chunk of 16, 32 or 64 tokens");
  constexpr int NT = C / 16;           // 16-row tiles per chunk
  constexpr int JPW = (2 * NT * NT + 3) / 4;  // K K^T and Q K^T tiles per wave
  constexpr int LDT = C + 4;
  constexpr int LDW = D * EB / 4 + 4;  // words per packed key / query row: 16-byte rows, 4 mod 8 banks
  constexpr int VE = 16 / EB, CPR = D / VE;
  constexpr int RMAX = 2;              // value heads whose gates are staged at once
  // two buffers: K rows then T, Q rows then A (about 40 KB in all at D = 128,
  // C = 64, so four work-groups share a CU and cover each other's memory waits)
  constexpr int UW = C * LDW > C * LDT ? C * LDW : C * LDT;
  __shared__ __align__(16) uint32_t s_u0[UW];
  __shared__ __align__(16) uint32_t s_u1[UW];
  __shared__ float s_M[4][16][17];
  uint32_t* const s_k = s_u0;  // then T (below)
  uint32_t* const s_q = s_u1;  // then A
  __shared__ float s_g[RMAX][C], s_beta[RMAX][C], s_gam[C];

  const int cs = blockIdx.x, hk = blockIdx.y;
  const int R = p.Hv / p.Hk;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int* cu = p.cu_seqlens;
  // largest n with n + cu[n] / C <= cs (the key is strictly increasing in n)
  int lo = 0, hi = p.N - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (mid + cu[mid] / C <= cs) lo = mid; else hi = mid - 1;
  }
  const int n = lo;
  const int c = cs - (n + cu[n] / C);
  const int seq_lo = cu[n], seq_hi = cu[n + 1];
  if (c < 0 || (int64_t)c * C >= (int64_t)(seq_hi - seq_lo)) return;  // unused chunk slot
  const int slot = p.slot_map[n];
  if (slot < 0 || (int64_t)slot >= p.num_slots) return;  // padded sequence: kernel 2 writes zeros
  const int t0 = seq_lo + c * C;
  const int len = min(C, seq_hi - t0);

  // keys and queries stay packed in their input dtype, rows >= len zeroed; thread
  // (r, t) = (tid / C, tid mod C) loads the gate inputs of value head hk R + r, token t.
  // Every thread loads (indices clamped into the chunk and the heads) and the
  // gate inputs go as raw bits of EB bytes, so all of them are one round: a
  // branch around a load, or a run-time dtype switch that widens inside its
  // branches, made the compiler wait for every load issued before.
  {
    constexpr int IT = (C * CPR + 255) / 256;
    u32x4 xk[IT], xq[IT];
#pragma unroll
    for (int u = 0; u < IT; ++u) {
      const int x = min(tid + u * 256, C * CPR - 1), r = x / CPR, cc = x - r * CPR;
      const int64_t off = (((int64_t)(t0 + min(r, len - 1)) * p.Hk + hk) * D + cc * VE) * EB;
      xk[u] = *reinterpret_cast<const u32x4*>(static_cast<const char*>(p.k) + off);
      xq[u] = *reinterpret_cast<const u32x4*>(static_cast<const char*>(p.q) + off);
    }
    const int gr = tid / C, gt = tid - gr * C;
    const bool gl = gr < RMAX && gr < R;
    const int h = hk * R + min(gr, min(RMAX, R) - 1);
    const int64_t gi = (int64_t)(t0 + min(gt, len - 1)) * p.Hv + h;
    const uint32_t ra = gate_bits<EB>(p.a, gi), rb = gate_bits<EB>(p.b, gi);
    const float al = p.A_log[h], db = p.dt_bias[h];
    const u32x4 z4 = {0u, 0u, 0u, 0u};
#pragma unroll
    for (int u = 0; u < IT; ++u) {
      const int x = tid + u * 256, r = x / CPR, cc = x - r * CPR;
      if (x < C * CPR) {
        *reinterpret_cast<u32x4*>(s_k + r * LDW + cc * 4) = r < len ? xk[u] : z4;
        *reinterpret_cast<u32x4*>(s_q + r * LDW + cc * 4) = r < len ? xq[u] : z4;
      }
    }
    if (gl) {
      const bool live = gt < len;
      s_g[gr][gt] = live ? gate_g(gate_value<EB>(ra, p.in_dt), al, db) : 0.f;
      s_beta[gr][gt] = live ? sigmoid_f(gate_value<EB>(rb, p.in_dt)) : 0.f;
    }
  }
  __syncthreads();
  const int lane0 = lane, tid0 = tid;
  // K K^T and Q K^T tiles (NT x NT of each; job = wave + 4 k), formed once for
  // every value head (16-bit rows: the exact bf16 / f16 products, fp32
  // accumulation); the upper tiles are not needed
  f32x4_t kt[JPW];
#pragma unroll
  for (int k = 0; k < JPW; ++k) {
    const int job = wave + 4 * k;
    const int isP = job / (NT * NT), I = (job / NT) % NT, J = job % NT;
    kt[k] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    if (job < 2 * NT * NT && J <= I)
      kt[k] = rows_xyt<D, EB>((isP ? s_q : s_k) + 16 * I * LDW, s_k + 16 * J * LDW, LDW, p.in_dt, lane);
  }

  for (int r = 0; r < R; ++r) {
    const int h = hk * R + r, rg = r % RMAX;
    // LDS bases and the thread indices made opaque per head, so the addresses of
    // the loop body are not hoisted out of it (they would hold a hundred registers)
    int zoff = 0, lane = lane0, tid = tid0;
    asm volatile("" : "+v"(zoff), "+v"(lane), "+v"(tid));
    float (*const s_T)[LDT] = reinterpret_cast<float (*)[LDT]>(s_u0 + zoff);
    float (*const s_A)[LDT] = reinterpret_cast<float (*)[LDT]>(s_u1 + zoff);
    __syncthreads();  // the key and query rows are read (first head), s_T is written out (later heads)
    if (rg == 0 && r > 0) {  // the next heads' gates
      const int gr = tid / C, gt = tid - gr * C;
      const int hg = h + min(gr, min(RMAX, R - r) - 1);  // every thread loads, as above
      const int64_t gi = (int64_t)(t0 + min(gt, len - 1)) * p.Hv + hg;
      const uint32_t ra = gate_bits<EB>(p.a, gi), rb = gate_bits<EB>(p.b, gi);
      const float al = p.A_log[hg], db = p.dt_bias[hg];
      if (gr < RMAX && r + gr < R) {
        const bool live = gt < len;
        s_g[gr][gt] = live ? gate_g(gate_value<EB>(ra, p.in_dt), al, db) : 0.f;
        s_beta[gr][gt] = live ? sigmoid_f(gate_value<EB>(rb, p.in_dt)) : 0.f;
      }
      __syncthreads();
    }
    if (wave == 0) {  // inclusive prefix sum of this head's g over the chunk
      float x = lane < C ? s_g[rg][lane] : 0.f;
#pragma unroll
      for (int off = 1; off < C; off <<= 1) {
        const float y = __shfl_up(x, off, 64);
        if (lane >= off) x += y;
      }
      if (lane < C) s_gam[lane] = x;
    }
    __syncthreads();

    float* wsp = ws + ((int64_t)cs * p.Hv + h) * ws_floats<C>();
    float* ws_T = wsp;
    float* ws_P = wsp + C * C;
    // A (strictly lower, into the Q buffer) and P (causal, to the workspace)
#pragma unroll
    for (int k = 0; k < JPW; ++k) {
      const int job = wave + 4 * k;
      const int isP = job / (NT * NT), I = (job / NT) % NT, J = job % NT;
      if (job < 2 * NT * NT) {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int t = 16 * I + acc_row(lane, e), sc = 16 * J + acc_col(lane);
          if (isP) ws_P[t * C + sc] = (sc <= t) ? expf(s_gam[t] - s_gam[sc]) * kt[k][e] : 0.f;
          else s_A[t][sc] = (sc < t) ? s_beta[rg][t] * expf(s_gam[t] - s_gam[sc]) * kt[k][e] : 0.f;
        }
      }
    }
    __syncthreads();

    // T = (I + A)^-1: diagonal 16x16 blocks by forward substitution, lane = (block, column)
    if (wave == 0 && lane < C) {
      const int blk = lane >> 4, j = lane & 15, base = 16 * blk;
      float x[16];
#pragma unroll
      for (int i = 0; i < 16; ++i) x[i] = (i == j) ? 1.f : 0.f;
#pragma unroll
      for (int i = 1; i < 16; ++i) {
#pragma unroll
        for (int s = 0; s < i; ++s) x[i] = fmaf(-s_A[base + i][base + s], x[s], x[i]);
      }
#pragma unroll
      for (int i = 0; i < 16; ++i) s_T[base + i][base + j] = x[i];
    }
    for (int i = tid; i < C * C; i += 256) {  // blocks above the diagonal are zero
      const int rr = i / C, cc = i - rr * C;
      if ((cc >> 4) > (rr >> 4)) s_T[rr][cc] = 0.f;
    }
    __syncthreads();
    // off-diagonal blocks, one level (I - J = lev) at a time:
    //   T_IJ = -T_II (sum_{k=J}^{I-1} A_Ik T_kJ)
    for (int lev = 1; lev < NT; ++lev) {
      const int J = wave, I = wave + lev;
      const bool act = I < NT;
      if (act) {
        f32x4_t m = {0.f, 0.f, 0.f, 0.f};
        for (int k0 = 0; k0 < 16 * lev; k0 += 16) {
          m = mma16<16>(m, [&](int i, int k) { return s_A[16 * I + i][16 * J + k0 + k]; },
                        [&](int k, int jj) { return s_T[16 * J + k0 + k][16 * J + jj]; }, lane);
        }
#pragma unroll
        for (int e = 0; e < 4; ++e) s_M[wave][acc_row(lane, e)][acc_col(lane)] = m[e];
      }
      __syncthreads();
      if (act) {
        f32x4_t t = {0.f, 0.f, 0.f, 0.f};
        t = mma16<16>(t, [&](int i, int k) { return s_T[16 * I + i][16 * I + k]; },
                      [&](int k, int jj) { return s_M[wave][k][jj]; }, lane);
#pragma unroll
        for (int e = 0; e < 4; ++e) s_T[16 * I + acc_row(lane, e)][16 * J + acc_col(lane)] = -t[e];
      }
      __syncthreads();
    }
    for (int i = tid; i < C * C; i += 256) ws_T[i] = s_T[i / C][i % C];
    if (tid < C) {
      wsp[2 * C * C + tid] = s_gam[tid];
      wsp[2 * C * C + C + tid] = s_beta[rg][tid];
      wsp[2 * C * C + 2 * C + tid] = expf(s_gam[tid]);
      wsp[2 * C * C + 3 * C + tid] = expf(s_gam[C - 1] - s_gam[tid]);
    }
  }
}

// ---------------------------------------------------------------- kernel 2
// dv columns per state-kernel workgroup (a multiple of 16)
#ifndef GDN_PREFILL_BV
#define GDN_PREFILL_BV 32
#endif

// waves of a state-kernel workgroup: its LDS allows one workgroup per CU, so
// the waves are what hides latency (measured on MI355X: 4 waves 2.19 ms, 8
// waves 1.53 ms, 16 waves 1.30 ms for the 4-sequence workload)
#ifndef GDN_PREFILL_STATE_WAVES
#define GDN_PREFILL_STATE_WAVES 16
#endif
constexpr int kStateThreads = 64 * GDN_PREFILL_STATE_WAVES;

template <int D>
struct PrefillGeom {
  static constexpr int BV = D < GDN_PREFILL_BV ? D : GDN_PREFILL_BV;  // dv columns per workgroup
  static constexpr int NB = D / BV;
  static constexpr int NJ = BV / 16;
};

template <int SDT, int D, int EB, int C>
__global__ void __launch_bounds__(kStateThreads) gdn_prefill_state_kernel(const PrefillArgs p, const float* __restrict__ ws) {
  using G = PrefillGeom<D>;
  constexpr int BV = G::BV, NB = G::NB, NJ = G::NJ;
  constexpr int NT = C / 16;  // 16-row tiles per chunk
  constexpr int LDK = D + 4, LDV = BV + 4, LDT = C + 4;
  constexpr int QRU = (C * LDK > 2 * C * LDV) ? C * LDK : 2 * C * LDV;
  __shared__ float s_k[C][LDK];
  __shared__ float s_qru[QRU];  // Q [C][LDK], then R [C][LDV] and U [C][LDV]
  __shared__ float s_v[C][LDV];
  __shared__ float s_T[C][LDT], s_P[C][LDT];
  __shared__ float s_S[D][LDV];
  __shared__ float s_X[2 * C][LDV];  // K S (rows 0..C-1), Q S (rows C..2C-1)
  __shared__ float s_gb[2][C];  // gamma, beta of the chunk
  __shared__ float s_eg[C], s_dec[C], s_egC;

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  // XCD-aware order: the NB column blocks of one (sequence, head) share bid % 8
  const int bid = blockIdx.x;
  const int x8 = bid & 7, y = bid >> 3;
  const int blk = y % NB;
  const int unit = (y / NB) * 8 + x8;
  if (unit >= p.N * p.Hv) return;
  const int n = unit / p.Hv, h = unit - n * p.Hv;
  const int hk = h / (p.Hv / p.Hk);
  const int seq_lo = p.cu_seqlens[n], seq_hi = p.cu_seqlens[n + 1];
  const int len = seq_hi - seq_lo;
  if (len <= 0) return;
  const int col0 = blk * BV;
  const int slot = p.slot_map[n];
  if (slot < 0 || (int64_t)slot >= p.num_slots) {  // padded sequence: zero outputs
    for (int i = tid; i < len * BV; i += kStateThreads) {
      const int t = i / BV, j = i - t * BV;
      store_elem(p.out, ((int64_t)(seq_lo + t) * p.Hv + h) * D + col0 + j, 0.f, p.out_dt);
    }
    return;
  }
  using ST = typename StateElem<SDT>::T;
  ST* tile = static_cast<ST*>(p.pool) + ((int64_t)slot * p.Hv + h) * (int64_t)(D * D);
  for (int i = tid; i < D * BV; i += kStateThreads) {
    const int r = i / BV, j = i - r * BV;
    s_S[r][j] = load_elem(tile, (int64_t)r * D + col0 + j, SDT);
  }

  float* s_q = s_qru;
  float* s_R = s_qru;
  float* s_U = s_qru + C * LDV;
  const float* s_beta = s_gb[1];
  const int nch = (len + C - 1) / C;

  // chunk inputs are staged through registers: the loads of chunk c + 1 are
  // issued right after chunk c reaches LDS and complete under its GEMMs
  RowStager<D, C, kStateThreads, EB> stk, stq;
  RowStager<BV, C, kStateThreads, EB> stv;
  RowStager<C, C, kStateThreads, 4> stT, stP;
  RowStager<C, 2, kStateThreads, 4> stg;
  auto issue = [&](int c) {
    const int t0 = seq_lo + c * C;
    const int L = min(C, seq_hi - t0);
    const float* wsp = ws + ((int64_t)(n + seq_lo / C + c) * p.Hv + h) * ws_floats<C>();
    auto krow = [&](int t) { return ((int64_t)(t0 + t) * p.Hk + hk) * D; };
    stk.issue(p.k, L, krow);
    stq.issue(p.q, L, krow);
    stv.issue(p.v, L, [&](int t) { return ((int64_t)(t0 + t) * p.Hv + h) * D + col0; });
    auto mrow = [](int r) { return (int64_t)r * C; };
    stT.issue(wsp, C, mrow);
    stP.issue(wsp + C * C, C, mrow);
    stg.issue(wsp + 2 * C * C, 2, mrow);
  };
  issue(0);
  for (int c = 0; c < nch; ++c) {
    const int t0 = seq_lo + c * C;
    const int L = min(C, seq_hi - t0);
    stk.commit(&s_k[0][0], LDK, p.in_dt);
    stq.commit(s_q, LDK, p.in_dt);
    stv.commit(&s_v[0][0], LDV, p.in_dt);
    stT.commit(&s_T[0][0], LDT, GDN_F32);
    stP.commit(&s_P[0][0], LDT, GDN_F32);
    stg.commit(&s_gb[0][0], C, GDN_F32);
    __syncthreads();
    if (c + 1 < nch) issue(c + 1);
    if (tid < C) {  // read after the next barrier
      const float gt = s_gb[0][tid], gC = s_gb[0][C - 1];
      s_eg[tid] = expf(gt);
      s_dec[tid] = expf(gC - gt);
      if (tid == 0) s_egC = expf(gC);
    }

    // X = [K; Q] S
    for (int job = wave; job < 2 * NT * NJ; job += kStateThreads / 64) {
      const int I = job / NJ, J = job - I * NJ;
      f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
      if (I < NT)
        acc = mma16<D>(acc, [&](int i, int k) { return s_k[16 * I + i][k]; },
                       [&](int k, int j) { return s_S[k][16 * J + j]; }, lane);
      else
        acc = mma16<D>(acc, [&](int i, int k) { return s_q[(16 * (I - NT) + i) * LDK + k]; },
                       [&](int k, int j) { return s_S[k][16 * J + j]; }, lane);
#pragma unroll
      for (int r = 0; r < 4; ++r) s_X[16 * I + acc_row(lane, r)][16 * J + acc_col(lane)] = acc[r];
    }
    __syncthreads();
    // R = diag(beta) (V - diag(e^gamma) K S)   (overwrites Q)
    for (int i = tid; i < C * BV; i += kStateThreads) {
      const int t = i / BV, j = i - t * BV;
      s_R[t * LDV + j] = s_beta[t] * (s_v[t][j] - s_eg[t] * s_X[t][j]);
    }
    __syncthreads();
    // U = T R
    for (int job = wave; job < NT * NJ; job += kStateThreads / 64) {
      const int I = job / NJ, J = job - I * NJ;
      f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
      acc = mma16<C>(acc, [&](int i, int k) { return s_T[16 * I + i][k]; },
                      [&](int k, int j) { return s_R[k * LDV + 16 * J + j]; }, lane);
#pragma unroll
      for (int r = 0; r < 4; ++r) s_U[(16 * I + acc_row(lane, r)) * LDV + 16 * J + acc_col(lane)] = acc[r];
    }
    __syncthreads();
    // O = scale (diag(e^gamma) Q S + P U)  and  S <- e^{gamma_C} S + (diag(dec) K)^T U
    const float egC = s_egC;
    for (int job = wave; job < (NT + D / 16) * NJ; job += kStateThreads / 64) {
      const int I = job / NJ, J = job - I * NJ;
      f32x4_t acc;
      if (I < NT) {
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int t = 16 * I + acc_row(lane, r);
          acc[r] = s_eg[t] * s_X[C + t][16 * J + acc_col(lane)];
        }
        acc = mma16<C>(acc, [&](int i, int k) { return s_P[16 * I + i][k]; },
                        [&](int k, int j) { return s_U[k * LDV + 16 * J + j]; }, lane);
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int t = 16 * I + acc_row(lane, r);
          if (t < L)
            store_elem(p.out, ((int64_t)(t0 + t) * p.Hv + h) * D + col0 + 16 * J + acc_col(lane), p.scale * acc[r],
                       p.out_dt);
        }
      } else {
        const int Is = I - NT;
#pragma unroll
        for (int r = 0; r < 4; ++r) acc[r] = egC * s_S[16 * Is + acc_row(lane, r)][16 * J + acc_col(lane)];
        acc = mma16<C>(acc, [&](int i, int k) { return s_k[k][16 * Is + i] * s_dec[k]; },
                        [&](int k, int j) { return s_U[k * LDV + 16 * J + j]; }, lane);
#pragma unroll
        for (int r = 0; r < 4; ++r) s_S[16 * Is + acc_row(lane, r)][16 * J + acc_col(lane)] = acc[r];
      }
    }
    __syncthreads();
  }
  for (int i = tid; i < D * BV; i += kStateThreads) {
    const int r = i / BV, j = i - r * BV;
    store_elem(tile, (int64_t)r * D + col0 + j, s_S[r][j], SDT);
  }
}

// ---------------------------------------------------------------- kernel 2, 16-bit inputs
// The same sequential chunk loop for bf16 / f16 inputs at head dims 64 and 128,
// arranged so that the MFMA pipes see little but MFMAs:
//  * In a block of 32 k values, lane (i, kk) of v_mfma_f32_16x16x4_f32 takes
//    k = 32 b + 8 kk + s in the s-th of eight consecutive instructions (one
//    permutation of the block's k for both operands), so every operand is a
//    16-byte run along k.
//  * The row-side operands that come from memory (K or Q rows for [K S] /
//    [Q S], T or P rows for T R / P U) are loaded by each wave straight into
//    registers, for chunk c + 1 as soon as chunk c has used them; they never
//    pass through LDS.
//  * LDS holds what the loop produces (S^T, R^T, U^T) and K^T for the state
//    update.  K^T is double-buffered: waves 8-15, idle while waves 0-7 form
//    U = T R, build chunk c + 1's K^T from a one-chunk-ahead register copy,
//    with one lane exchange per row pair and an XOR swizzle of 16-byte
//    column groups that keeps both its writes and its reads free of bank
//    conflicts.  The gate vectors are double-buffered alongside.
// Three barriers per chunk: after [K S] / [Q S] (R^T ready), after U = T R
// (U^T ready), after the outputs and the state update (S^T ready).
constexpr int kS16Threads = 1024;

// XCD-aware order of the k-contiguous state kernels' workgroups: every workgroup
// of one (sequence, key head), its Hv / Hk value heads times NB column blocks,
// shares bid mod 8, so one XCD's L2 fetches that key head's key and query rows
// for all of them.  unit = n Hv + h, or -1 past the last group.
__device__ __forceinline__ void key_group_unit(int bid, int NB, const PrefillArgs& p, int& unit, int& blk) {
  const int R = p.Hv / p.Hk, per = R * NB;
  const int x8 = bid & 7, y = bid >> 3;
  const int sub = y % per, grp = (y / per) * 8 + x8;
  blk = sub % NB;
  unit = grp < p.N * p.Hk ? grp * R + sub / NB : -1;
}

template <int IDT>
__device__ __forceinline__ void unpack8(const u32x4 w, float* f) {
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    if constexpr (IDT == GDN_BF16) {
      f[2 * i] = __uint_as_float(w[i] << 16);
      f[2 * i + 1] = __uint_as_float(w[i] & 0xffff0000u);
    } else {
      f[2 * i] = f16_bits_to_f32(w[i] & 0xffffu);
      f[2 * i + 1] = f16_bits_to_f32(w[i] >> 16);
    }
  }
}

template <int IDT>
__device__ __forceinline__ float half_to_f32(uint32_t h) {
  if constexpr (IDT == GDN_BF16) return __uint_as_float(h << 16);
  else return f16_bits_to_f32(h);
}

__device__ __forceinline__ f32x4 ld4(const float* p) { return *reinterpret_cast<const f32x4*>(p); }

// acc += A B over one block of 32 k: a[8] and b[8] hold this lane's eight k values
__device__ __forceinline__ f32x4 mfma8(f32x4 acc, const float* a, const float* b) {
#pragma unroll
  for (int s = 0; s < 8; ++s) acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a[s], b[s], acc, 0, 0, 0);
  return acc;
}

// One output element through a buffer resource: stores at or past the
// resource's byte size are dropped by the hardware, so every lane issues the
// same store whether or not its row exists (keeps vector-memory counts static).
__device__ __forceinline__ void out_store(__amdgpu_buffer_rsrc_t r, int byte_off, float x, int dt) {
  if (dt == GDN_F32) {
    __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(x), r, byte_off, 0, 0);
  } else if (dt == GDN_BF16) {
    __builtin_amdgcn_raw_buffer_store_b16(__builtin_bit_cast(unsigned short, (__bf16)x), r, byte_off, 0, 0);
  } else {
    __builtin_amdgcn_raw_buffer_store_b16(__builtin_bit_cast(unsigned short, (_Float16)x), r, byte_off, 0, 0);
  }
}

template <int SDT, int D, int IDT>
__global__ void __launch_bounds__(kS16Threads) gdn_prefill_state16_kernel(const PrefillArgs p, const float* __restrict__ ws) {
  constexpr int BV = 32, NB = D / BV, NT = kS16Threads, KB = D / 32;
  static_assert(D == 64 || D == 128, "16-bit state kernel: D = 64 or 128");
  constexpr int LTW = kC / 2 + 4;  // words per K^T row: 8 column groups of 4 words (swizzled) + pad
  constexpr int LTF = kC + 4;      // floats per R^T / U^T row
  constexpr int LSF = D + 4;       // floats per S^T row
  constexpr int KTL = kC * D / 8 / 512;  // K^T loads per lane of waves 8-15
  __shared__ __align__(16) uint32_t s_kt[2][D * LTW];
  __shared__ __align__(16) float s_St[BV * LSF];
  __shared__ __align__(16) float s_Rt[BV * LTF];
  __shared__ __align__(16) float s_Ut[BV * LTF];
  __shared__ __align__(16) float s_g[2][4 * kC];  // gamma, beta, e^gamma, e^{gamma_C - gamma}

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int li = lane & 15, kk = lane >> 4;
  int unit, blk;
  key_group_unit(blockIdx.x, NB, p, unit, blk);
  if (unit < 0) return;
  const int n = unit / p.Hv, h = unit - n * p.Hv;
  const int hk = h / (p.Hv / p.Hk);
  const int seq_lo = p.cu_seqlens[n], seq_hi = p.cu_seqlens[n + 1];
  const int len = seq_hi - seq_lo;
  if (len <= 0) return;
  const int col0 = blk * BV;
  const int slot = p.slot_map[n];
  if (slot < 0 || (int64_t)slot >= p.num_slots) {  // padded sequence: zero outputs
    for (int i = tid; i < len * BV; i += NT) {
      const int t = i / BV, j = i - t * BV;
      store_elem(p.out, ((int64_t)(seq_lo + t) * p.Hv + h) * D + col0 + j, 0.f, p.out_dt);
    }
    return;
  }
  using ST = typename StateElem<SDT>::T;
  ST* tile = static_cast<ST*>(p.pool) + ((int64_t)slot * p.Hv + h) * (int64_t)(D * D);
  for (int i = tid; i < D * BV; i += NT) {
    const int r = i / BV, j = i - r * BV;
    s_St[j * LSF + r] = load_elem(tile, (int64_t)r * D + col0 + j, SDT);
  }
  const int nch = (len + kC - 1) / kC;
  auto chunk_len = [&](int c) { return min(kC, len - c * kC); };
  auto chunk_ws = [&](int c) { return ws + ((int64_t)(n + seq_lo / kC + c) * p.Hv + h) * kWsFloats; };

  // wave roles: tile (I, J) of the 64 x 32 chunk outputs; waves 0-7 hold K and T
  // rows, waves 8-15 Q and P rows
  const bool lo = wave < 8;
  const int jw = wave & 7, I = jw >> 1, J = jw & 1;
  const int arow = 16 * I + li;
  const uint16_t* a1src = static_cast<const uint16_t*>(lo ? p.k : p.q);
  u32x4 a1[KB];
  f32x4 a2[4];
  uint32_t vv[4];
  auto load_a1 = [&](int c) {
    const int r = min(arow, chunk_len(c) - 1);  // rows past the end are zeroed where used
    const uint16_t* src = a1src + ((int64_t)(seq_lo + c * kC + r) * p.Hk + hk) * D + 8 * kk;
#pragma unroll
    for (int b = 0; b < KB; ++b) a1[b] = *reinterpret_cast<const u32x4*>(src + 32 * b);
  };
  auto load_a2 = [&](int c) {  // T rows (waves 0-7) or P rows (waves 8-15)
    const float* src = chunk_ws(c) + (lo ? 0 : kC * kC) + arow * kC + 8 * kk;
#pragma unroll
    for (int b = 0; b < 2; ++b) {
      a2[2 * b] = ld4(src + 32 * b);
      a2[2 * b + 1] = ld4(src + 32 * b + 4);
    }
  };
  auto load_v = [&](int c) {  // V at the accumulator positions of the [K S] tile
    const int L = chunk_len(c);
    const uint16_t* src = static_cast<const uint16_t*>(p.v) + (int64_t)h * D + col0 + 16 * J + li;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int r = min(16 * I + 4 * kk + e, L - 1);
      vv[e] = src[(int64_t)(seq_lo + c * kC + r) * p.Hv * D];
    }
  };
  // K^T staging (loaded by every wave, committed by waves 8-15): lane bits 0-2 =
  // 8-column group, 3-4 = row pair, 5 = row parity; waves w and 8 + w cover
  // rows 8 w .. 8 w + 7
  const int kw = wave & 7, kcg = lane & 7, krp = (lane >> 3) & 3, kodd = lane >> 5;
  const int krow = 8 * kw + 2 * krp + kodd;
  u32x4 ktr[KTL];
  f32x4 gr;
  auto load_kt = [&](int c) {
    const int r = min(krow, chunk_len(c) - 1);
    const uint16_t* src = static_cast<const uint16_t*>(p.k) + ((int64_t)(seq_lo + c * kC + r) * p.Hk + hk) * D + 8 * kcg;
#pragma unroll
    for (int u = 0; u < KTL; ++u) ktr[u] = *reinterpret_cast<const u32x4*>(src + 64 * u);
    gr = ld4(chunk_ws(c) + 2 * kC * kC + 4 * lane);
  };
  auto commit_kt = [&](int c) {
    const bool dead = krow >= chunk_len(c);
    uint32_t* kt = s_kt[c & 1];
#pragma unroll
    for (int u = 0; u < KTL; ++u) {
      u32x4 w = ktr[u];
      if (dead) w = u32x4{0u, 0u, 0u, 0u};
      // the even row keeps columns 0-3 of its group and takes the odd row's; the odd row columns 4-7
      const uint32_t give0 = kodd ? w[0] : w[2], give1 = kodd ? w[1] : w[3];
      const uint32_t own0 = kodd ? w[2] : w[0], own1 = kodd ? w[3] : w[1];
      const uint32_t got0 = __shfl_xor(give0, 32, 64), got1 = __shfl_xor(give1, 32, 64);
      const int d0 = 64 * u + 8 * kcg + (kodd ? 4 : 0);
      const int col = 4 * (kw ^ kcg) + krp;  // swizzled column group (d0 >> 3 & 7 == kcg) + row pair
#pragma unroll
      for (int m = 0; m < 4; ++m) {
        const uint32_t ow = m < 2 ? own0 : own1, gw = m < 2 ? got0 : got1;
        const uint32_t mine = (m & 1) ? (ow >> 16) : (ow & 0xffffu);
        const uint32_t theirs = (m & 1) ? (gw >> 16) : (gw & 0xffffu);
        kt[(d0 + m) * LTW + col] = kodd ? (theirs | (mine << 16)) : (mine | (theirs << 16));
      }
    }
    if (wave == 8) *reinterpret_cast<f32x4*>(s_g[c & 1] + 4 * lane) = gr;
  };

  // Every wave issues the same vector-memory instructions in the same order
  // each chunk (loads of a chunk past the last one re-read the last, K^T and
  // V rows are loaded by all waves, output stores past the end are dropped),
  // so the compiler's wait counts name exactly the loads each use needs and
  // the one-chunk-ahead loads stay in flight under the products.
  load_kt(0);
  load_a1(0);
  load_v(0);
  if (!lo) commit_kt(0);
  load_kt(min(1, nch - 1));
  load_a2(0);
  __syncthreads();

  const int ob = p.out_dt == GDN_F32 ? 4 : 2;
  for (int c = 0; c < nch; ++c) {
    const int t0 = seq_lo + c * kC;
    const int L = chunk_len(c);
    const int cn = min(c + 1, nch - 1);
    const float* g = s_g[c & 1];
    // ---- P1: [K S] (waves 0-7) or [Q S] (waves 8-15) for tile (I, J)
    f32x4 qs;
    {
      const float* Bt = s_St + (16 * J + li) * LSF + 8 * kk;
      f32x4 acc = {0.f, 0.f, 0.f, 0.f};
      const bool live = arow < L;
#pragma unroll
      for (int b = 0; b < KB; ++b) {
        float a[8], bb[8];
        unpack8<IDT>(a1[b], a);
        const f32x4 b0 = ld4(Bt + 32 * b), b1 = ld4(Bt + 32 * b + 4);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          a[e] = live ? a[e] : 0.f;
          a[4 + e] = live ? a[4 + e] : 0.f;
          bb[e] = b0[e];
          bb[4 + e] = b1[e];
        }
        acc = mfma8(acc, a, bb);
      }
      load_a1(cn);
      if (lo) {  // R^T[j][t] = beta_t (V[t][j] - e^{gamma_t} (K S)[t][j])
        const int tb = 16 * I + 4 * kk;
        const f32x4 be = ld4(g + kC + tb), eg = ld4(g + 2 * kC + tb);
        f32x4 r;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const float v = tb + e < L ? half_to_f32<IDT>(vv[e]) : 0.f;
          r[e] = be[e] * (v - eg[e] * acc[e]);
        }
        *reinterpret_cast<f32x4*>(s_Rt + (16 * J + li) * LTF + tb) = r;
      }
      load_v(cn);
      qs = acc;
    }
    __syncthreads();
    // ---- P2: U = T R on waves 0-7 (stored as U^T); waves 8-15 stage chunk c + 1's K^T
    if (lo) {
      const float* Bt = s_Rt + (16 * J + li) * LTF + 8 * kk;
      f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int b = 0; b < 2; ++b) {
        float a[8], bb[8];
        const f32x4 b0 = ld4(Bt + 32 * b), b1 = ld4(Bt + 32 * b + 4);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          a[e] = a2[2 * b][e];
          a[4 + e] = a2[2 * b + 1][e];
          bb[e] = b0[e];
          bb[4 + e] = b1[e];
        }
        acc = mfma8(acc, a, bb);
      }
      *reinterpret_cast<f32x4*>(s_Ut + (16 * J + li) * LTF + 16 * I + 4 * kk) = acc;
    } else {
      commit_kt(c + 1);  // past the last chunk this fills the idle buffer with unused rows
    }
    load_kt(min(c + 2, nch - 1));
    __syncthreads();
    // ---- P3: O = scale (e^gamma [Q S] + P U) on waves 8-15
    f32x4 o = {0.f, 0.f, 0.f, 0.f};
    if (!lo) {
      const float* Bt = s_Ut + (16 * J + li) * LTF + 8 * kk;
      const f32x4 eg = ld4(g + 2 * kC + 16 * I + 4 * kk);
#pragma unroll
      for (int e = 0; e < 4; ++e) o[e] = eg[e] * qs[e];
#pragma unroll
      for (int b = 0; b < 2; ++b) {
        float a[8], bb[8];
        const f32x4 b0 = ld4(Bt + 32 * b), b1 = ld4(Bt + 32 * b + 4);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          a[e] = a2[2 * b][e];
          a[4 + e] = a2[2 * b + 1][e];
          bb[e] = b0[e];
          bb[4 + e] = b1[e];
        }
        o = mfma8(o, a, bb);
      }
    }
    // ---- P3: S <- e^{gamma_C} S + (diag(dec) K)^T U; tile rows 16 Is.. of S, columns 16 Js..
    {
      const uint32_t* kt = s_kt[c & 1];
      const float egC = g[3 * kC - 1];
      for (int job = wave; job < (D / 16) * 2; job += NT / 64) {
        const int Is = job >> 1, Js = job & 1;
        const int i = 16 * Is + li;
        const uint32_t* A = kt + i * LTW;
        const int sw = (i >> 3) & 7;
        const float* Bt = s_Ut + (16 * Js + li) * LTF + 8 * kk;
        f32x4* Sp = reinterpret_cast<f32x4*>(s_St + (16 * Js + li) * LSF + 16 * Is + 4 * kk);
        u32x4 aw[2];
#pragma unroll
        for (int b = 0; b < 2; ++b) aw[b] = *reinterpret_cast<const u32x4*>(A + 4 * ((4 * b + kk) ^ sw));
        f32x4 acc = *Sp;
#pragma unroll
        for (int e = 0; e < 4; ++e) acc[e] *= egC;
#pragma unroll
        for (int b = 0; b < 2; ++b) {
          float a[8], bb[8];
          unpack8<IDT>(aw[b], a);
          const f32x4 d0 = ld4(g + 3 * kC + 32 * b + 8 * kk), d1 = ld4(g + 3 * kC + 32 * b + 8 * kk + 4);
          const f32x4 b0 = ld4(Bt + 32 * b), b1 = ld4(Bt + 32 * b + 4);
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            a[e] *= d0[e];
            a[4 + e] *= d1[e];
            bb[e] = b0[e];
            bb[4 + e] = b1[e];
          }
          acc = mfma8(acc, a, bb);
        }
        *Sp = acc;  // element e of lane (li, kk) is S(16 Is + 4 kk + e, 16 Js + li)
      }
    }
    {  // outputs of this chunk: rows t0 .. t0 + L - 1; waves 0-7 store nowhere
      const __amdgpu_buffer_rsrc_t r = __builtin_amdgcn_make_buffer_rsrc(
          static_cast<char*>(p.out) + (int64_t)t0 * p.Hv * D * ob, (short)0, L * p.Hv * D * ob, 0x00020000);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int t = 16 * I + 4 * kk + e;
        const int off = lo ? 0x7ffffff0 : ((t * p.Hv + h) * D + col0 + 16 * J + li) * ob;
        out_store(r, off, p.scale * o[e], p.out_dt);
      }
    }
    load_a2(cn);
    __syncthreads();
  }
  for (int i = tid; i < D * BV; i += NT) {
    const int r = i / BV, j = i - r * BV;
    store_elem(tile, (int64_t)r * D + col0 + j, s_St[j * LSF + r], SDT);
  }
}

// ---------------------------------------------------------------- kernel 2, bf16 inputs
// bf16 keys and queries are exact MFMA operands, so the three products that
// have a key or query on one side run on v_mfma_f32_16x16x32_bf16 with the
// fp32 side written as the sum of three bf16 terms (x = x1 + x2 + x3, each
// the bf16 rounding of what the earlier terms leave; together they keep more
// bits than fp32).  Each such product is three bf16 MFMAs per 32 k, against
// eight fp32 ones, and its results match fp32 arithmetic to within fp32
// rounding:  [K S] and [Q S] take S as three bf16 planes of S^T, the state
// update takes K^T (diag(dec) U) with diag(dec) U as three planes.  The two
// products with fp32 on both sides (T R and P U) stay on fp32 MFMA.  Layout,
// staging and wave roles are those of the 16-bit kernel above.
typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));

__device__ __forceinline__ f32x4 mfma_bf16(const u32x4 a, const u32x4 b, f32x4 acc) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a), __builtin_bit_cast(bf16x8_t, b), acc,
                                                 0, 0, 0);
}

// x = x1 + x2 + x3 in bf16 (round to nearest even); the differences are exact in fp32
__device__ __forceinline__ void split3(float x, uint32_t* h) {
  const __bf16 b1 = (__bf16)x;
  const float r1 = x - (float)b1;
  const __bf16 b2 = (__bf16)r1;
  const float r2 = r1 - (float)b2;
  const __bf16 b3 = (__bf16)r2;
  h[0] = __builtin_bit_cast(unsigned short, b1);
  h[1] = __builtin_bit_cast(unsigned short, b2);
  h[2] = __builtin_bit_cast(unsigned short, b3);
}

// four consecutive fp32 values -> three planes of two packed words each
__device__ __forceinline__ void split3x4(const f32x4 v, u32x2* planes) {
  uint32_t h[4][3];
#pragma unroll
  for (int e = 0; e < 4; ++e) split3(v[e], h[e]);
#pragma unroll
  for (int x = 0; x < 3; ++x) planes[x] = u32x2{h[0][x] | (h[1][x] << 16), h[2][x] | (h[3][x] << 16)};
}

template <int SDT, int D>
__global__ void __launch_bounds__(kS16Threads) gdn_prefill_state_bf16_kernel(const PrefillArgs p, const float* __restrict__ ws) {
  constexpr int BV = 32, NB = D / BV, NT = kS16Threads, KB = D / 32;
  static_assert(D == 64 || D == 128, "bf16 state kernel: D = 64 or 128");
  constexpr int LTW = kC / 2 + 4;  // words per K^T row (8 swizzled 4-word column groups + pad) and per (dec U)^T plane row
  constexpr int LTF = kC + 4;      // floats per R^T / U^T row
  constexpr int LSF = D + 4;       // floats per S^T row
  constexpr int LSW = D / 2 + 4;   // words per S^T plane row
  constexpr int LKW = D / 2 + 4;   // words per K row
  constexpr int KTL = kC * D / 8 / 512;
  __shared__ __align__(16) uint32_t s_kt[2][D * LTW];
  __shared__ __align__(16) uint32_t s_kr[2][kC * LKW];
  __shared__ __align__(16) float s_St[BV * LSF];
  __shared__ __align__(16) uint32_t s_Sp[3][BV * LSW];
  __shared__ __align__(16) float s_Rt[BV * LTF];
  __shared__ __align__(16) float s_Ut[BV * LTF];
  __shared__ __align__(16) uint32_t s_DUp[3][BV * LTW];
  __shared__ __align__(16) float s_g[2][4 * kC];  // gamma, beta, e^gamma, e^{gamma_C - gamma}

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int li = lane & 15, kk = lane >> 4;
  int unit, blk;
  key_group_unit(blockIdx.x, NB, p, unit, blk);
  if (unit < 0) return;
  const int n = unit / p.Hv, h = unit - n * p.Hv;
  const int hk = h / (p.Hv / p.Hk);
  const int seq_lo = p.cu_seqlens[n], seq_hi = p.cu_seqlens[n + 1];
  const int len = seq_hi - seq_lo;
  if (len <= 0) return;
  const int col0 = blk * BV;
  const int slot = p.slot_map[n];
  if (slot < 0 || (int64_t)slot >= p.num_slots) {  // padded sequence: zero outputs
    for (int i = tid; i < len * BV; i += NT) {
      const int t = i / BV, j = i - t * BV;
      store_elem(p.out, ((int64_t)(seq_lo + t) * p.Hv + h) * D + col0 + j, 0.f, p.out_dt);
    }
    return;
  }
  using ST = typename StateElem<SDT>::T;
  ST* tile = static_cast<ST*>(p.pool) + ((int64_t)slot * p.Hv + h) * (int64_t)(D * D);
  // S^T (fp32) and its three bf16 planes; lane quad (j, 4 rows)
  for (int i = tid; i < BV * (D / 4); i += NT) {
    const int j = i / (D / 4), r4 = (i - j * (D / 4)) * 4;
    f32x4 v;
#pragma unroll
    for (int e = 0; e < 4; ++e) v[e] = load_elem(tile, (int64_t)(r4 + e) * D + col0 + j, SDT);
    *reinterpret_cast<f32x4*>(s_St + j * LSF + r4) = v;
    u32x2 pl[3];
    split3x4(v, pl);
#pragma unroll
    for (int x = 0; x < 3; ++x) *reinterpret_cast<u32x2*>(s_Sp[x] + j * LSW + r4 / 2) = pl[x];
  }
  const int nch = (len + kC - 1) / kC;
  auto chunk_len = [&](int c) { return min(kC, len - c * kC); };
  auto chunk_ws = [&](int c) { return ws + ((int64_t)(n + seq_lo / kC + c) * p.Hv + h) * kWsFloats; };

  // Fixed wave roles, each with its own chunk loop and the same three barriers
  // per chunk:
  //   waves 0-3  (K role): [K S] for rows 16 w.., both column tiles; R^T; U = T R
  //   waves 4-7  (Q role): [Q S] for rows 16 (w - 4).., both column tiles; outputs
  //   waves 8-15 (S role): K and gate staging one chunk ahead (K^T for the
  //                        update, K rows for the K role); the state update
  // Every global element a work-group reads is loaded by one lane only, one
  // chunk ahead, and each role issues the same loads every chunk.  The K role
  // takes its key rows from the S role's LDS copy: reading them from memory
  // as well cost 3% of the kernel's time.
  // Rows past a chunk's end read the chunk's last row instead (key rows are
  // zero there): beta is zero there, so their [K S] rows, R rows and U rows
  // vanish, and their outputs are dropped.
  const int I = wave & 3;
  const int arow = 16 * I + li;
  // [X S] for rows 16 I.. and both 16-column tiles, S from its three planes.
  // The six plane reads of block b + 1 are issued before the MFMAs of block b
  // (the scheduling barrier keeps the compiler from sinking them), so LDS
  // latency hides behind the MFMAs of the same wave.
  auto xs_tiles = [&](const u32x4* a1, f32x4* res) {
    f32x4 h0[2] = {{0.f, 0.f, 0.f, 0.f}, {0.f, 0.f, 0.f, 0.f}}, h1[2] = {h0[0], h0[0]};
    u32x4 sb[2][2][3];
    auto fetch = [&](int b, u32x4 (*dst)[3]) {
#pragma unroll
      for (int J = 0; J < 2; ++J)
#pragma unroll
        for (int x = 0; x < 3; ++x)
          dst[J][x] = *reinterpret_cast<const u32x4*>(s_Sp[x] + (16 * J + li) * LSW + 4 * kk + 16 * b);
    };
    fetch(0, sb[0]);
#pragma unroll
    for (int b = 0; b < KB; ++b) {
      if (b + 1 < KB) fetch(b + 1, sb[(b + 1) & 1]);
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int J = 0; J < 2; ++J) {
        h0[J] = mfma_bf16(a1[b], sb[b & 1][J][0], h0[J]);
        h1[J] = mfma_bf16(a1[b], sb[b & 1][J][1], h1[J]);
        h1[J] = mfma_bf16(a1[b], sb[b & 1][J][2], h1[J]);
      }
    }
#pragma unroll
    for (int J = 0; J < 2; ++J)
#pragma unroll
      for (int e = 0; e < 4; ++e) res[J][e] = h0[J][e] + h1[J][e];
  };
  // acc[J] += (rows 16 I.. of T or P, registers) (B^T rows 16 J + li at bt, row
  // stride LTF) for both column tiles.  T and P are lower triangular, so row
  // block IC contracts over token blocks 0..IC only; lane (li, kk) holds
  // tokens 16 m + 4 kk + s of block m, which MFMA s contracts.  The B reads
  // are issued before the MFMAs.
  auto tri_tiles = [&](auto Ic, const f32x4* a2, const float* bt, f32x4* acc) {
    constexpr int IC = decltype(Ic)::value;
    f32x4 bv[IC + 1][2];
#pragma unroll
    for (int m = 0; m <= IC; ++m)
#pragma unroll
      for (int J = 0; J < 2; ++J) bv[m][J] = ld4(bt + (16 * J + li) * LTF + 16 * m + 4 * kk);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int m = 0; m <= IC; ++m)
#pragma unroll
      for (int e = 0; e < 4; ++e)
#pragma unroll
        for (int J = 0; J < 2; ++J)
          acc[J] = __builtin_amdgcn_mfma_f32_16x16x4f32(a2[m][e], bv[m][J][e], acc[J], 0, 0, 0);
  };
  auto load_rows = [&](const void* src, int c, u32x4* a1) {  // K or Q rows 16 I + li
    const int r = min(arow, chunk_len(c) - 1);
    const uint16_t* q = static_cast<const uint16_t*>(src) + ((int64_t)(seq_lo + c * kC + r) * p.Hk + hk) * D + 8 * kk;
#pragma unroll
    for (int b = 0; b < KB; ++b) a1[b] = *reinterpret_cast<const u32x4*>(q + 32 * b);
  };
  // T (which 0) or P (which 1) rows 16 I + li, token blocks 0..IC (the blocks
  // above the diagonal are zero)
  auto load_tri = [&](auto Ic, int c, int which, f32x4* a2) {
    constexpr int IC = decltype(Ic)::value;
    const float* q = chunk_ws(c) + which * kC * kC + arow * kC + 4 * kk;
#pragma unroll
    for (int m = 0; m <= IC; ++m) a2[m] = ld4(q + 16 * m);
  };

  // The K and Q roles are built once per row block (IC = wave mod 4), so that
  // every wave issues a fixed set of T or P loads and MFMAs.
  auto k_role = [&](auto Ic) {
    // ================================================================ K role
    u32x4 a1[KB];
    f32x4 a2[4];
    auto read_rows = [&](int c) {  // K rows 16 I + li of chunk c, staged by the S role (zero past the end)
      const uint32_t* q = s_kr[c & 1] + arow * LKW + 4 * kk;
#pragma unroll
      for (int b = 0; b < KB; ++b) a1[b] = *reinterpret_cast<const u32x4*>(q + 16 * b);
    };
    uint32_t vv[2][4];
    auto load_v = [&](int c) {  // V at the accumulator positions of both [K S] tiles
      const int L = chunk_len(c);
      const uint16_t* q = static_cast<const uint16_t*>(p.v) + (int64_t)h * D + col0 + li;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int64_t row = (int64_t)(seq_lo + c * kC + min(16 * I + 4 * kk + e, L - 1)) * p.Hv * D;
        vv[0][e] = q[row];
        vv[1][e] = q[row + 16];
      }
    };
    load_v(0);
    load_tri(Ic, 0, 0, a2);
    __syncthreads();
    read_rows(0);
    for (int c = 0; c < nch; ++c) {
      const int L = chunk_len(c), cn = min(c + 1, nch - 1);
      const float* g = s_g[c & 1];
      const int tb = 16 * I + 4 * kk;
      {  // P1: [K S], then R^T[j][t] = beta_t (V[t][j] - e^{gamma_t} (K S)[t][j])
        f32x4 ks[2];
        xs_tiles(a1, ks);
        const f32x4 be = ld4(g + kC + tb), eg = ld4(g + 2 * kC + tb);
#pragma unroll
        for (int J = 0; J < 2; ++J) {
          f32x4 r;
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const float v = tb + e < L ? __uint_as_float(vv[J][e] << 16) : 0.f;
            r[e] = be[e] * (v - eg[e] * ks[J][e]);
          }
          *reinterpret_cast<f32x4*>(s_Rt + (16 * J + li) * LTF + tb) = r;
        }
        load_v(cn);
      }
      __syncthreads();
      {  // P2: U = T R; U^T in fp32 and diag(dec) U as three bf16 planes
        f32x4 u[2] = {{0.f, 0.f, 0.f, 0.f}, {0.f, 0.f, 0.f, 0.f}};
        tri_tiles(Ic, a2, s_Rt, u);
        load_tri(Ic, cn, 0, a2);
        read_rows(c + 1);  // committed before the first barrier of this chunk
        const f32x4 dc = ld4(g + 3 * kC + tb);
#pragma unroll
        for (int J = 0; J < 2; ++J) {
          const int jr = 16 * J + li;
          *reinterpret_cast<f32x4*>(s_Ut + jr * LTF + tb) = u[J];
          f32x4 du;
#pragma unroll
          for (int e = 0; e < 4; ++e) du[e] = dc[e] * u[J][e];
          u32x2 pl[3];
          split3x4(du, pl);
#pragma unroll
          for (int x = 0; x < 3; ++x) *reinterpret_cast<u32x2*>(s_DUp[x] + jr * LTW + tb / 2) = pl[x];
        }
      }
      __syncthreads();
      __syncthreads();
    }
  };
  auto q_role = [&](auto Ic) {
    // ================================================================ Q role
    u32x4 a1[KB];
    f32x4 a2[4];
    const int ob = p.out_dt == GDN_F32 ? 4 : 2;
    load_rows(p.q, 0, a1);
    load_tri(Ic, 0, 1, a2);
    __syncthreads();
    for (int c = 0; c < nch; ++c) {
      const int t0 = seq_lo + c * kC;
      const int L = chunk_len(c), cn = min(c + 1, nch - 1);
      const float* g = s_g[c & 1];
      f32x4 qs[2];
      xs_tiles(a1, qs);  // P1
      load_rows(p.q, cn, a1);
      __syncthreads();
      __syncthreads();
      {  // P3: O = scale (e^gamma [Q S] + P U)
        const f32x4 eg = ld4(g + 2 * kC + 16 * I + 4 * kk);
        f32x4 o[2];
#pragma unroll
        for (int J = 0; J < 2; ++J)
#pragma unroll
          for (int e = 0; e < 4; ++e) o[J][e] = eg[e] * qs[J][e];
        tri_tiles(Ic, a2, s_Ut, o);
        load_tri(Ic, cn, 1, a2);
        // rows t0 .. t0 + L - 1 of the output; stores past the end are dropped
        const __amdgpu_buffer_rsrc_t r = __builtin_amdgcn_make_buffer_rsrc(
            static_cast<char*>(p.out) + (int64_t)t0 * p.Hv * D * ob, (short)0, L * p.Hv * D * ob, 0x00020000);
#pragma unroll
        for (int J = 0; J < 2; ++J)
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const int t = 16 * I + 4 * kk + e;
            out_store(r, ((t * p.Hv + h) * D + col0 + 16 * J + li) * ob, p.scale * o[J][e], p.out_dt);
          }
      }
      __syncthreads();
    }
  };
  using I0 = std::integral_constant<int, 0>;
  using I1 = std::integral_constant<int, 1>;
  using I2 = std::integral_constant<int, 2>;
  using I3 = std::integral_constant<int, 3>;
  if (wave < 4) {
    switch (I) {
      case 0: k_role(I0{}); break;
      case 1: k_role(I1{}); break;
      case 2: k_role(I2{}); break;
      default: k_role(I3{}); break;
    }
  } else if (wave < 8) {
    switch (I) {
      case 0: q_role(I0{}); break;
      case 1: q_role(I1{}); break;
      case 2: q_role(I2{}); break;
      default: q_role(I3{}); break;
    }
  } else {
    // ================================================================ S role
    // K^T staging: lane bits 0-2 = 8-column group, 3-4 = row pair, 5 = row
    // parity; wave 8 + w covers rows 8 w .. 8 w + 7
    const int kw = wave - 8, kcg = lane & 7, krp = (lane >> 3) & 3, kodd = lane >> 5;
    const int krow = 8 * kw + 2 * krp + kodd;
    u32x4 ktr[KTL];
    f32x4 gr;
    auto load_kt = [&](int c) {
      const int r = min(krow, chunk_len(c) - 1);
      const uint16_t* q = static_cast<const uint16_t*>(p.k) + ((int64_t)(seq_lo + c * kC + r) * p.Hk + hk) * D + 8 * kcg;
#pragma unroll
      for (int u = 0; u < KTL; ++u) ktr[u] = *reinterpret_cast<const u32x4*>(q + 64 * u);
      gr = ld4(chunk_ws(c) + 2 * kC * kC + 4 * lane);
    };
    auto commit_kt = [&](int c) {  // chunk c's K^T and gates into buffer c & 1
      const bool dead = krow >= chunk_len(c);
      uint32_t* kt = s_kt[c & 1];
#pragma unroll
      for (int u = 0; u < KTL; ++u) {
        u32x4 w = ktr[u];
        if (dead) w = u32x4{0u, 0u, 0u, 0u};
        *reinterpret_cast<u32x4*>(s_kr[c & 1] + krow * LKW + 4 * kcg + 32 * u) = w;
        // the even row keeps columns 0-3 of its group and takes the odd row's; the odd row columns 4-7
        const uint32_t give0 = kodd ? w[0] : w[2], give1 = kodd ? w[1] : w[3];
        const uint32_t own0 = kodd ? w[2] : w[0], own1 = kodd ? w[3] : w[1];
        const uint32_t got0 = __shfl_xor(give0, 32, 64), got1 = __shfl_xor(give1, 32, 64);
        const int d0 = 64 * u + 8 * kcg + (kodd ? 4 : 0);
        const int col = 4 * (kw ^ kcg) + krp;  // swizzled column group (d0 >> 3 & 7 == kcg) + row pair
#pragma unroll
        for (int m = 0; m < 4; ++m) {
          const uint32_t ow = m < 2 ? own0 : own1, gw = m < 2 ? got0 : got1;
          const uint32_t mine = (m & 1) ? (ow >> 16) : (ow & 0xffffu);
          const uint32_t theirs = (m & 1) ? (gw >> 16) : (gw & 0xffffu);
          kt[(d0 + m) * LTW + col] = kodd ? (theirs | (mine << 16)) : (mine | (theirs << 16));
        }
      }
      if (wave == 8) *reinterpret_cast<f32x4*>(s_g[c & 1] + 4 * lane) = gr;
    };
    load_kt(0);
    commit_kt(0);
    load_kt(min(1, nch - 1));
    __syncthreads();
    for (int c = 0; c < nch; ++c) {
      commit_kt(c + 1);  // past the last chunk this fills the idle buffer with unused rows
      load_kt(min(c + 2, nch - 1));
      __syncthreads();
      __syncthreads();
      {  // P3: S <- e^{gamma_C} S + K^T (diag(dec) U); tiles of rows 16 Is.., columns 16 Js..
        const uint32_t* kt = s_kt[c & 1];
        const float egC = s_g[c & 1][3 * kC - 1];
#pragma unroll
        for (int jj = 0; jj < (D / 16) * 2 / 8; ++jj) {
          const int job = kw + 8 * jj;
          const int Is = job >> 1, Js = job & 1;
          const int i = 16 * Is + li, jr = 16 * Js + li;
          const uint32_t* A = kt + i * LTW;
          const int sw = (i >> 3) & 7;
          f32x4* Sp = reinterpret_cast<f32x4*>(s_St + jr * LSF + 16 * Is + 4 * kk);
          f32x4 acc0 = *Sp, acc1 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
          for (int e = 0; e < 4; ++e) acc0[e] *= egC;
#pragma unroll
          for (int b = 0; b < 2; ++b) {
            const u32x4 aw = *reinterpret_cast<const u32x4*>(A + 4 * ((4 * b + kk) ^ sw));
            const int bo = jr * LTW + 16 * b + 4 * kk;
            acc0 = mfma_bf16(aw, *reinterpret_cast<const u32x4*>(s_DUp[0] + bo), acc0);
            acc1 = mfma_bf16(aw, *reinterpret_cast<const u32x4*>(s_DUp[1] + bo), acc1);
            acc1 = mfma_bf16(aw, *reinterpret_cast<const u32x4*>(s_DUp[2] + bo), acc1);
          }
          f32x4 acc;
#pragma unroll
          for (int e = 0; e < 4; ++e) acc[e] = acc0[e] + acc1[e];
          *Sp = acc;  // element e of lane (li, kk) is S(16 Is + 4 kk + e, 16 Js + li)
          u32x2 pl[3];
          split3x4(acc, pl);
#pragma unroll
          for (int x = 0; x < 3; ++x) *reinterpret_cast<u32x2*>(s_Sp[x] + jr * LSW + 8 * Is + 2 * kk) = pl[x];
        }
      }
      __syncthreads();
    }
  }
  for (int i = tid; i < D * BV; i += NT) {
    const int r = i / BV, j = i - r * BV;
    store_elem(tile, (int64_t)r * D + col0 + j, s_St[j * LSF + r], SDT);
  }
}

template <int D>
static hipError_t launch_state_bf16(const PrefillArgs& a, int state_dt, unsigned grid, float* ws, hipStream_t s) {
  switch (state_dt) {
    case GDN_F32:
      hipLaunchKernelGGL((gdn_prefill_state_bf16_kernel<GDN_F32, D>), dim3(grid), dim3(kS16Threads), 0, s, a, ws);
      break;
    case GDN_BF16:
      hipLaunchKernelGGL((gdn_prefill_state_bf16_kernel<GDN_BF16, D>), dim3(grid), dim3(kS16Threads), 0, s, a, ws);
      break;
    case GDN_F16:
      hipLaunchKernelGGL((gdn_prefill_state_bf16_kernel<GDN_F16, D>), dim3(grid), dim3(kS16Threads), 0, s, a, ws);
      break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

template <int D, int IDT>
static hipError_t launch_state16(const PrefillArgs& a, int state_dt, unsigned grid, float* ws, hipStream_t s) {
  switch (state_dt) {
    case GDN_F32:
      hipLaunchKernelGGL((gdn_prefill_state16_kernel<GDN_F32, D, IDT>), dim3(grid), dim3(kS16Threads), 0, s, a, ws);
      break;
    case GDN_BF16:
      hipLaunchKernelGGL((gdn_prefill_state16_kernel<GDN_BF16, D, IDT>), dim3(grid), dim3(kS16Threads), 0, s, a, ws);
      break;
    case GDN_F16:
      hipLaunchKernelGGL((gdn_prefill_state16_kernel<GDN_F16, D, IDT>), dim3(grid), dim3(kS16Threads), 0, s, a, ws);
      break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

template <int D, int EB, int C>
static hipError_t launch_prefill_d(const PrefillArgs& a, int state_dt, float* ws, hipStream_t s) {
  const int64_t ncs = prefill_chunk_slots(a.N, a.total_tokens, C);
  constexpr bool k_contig = EB == 2 && (D == 64 || D == 128) && C == kC;
  hipLaunchKernelGGL((gdn_prefill_chunk_kernel<D, EB, C>), dim3((unsigned)ncs, (unsigned)a.Hk), dim3(256), 0, s, a, ws);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int64_t units = (int64_t)a.N * a.Hv;
  if constexpr (k_contig) {  // 16-bit inputs, wide heads: the k-contiguous kernel
    const int64_t groups = (int64_t)a.N * a.Hk;
    const unsigned grid = (unsigned)(((groups + 7) / 8) * 8 * (a.Hv / a.Hk) * (D / 32));
    return a.in_dt == GDN_BF16 ? launch_state_bf16<D>(a, state_dt, grid, ws, s)
                               : launch_state16<D, GDN_F16>(a, state_dt, grid, ws, s);
  } else {
    const unsigned grid = (unsigned)(((units + 7) / 8) * 8 * PrefillGeom<D>::NB);
    switch (state_dt) {
      case GDN_F32:
        hipLaunchKernelGGL((gdn_prefill_state_kernel<GDN_F32, D, EB, C>), dim3(grid), dim3(kStateThreads), 0, s, a, ws);
        break;
      case GDN_BF16:
        hipLaunchKernelGGL((gdn_prefill_state_kernel<GDN_BF16, D, EB, C>), dim3(grid), dim3(kStateThreads), 0, s, a, ws);
        break;
      case GDN_F16:
        hipLaunchKernelGGL((gdn_prefill_state_kernel<GDN_F16, D, EB, C>), dim3(grid), dim3(kStateThreads), 0, s, a, ws);
        break;
      default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
  }
}

template <int D, int C>
static hipError_t launch_prefill_eb(const PrefillArgs& a, int state_dt, float* ws, hipStream_t s) {
  return a.in_dt == GDN_F32 ? launch_prefill_d<D, 4, C>(a, state_dt, ws, s) : launch_prefill_d<D, 2, C>(a, state_dt, ws, s);
}

template <int C>
static hipError_t launch_prefill_c(const PrefillArgs& a, int state_dt, int D, float* ws, hipStream_t s) {
  switch (D) {
    case 16: return launch_prefill_eb<16, C>(a, state_dt, ws, s);
    case 32: return launch_prefill_eb<32, C>(a, state_dt, ws, s);
    case 64: return launch_prefill_eb<64, C>(a, state_dt, ws, s);
    case 128: return launch_prefill_eb<128, C>(a, state_dt, ws, s);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_prefill(const PrefillArgs& a, int state_dt, int D, int chunk, float* ws, hipStream_t s) {
  switch (chunk) {
    case 16: return launch_prefill_c<16>(a, state_dt, D, ws, s);
    case 32: return launch_prefill_c<32>(a, state_dt, D, ws, s);
    case 64: return launch_prefill_c<64>(a, state_dt, D, ws, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace gdn
