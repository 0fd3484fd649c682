// ReplaySSM-style GDN decode: a checkpoint S0 per (slot, value head) plus a
// ring of the last <= L state-building inputs (k, v, g, beta) replaces the
// per-step full-state write (AREX ReplaySSM article, "cache inputs, not state"
// section).  Every kernel works on independent (sequence, value head) units:
// a unit owns its checkpoint tile, its ring entries and its ring pointers.
//
// A step of T tokens runs three kernels:
//   fold   - if count + T > L, fold the committed entries into S0 (sequential
//            rank-1 updates on the tile held in VGPRs), write S0 back rounded
//            once and empty the ring; every other unit exits at once;
//   prep   - stage the live entries and the window, compute per window
//            position t the vectors w_t and acc_t below, append the window
//            to the ring;
//   stream - o_t = scale (S0^T w_t + acc_t): one read pass over S0 for all T
//            positions, a plain batched matrix-vector product that runs at
//            high occupancy.
//
// prep unrolls S_i = a_i (I - b_i k_i k_i^T) S_{i-1} + b_i k_i v_i^T
// (a_i = exp(g_i)).  Transposing gives S_n^T q = S0^T w + acc with
//     w   = e^{G_n} q - sum_j e^{G_j} c_j k_j,    acc = sum_j c_j v_j,
//     c_i = b_i (e^{G_n - G_i} (k_i . q) - sum_{j > i} e^{G_j - G_i} (k_i . k_j) c_j)
// where G_j is the sum of g over the live entries up to j (every exponent is
// <= 0).  The c are one small back substitution over the Gram matrix of the
// live keys and their products with q, so a window position costs
// O(n (dk + dv)) plus O(n^2) scalars and S_n itself is never materialised.
#include "gdn_device.h"
#include "gdn_launch.h"

// streaming (non-temporal) checkpoint loads and stores for fp32 checkpoints
#ifndef GDN_REPLAY_NT_F32
#define GDN_REPLAY_NT_F32 1
#endif
// waves per workgroup of the stream and fold kernels
#ifndef GDN_REPLAY_WAVES
#define GDN_REPLAY_WAVES 4
#endif
#ifndef GDN_REPLAY_WAVES_16
#define GDN_REPLAY_WAVES_16 2
#endif

namespace gdn {

template <int SDT, int D>
using ReplayGeom = TileGeom<SDT, D, SDT == GDN_F32 ? GDN_REPLAY_WAVES : GDN_REPLAY_WAVES_16>;

constexpr int kStageRows = 16;  // entry rows staged per batch of loads
constexpr int kStreamTB = 4;    // window positions reduced per pass over the tile

// Dynamic LDS of the fold kernel (floats): committed entries k, v [L][D+1], exp(g) and beta [L].
__host__ __device__ inline size_t replay_fold_lds_bytes(int D, int L) {
  return (size_t)L * (2 * ((size_t)D + 1) + 2) * sizeof(float);
}

size_t replay_workspace_bytes(int64_t B, int Hv, int T, int D) {
  return (size_t)B * (size_t)Hv * (size_t)T * 2 * (size_t)D * sizeof(float);
}

struct RingPos {
  int st, cnt;
};

// Ring pointers are clamped into range so that a corrupted pointer pair cannot
// send an access outside the unit's entries.
__device__ __forceinline__ RingPos ring_pos(const RingArgs& R, int64_t unit) {
  const int L = R.L;
  int st = R.start[unit], cnt = R.count[unit];
  st = ((st % L) + L) % L;
  cnt = cnt < 0 ? 0 : (cnt > L ? L : cnt);
  return RingPos{st, cnt};
}

// ---------------------------------------------------------------- fold
// Also the flush (T == 0: fold whenever the ring is not empty).
template <int SDT, int D, bool NT, int EB>
__global__ void __launch_bounds__((ReplayGeom<SDT, D>::NW * 64))
gdn_replay_fold_kernel(const ReplayArgs P) {
  using G = ReplayGeom<SDT, D>;
  constexpr int VEC = G::VEC, LPR = G::LPR, RPW = G::RPW, NW = G::NW, PASSES = G::PASSES;
  constexpr int NTH = NW * 64;
  constexpr int LDE = D + 1;
  using IO = TileIO<SDT, VEC, NT>;
  using ST = typename StateElem<SDT>::T;
  using Stager = RowStager<D, kStageRows, NTH, EB>;

  extern __shared__ float s_dyn[];
  __shared__ float s_red[2][NW][D];

  const DecodeArgs& p = P.d;
  const RingArgs& R = P.ring;
  const int T = P.T, L = R.L;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int b = blockIdx.x / p.Hv;
  const int h = blockIdx.x - b * p.Hv;
  const int slot = p.slot_map[b];
  if (slot < 0 || (int64_t)slot >= p.num_slots) return;
  const int64_t unit = (int64_t)slot * p.Hv + h;
  const RingPos rp = ring_pos(R, unit);
  const int st = rp.st, cnt = rp.cnt;
  const bool fold = (T > 0) ? (cnt + T > L) : (cnt > 0);
  if (!fold) return;

  ST* tile = static_cast<ST*>(p.pool) + unit * (int64_t)(D * D);
  const int c0 = (lane % LPR) * VEC;
  const int r0 = wave * RPW + lane / LPR;
  float s[PASSES][VEC];
#pragma unroll
  for (int pp = 0; pp < PASSES; ++pp) IO::widen(IO::load_raw(tile + (r0 + pp * NW * RPW) * D + c0), s[pp]);

  float* e_k = s_dyn;           // [L][LDE]
  float* e_v = e_k + L * LDE;   // [L][LDE]
  float* e_a = e_v + L * LDE;   // [L] exp(g)
  float* e_b = e_a + L;         // [L] beta
  const int64_t ring_e = unit * L;
  for (int t = tid; t < cnt; t += NTH) {
    const int j = (st + t) % L;
    e_a[t] = expf(R.g[ring_e + j]);
    e_b[t] = R.beta[ring_e + j];
  }
  for (int r0s = 0; r0s < cnt; r0s += kStageRows) {
    Stager sk, sv;
    auto ring_row = [&](int r) { return (ring_e + (st + r0s + r) % L) * D; };
    const int nr = min(kStageRows, cnt - r0s);
    sk.issue(R.k, nr, ring_row);
    sv.issue(R.v, nr, ring_row);
    sk.commit(e_k + r0s * LDE, LDE, p.in_dt, nr);
    sv.commit(e_v + r0s * LDE, LDE, p.in_dt, nr);
  }
  __syncthreads();

  for (int i = 0; i < cnt; ++i) {
    const float* ki = e_k + i * LDE;
    float kvp[VEC];
#pragma unroll
    for (int e = 0; e < VEC; ++e) kvp[e] = 0.f;
#pragma unroll
    for (int pp = 0; pp < PASSES; ++pp) {
      const float kr = ki[r0 + pp * NW * RPW];
#pragma unroll
      for (int e = 0; e < VEC; ++e) kvp[e] = fmaf(s[pp][e], kr, kvp[e]);
    }
    float* red = s_red[i & 1][0];  // double-buffered: one barrier per entry
#pragma unroll
    for (int e = 0; e < VEC; ++e) kvp[e] = xor_sum_from<LPR>(kvp[e]);
    if (lane < LPR) {
#pragma unroll
      for (int e = 0; e < VEC; ++e) red[wave * D + c0 + e] = kvp[e];
    }
    __syncthreads();
    const float al = e_a[i], be = e_b[i];
    float delta[VEC];
#pragma unroll
    for (int e = 0; e < VEC; ++e) {
      float kv = 0.f;
#pragma unroll
      for (int w = 0; w < NW; ++w) kv += red[w * D + c0 + e];
      delta[e] = be * (e_v[i * LDE + c0 + e] - al * kv);
    }
#pragma unroll
    for (int pp = 0; pp < PASSES; ++pp) {
      const float kr = ki[r0 + pp * NW * RPW];
#pragma unroll
      for (int e = 0; e < VEC; ++e) s[pp][e] = fmaf(al, s[pp][e], kr * delta[e]);
    }
  }
#pragma unroll
  for (int pp = 0; pp < PASSES; ++pp) IO::store(tile + (r0 + pp * NW * RPW) * D + c0, s[pp]);
  if (tid == 0) {
    R.start[unit] = (st + cnt) % L;
    R.count[unit] = 0;
  }
}

// ---------------------------------------------------------------- prep
// One wave per unit.  Loads are issued in two independent rounds: the window
// rows (which need only the row index) together with the slot, then the
// unit's whole ring block in ring order, its gates and its pointers (which
// need only the slot); the live entries are picked out of the block in LDS.
// Keys and values stay packed (input dtype) in LDS and are widened on use.
template <int EB>
struct PackedRow {
  // element c of a packed row (EB = 4: f32 words; EB = 2: bf16 / f16 pairs)
  __device__ __forceinline__ static float get(const uint32_t* row, int c, int dt) {
    if constexpr (EB == 4) {
      return __uint_as_float(row[c]);
    } else {
      const uint32_t w = row[c >> 1];
      const uint32_t h16 = (c & 1) ? (w >> 16) : (w & 0xffffu);
      return dt == GDN_BF16 ? bf16_bits_to_f32(h16) : f16_bits_to_f32(h16);
    }
  }
};

// One 16 x 16 tile of X Y^T over D columns on MFMA, X and Y packed rows in
// LDS (row stride ldw words); rows at or beyond nx / ny read as zero.  Lane l
// supplies X[l % 16][k-block l / 16] and Y[l % 16][same block]; element r of
// the result is (4 (l / 16) + r, l % 16).  16-bit rows use the gfx950
// 16x16x32 bf16 / f16 instructions (products of two 16-bit values are exact in
// FP32), f32 rows the 16x16x4 f32 one.
template <int D, int EB>
__device__ __forceinline__ f32x4 tile_xyt(const uint32_t* X, int nx, const uint32_t* Y, int ny, int ldw, int dt,
                                          int lane) {
  const int i = lane & 15, kb = lane >> 4;
  const bool xv = i < nx, yv = i < ny;
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
  if constexpr (EB == 2) {
    typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
    typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
#pragma unroll
    for (int s = 0; s < (D + 31) / 32; ++s) {
      const int w0 = 16 * s + 4 * kb;  // word of element 32 s + 8 kb; words past D / 2 read as zero
      const bool kv = w0 < D / 2;
      u32x4 a = {0u, 0u, 0u, 0u}, b = a;
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        if (xv && kv) a[w] = X[i * ldw + w0 + w];
        if (yv && kv) b[w] = Y[i * ldw + w0 + w];
      }
      if (dt == GDN_BF16)
        acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a), __builtin_bit_cast(bf16x8, b),
                                                      acc, 0, 0, 0);
      else
        acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8, a), __builtin_bit_cast(f16x8, b), acc,
                                                     0, 0, 0);
    }
  } else {
#pragma unroll 8
    for (int s = 0; s < D / 4; ++s) {
      const float a = xv ? __uint_as_float(X[i * ldw + 4 * s + kb]) : 0.f;
      const float b = yv ? __uint_as_float(Y[i * ldw + 4 * s + kb]) : 0.f;
      acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, acc, 0, 0, 0);
    }
  }
  return acc;
}

// Dynamic LDS of the prep kernel: packed keys and values [E][D * EB / 4 + 1]
// words each (E = L + T), packed window queries [T][...], then floats: gates
// (g, beta, prefix G) [E] each, Gram matrix [E][E], key / query products
// [E][T], coefficients c and e^G c [T][E] each.
__host__ __device__ inline size_t replay_prep_words(int D, int EB, int L, int T) {
  const size_t E = (size_t)L + (size_t)T, row = (size_t)D * EB / 4 + 1;
  return 2 * E * row + (size_t)T * row + 3 * E + E * E + 3 * E * T;
}
__host__ __device__ inline size_t replay_prep_lds_bytes(int D, int L, int T) {
  return replay_prep_words(D, 4, L, T) * sizeof(float);  // the f32-input size bounds both
}

template <int D, int EB>
__global__ void __launch_bounds__(64) gdn_replay_prep_kernel(const ReplayArgs P, float* __restrict__ ws) {
  constexpr int VE = 16 / EB;             // elements per 16-byte load
  constexpr int CPR = D / VE;             // 16-byte loads per row
  constexpr int LDW = D * EB / 4 + 1;     // LDS words per packed row (+1: bank spread)
  constexpr int RB = (64 / CPR) > 0 ? 64 / CPR : 1;  // rows per wave-wide load round
  static_assert(64 % CPR == 0, "a wave covers whole rows");
  using Row = PackedRow<EB>;
  extern __shared__ uint32_t s_words[];

  const DecodeArgs& p = P.d;
  const RingArgs& R = P.ring;
  const int T = P.T, L = R.L;
  const int lane = threadIdx.x;
  const int b = blockIdx.x / p.Hv;
  const int h = blockIdx.x - b * p.Hv;
  const int hk = h / (p.Hv / p.Hk);
  const int E = L + T;
  uint32_t* e_k = s_words;                  // [E][LDW] live order: committed, then window
  uint32_t* e_v = e_k + E * LDW;            // [E][LDW]
  uint32_t* e_q = e_v + E * LDW;            // [T][LDW]
  float* e_g = reinterpret_cast<float*>(e_q + T * LDW);  // [E]
  float* e_b = e_g + E;                     // [E]
  float* e_G = e_b + E;                     // [E]
  float* s_gram = e_G + E;                  // [E][E]
  float* s_kq = s_gram + E * E;             // [E][T]
  float* s_c = s_kq + E * T;                // [T][E]
  float* s_ec = s_c + T * E;                // [T][E]

  const int lr = lane / CPR, lc = (lane - lr * CPR) * VE;  // this lane's row offset and column in a round
  const char* kin = static_cast<const char*>(p.k);
  const char* vin = static_cast<const char*>(p.v);
  const char* qin = static_cast<const char*>(p.q);

  // Batches of 4 load rounds (RB rows each) through registers; `rowptr(r)`
  // gives the global address of row r, `dst(r)` its LDS row (or null to skip).
  auto load_batch = [&](int r0, int nrows, auto rowptr, u32x4 (&x)[4]) {
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int r = (r0 + u) * RB + lr;
      u32x4 z = {0u, 0u, 0u, 0u};
      if (r < nrows) z = *reinterpret_cast<const u32x4*>(rowptr(r) + lc * EB);
      x[u] = z;
    }
  };
  auto commit_batch = [&](int r0, int nrows, auto dst, const u32x4 (&x)[4]) {
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int r = (r0 + u) * RB + lr;
      uint32_t* d = (r < nrows) ? dst(r) : nullptr;
      if (d != nullptr) {
#pragma unroll
        for (int w = 0; w < 4; ++w) d[lc * EB / 4 + w] = x[u][w];
      }
    }
  };
  auto win_k = [&](int t) { return kin + (((int64_t)b * T + t) * p.Hk + hk) * D * EB; };
  auto win_v = [&](int t) { return vin + (((int64_t)b * T + t) * p.Hv + h) * D * EB; };
  auto win_q = [&](int t) { return qin + (((int64_t)b * T + t) * p.Hk + hk) * D * EB; };

  // ---- round 1: the slot, the first window rows and the window gate inputs
  const int slot = p.slot_map[b];
  u32x4 wk[4], wv[4], wq[4];
  load_batch(0, T, win_k, wk);
  load_batch(0, T, win_v, wv);
  load_batch(0, T, win_q, wq);
  float ga = 0.f, gb = 0.f;
  if (lane < T) {
    const int64_t gi = ((int64_t)b * T + lane) * p.Hv + h;
    ga = load_elem(p.a, gi, p.in_dt);
    gb = load_elem(p.b, gi, p.in_dt);
  }
  if (slot < 0 || (int64_t)slot >= p.num_slots) return;  // padded row (the stream kernel writes zeros)
  const int64_t unit = (int64_t)slot * p.Hv + h;

  // ---- round 2: the unit's whole ring block (ring order), its gates and pointers
  const int64_t ring_e = unit * L;
  const char* rk = static_cast<const char*>(R.k) + ring_e * D * EB;
  const char* rv = static_cast<const char*>(R.v) + ring_e * D * EB;
  auto ring_k = [&](int j) { return rk + (int64_t)j * D * EB; };
  auto ring_v = [&](int j) { return rv + (int64_t)j * D * EB; };
  u32x4 xk[4], xv[4];
  load_batch(0, L, ring_k, xk);
  load_batch(0, L, ring_v, xv);
  float rg = 0.f, rb = 0.f;
  if (lane < L) {
    rg = R.g[ring_e + lane];
    rb = R.beta[ring_e + lane];
  }
  const RingPos rp = ring_pos(R, unit);
  const int st = rp.st;
  const int cnt = min(rp.cnt, L - T);  // the fold kernel left room for the window

  // ---- commit in live order: committed entries 0..cnt-1, then the window
  auto live_k = [&](int j) -> uint32_t* {  // ring index j -> its live row, if live
    const int live = (j - st + L) % L;
    return live < cnt ? e_k + live * LDW : nullptr;
  };
  auto live_v = [&](int j) -> uint32_t* {
    const int live = (j - st + L) % L;
    return live < cnt ? e_v + live * LDW : nullptr;
  };
  auto wdst_k = [&](int t) -> uint32_t* { return e_k + (cnt + t) * LDW; };
  auto wdst_v = [&](int t) -> uint32_t* { return e_v + (cnt + t) * LDW; };
  auto wdst_q = [&](int t) -> uint32_t* { return e_q + t * LDW; };
  commit_batch(0, T, wdst_k, wk);
  commit_batch(0, T, wdst_v, wv);
  commit_batch(0, T, wdst_q, wq);
  commit_batch(0, L, live_k, xk);
  commit_batch(0, L, live_v, xv);
  for (int r0 = 4; r0 * RB < T; r0 += 4) {  // longer windows
    load_batch(r0, T, win_k, wk);
    load_batch(r0, T, win_v, wv);
    load_batch(r0, T, win_q, wq);
    commit_batch(r0, T, wdst_k, wk);
    commit_batch(r0, T, wdst_v, wv);
    commit_batch(r0, T, wdst_q, wq);
  }
  for (int r0 = 4; r0 * RB < L; r0 += 4) {  // longer rings
    load_batch(r0, L, ring_k, xk);
    load_batch(r0, L, ring_v, xv);
    commit_batch(r0, L, live_k, xk);
    commit_batch(r0, L, live_v, xv);
  }
  // gates in live order: committed from the ring block, the window from its inputs
  if (lane < L) {
    const int live = (lane - st + L) % L;
    if (live < cnt) {
      e_g[live] = rg;
      e_b[live] = rb;
    }
  }
  float wg = 0.f, wbeta = 0.f;
  if (lane < T) {
    wg = gate_g(ga, p.A_log[h], p.dt_bias[h]);
    wbeta = sigmoid_f(gb);
    e_g[cnt + lane] = wg;
    e_b[cnt + lane] = wbeta;
  }
  __syncthreads();

  // ---- append the window to the ring (raw input bytes) and move the pointers
  const int base = (st + cnt) % L;
  {
    const char* kin2 = static_cast<const char*>(p.k);
    for (int x = lane; x < T * CPR; x += 64) {
      const int t = x / CPR, c = (x - t * CPR) * VE;
      const int64_t j = ring_e + (base + t) % L;
      const int64_t ko = ((((int64_t)b * T + t) * p.Hk + hk) * D + c) * EB;
      const int64_t vo = ((((int64_t)b * T + t) * p.Hv + h) * D + c) * EB;
      *reinterpret_cast<u32x4*>(static_cast<char*>(R.k) + (j * D + c) * EB) =
          *reinterpret_cast<const u32x4*>(kin2 + ko);
      *reinterpret_cast<u32x4*>(static_cast<char*>(R.v) + (j * D + c) * EB) =
          *reinterpret_cast<const u32x4*>(vin + vo);
    }
    if (lane < T) {
      const int64_t j = ring_e + (base + lane) % L;
      R.g[j] = wg;
      R.beta[j] = wbeta;
    }
    if (lane == 0) {
      R.start[unit] = st;
      R.count[unit] = cnt + T;
    }
  }

  // ---- prefix sums of g over the live entries
  const int n_all = cnt + T;
  {
    float x = (lane < n_all) ? e_g[lane] : 0.f;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
      const float y = __shfl_up(x, off, 64);
      if (lane >= off) x += y;
    }
    if (lane < n_all) e_G[lane] = x;
  }
  // ---- Gram matrix of the live keys and key / query products, 16 x 16 MFMA tiles
  {
    const int nt = (n_all + 15) >> 4, qt = (T + 15) >> 4;
    const int i4 = 4 * (lane >> 4), jc = lane & 15;
    for (int I = 0; I < nt; ++I) {
      for (int J = I; J < nt; ++J) {
        const f32x4 g = tile_xyt<D, EB>(e_k + 16 * I * LDW, n_all - 16 * I, e_k + 16 * J * LDW, n_all - 16 * J, LDW,
                                        p.in_dt, lane);
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int i = 16 * I + i4 + r, j = 16 * J + jc;
          if (i < n_all && j < n_all) s_gram[i * E + j] = g[r];
        }
      }
      for (int J = 0; J < qt; ++J) {
        const f32x4 g = tile_xyt<D, EB>(e_k + 16 * I * LDW, n_all - 16 * I, e_q + 16 * J * LDW, T - 16 * J, LDW,
                                        p.in_dt, lane);
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int i = 16 * I + i4 + r, t = 16 * J + jc;
          if (i < n_all && t < T) s_kq[i * T + t] = g[r];
        }
      }
    }
  }
  __syncthreads();

  // ---- back substitution for each window position: lane j holds the residual of live entry j
  for (int t = 0; t < T; ++t) {
    const int e_last = cnt + t;
    const float Gn = e_G[e_last];
    const int j = lane;
    const bool live = j <= e_last;
    const float Gj = live ? e_G[j] : 0.f;
    float r = live ? expf(Gn - Gj) * s_kq[j * T + t] : 0.f;
    float cj = 0.f;
    for (int i = e_last; i >= 0; --i) {
      // c_i = beta_i * residual_i, then every earlier entry drops its term
      const float ci =
          __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, e_b[i] * r), i));
      if (j == i) cj = ci;
      if (live && j < i) r = fmaf(-expf(e_G[i] - Gj) * s_gram[j * E + i], ci, r);
    }
    if (live) {
      s_c[t * E + j] = cj;
      s_ec[t * E + j] = expf(Gj) * cj;
    }
  }
  __syncthreads();
  // ---- w_t = e^{G_n} q_t - sum_j e^{G_j} c_j k_j and acc_t = sum_j c_j v_j, to the workspace
  float* wsu = ws + ((int64_t)b * p.Hv + h) * T * 2 * D;
  for (int x = lane; x < T * D; x += 64) {
    const int t = x / D, c = x - t * D;
    const int e_last = cnt + t;
    float w = expf(e_G[e_last]) * Row::get(e_q + t * LDW, c, p.in_dt);
    float acc = 0.f;
    for (int jj = 0; jj <= e_last; ++jj) {
      w = fmaf(-s_ec[t * E + jj], Row::get(e_k + jj * LDW, c, p.in_dt), w);
      acc = fmaf(s_c[t * E + jj], Row::get(e_v + jj * LDW, c, p.in_dt), acc);
    }
    wsu[(2 * t) * D + c] = w;
    wsu[(2 * t + 1) * D + c] = acc;
  }
}

// ---------------------------------------------------------------- stream
template <int SDT, int D, bool NT, int TB>
__global__ void __launch_bounds__((ReplayGeom<SDT, D>::NW * 64))
gdn_replay_stream_kernel(const ReplayArgs P, const float* __restrict__ ws) {
  using G = ReplayGeom<SDT, D>;
  constexpr int VEC = G::VEC, LPR = G::LPR, RPW = G::RPW, NW = G::NW, PASSES = G::PASSES;
  constexpr int NTH = NW * 64;
  using IO = TileIO<SDT, VEC, NT>;
  using ST = typename StateElem<SDT>::T;
  extern __shared__ float s_w[];  // [T][D]
  __shared__ float s_out[TB][NW][D];

  const DecodeArgs& p = P.d;
  const int T = P.T;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int b = blockIdx.x / p.Hv;
  const int h = blockIdx.x - b * p.Hv;
  const int slot = p.slot_map[b];
  if (slot < 0 || (int64_t)slot >= p.num_slots) {  // padded row
    for (int i = tid; i < T * D; i += NTH) {
      const int t = i / D, c = i - t * D;
      store_elem(p.out, (((int64_t)b * T + t) * p.Hv + h) * D + c, 0.f, p.out_dt);
    }
    return;
  }
  const ST* tile = static_cast<const ST*>(p.pool) + ((int64_t)slot * p.Hv + h) * (int64_t)(D * D);
  const int c0 = (lane % LPR) * VEC;
  const int r0 = wave * RPW + lane / LPR;
  typename IO::Raw raw[PASSES];
#pragma unroll
  for (int pp = 0; pp < PASSES; ++pp) raw[pp] = IO::load_raw(tile + (r0 + pp * NW * RPW) * D + c0);
  const float* wsu = ws + ((int64_t)b * p.Hv + h) * T * 2 * D;
  for (int i = tid; i < T * D; i += NTH) {
    const int t = i / D, c = i - t * D;
    s_w[t * D + c] = wsu[2 * t * D + c];
  }
  __syncthreads();

  for (int t0 = 0; t0 < T; t0 += TB) {
    const int nt = (T - t0) < TB ? (T - t0) : TB;
    float part[TB][VEC];
#pragma unroll
    for (int tb = 0; tb < TB; ++tb)
#pragma unroll
      for (int e = 0; e < VEC; ++e) part[tb][e] = 0.f;
#pragma unroll
    for (int pp = 0; pp < PASSES; ++pp) {
      const int r = r0 + pp * NW * RPW;
      float sv[VEC];
      IO::widen(raw[pp], sv);
#pragma unroll
      for (int tb = 0; tb < TB; ++tb) {
        if (tb < nt) {
          const float wr = s_w[(t0 + tb) * D + r];
#pragma unroll
          for (int e = 0; e < VEC; ++e) part[tb][e] = fmaf(sv[e], wr, part[tb][e]);
        }
      }
    }
#pragma unroll
    for (int tb = 0; tb < TB; ++tb) {
      if (tb < nt) {
#pragma unroll
        for (int e = 0; e < VEC; ++e) part[tb][e] = xor_sum_from<LPR>(part[tb][e]);
        if (lane < LPR) {
#pragma unroll
          for (int e = 0; e < VEC; ++e) s_out[tb][wave][c0 + e] = part[tb][e];
        }
      }
    }
    __syncthreads();
    for (int i = tid; i < nt * D; i += NTH) {
      const int tb = i / D, c = i - tb * D;
      float o = wsu[(2 * (t0 + tb) + 1) * D + c];
#pragma unroll
      for (int w = 0; w < NW; ++w) o += s_out[tb][w][c];
      store_elem(p.out, (((int64_t)b * T + t0 + tb) * p.Hv + h) * D + c, p.scale * o, p.out_dt);
    }
    __syncthreads();
  }
}

// ---------------------------------------------------------------- rollback
__global__ void gdn_replay_rollback_kernel(const ReplayArgs P) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const DecodeArgs& p = P.d;
  if (i >= (int64_t)p.B * p.Hv) return;
  const int b = (int)(i / p.Hv);
  const int h = (int)(i - (int64_t)b * p.Hv);
  const int slot = p.slot_map[b];
  if (slot < 0 || (int64_t)slot >= p.num_slots) return;
  int r = P.num_rejected[b];
  r = r < 0 ? 0 : r;
  int32_t* cnt = P.ring.count + (int64_t)slot * p.Hv + h;
  const int c = *cnt - r;
  *cnt = c < 0 ? 0 : c;
}

// ---------------------------------------------------------------- launchers
template <int SDT, int D, int EB>
static hipError_t launch_fold(const ReplayArgs& a, hipStream_t s) {
  using G = ReplayGeom<SDT, D>;
  constexpr bool NT = (SDT == GDN_F32) && (GDN_REPLAY_NT_F32 != 0);
  const unsigned grid = (unsigned)((int64_t)a.d.B * a.d.Hv);
  const size_t lds = replay_fold_lds_bytes(D, a.ring.L);
  hipLaunchKernelGGL((gdn_replay_fold_kernel<SDT, D, NT, EB>), dim3(grid), dim3(G::NW * 64), lds, s, a);
  return hipGetLastError();
}

template <int SDT, int D>
static hipError_t launch_replay_t(const ReplayArgs& a, float* ws, hipStream_t s) {
  using G = ReplayGeom<SDT, D>;
  constexpr bool NT = (SDT == GDN_F32) && (GDN_REPLAY_NT_F32 != 0);
  const bool f32_in = a.d.in_dt == GDN_F32;
  hipError_t e = f32_in ? launch_fold<SDT, D, 4>(a, s) : launch_fold<SDT, D, 2>(a, s);
  if (e != hipSuccess || a.T == 0) return e;
  const unsigned grid = (unsigned)((int64_t)a.d.B * a.d.Hv);
  if (f32_in)
    hipLaunchKernelGGL((gdn_replay_prep_kernel<D, 4>), dim3(grid), dim3(64),
                       replay_prep_words(D, 4, a.ring.L, a.T) * sizeof(float), s, a, ws);
  else
    hipLaunchKernelGGL((gdn_replay_prep_kernel<D, 2>), dim3(grid), dim3(64),
                       replay_prep_words(D, 2, a.ring.L, a.T) * sizeof(float), s, a, ws);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  const size_t lds_w = (size_t)a.T * D * sizeof(float);
  if (a.T <= 1)
    hipLaunchKernelGGL((gdn_replay_stream_kernel<SDT, D, NT, 1>), dim3(grid), dim3(G::NW * 64), lds_w, s, a, ws);
  else
    hipLaunchKernelGGL((gdn_replay_stream_kernel<SDT, D, NT, kStreamTB>), dim3(grid), dim3(G::NW * 64), lds_w, s, a,
                       ws);
  return hipGetLastError();
}

template <int SDT>
static hipError_t launch_replay_sdt(const ReplayArgs& a, int D, float* ws, hipStream_t s) {
  switch (D) {
    case 16: return launch_replay_t<SDT, 16>(a, ws, s);
    case 32: return launch_replay_t<SDT, 32>(a, ws, s);
    case 64: return launch_replay_t<SDT, 64>(a, ws, s);
    case 128: return launch_replay_t<SDT, 128>(a, ws, s);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_replay(const ReplayArgs& a, int state_dt, int D, float* ws, hipStream_t s) {
  if (a.d.B == 0) return hipSuccess;
  switch (state_dt) {
    case GDN_F32: return launch_replay_sdt<GDN_F32>(a, D, ws, s);
    case GDN_BF16: return launch_replay_sdt<GDN_BF16>(a, D, ws, s);
    case GDN_F16: return launch_replay_sdt<GDN_F16>(a, D, ws, s);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_replay_flush(const ReplayArgs& a, int state_dt, int D, hipStream_t s) {
  ReplayArgs f = a;
  f.T = 0;
  return launch_replay(f, state_dt, D, nullptr, s);
}

hipError_t launch_replay_rollback(const ReplayArgs& a, hipStream_t s) {
  if (a.d.B == 0) return hipSuccess;
  const int64_t n = (int64_t)a.d.B * a.d.Hv;
  const unsigned grid = (unsigned)((n + 255) / 256);
  hipLaunchKernelGGL(gdn_replay_rollback_kernel, dim3(grid), dim3(256), 0, s, a);
  return hipGetLastError();
}

size_t replay_lds_total(int D, int L, int T) {
  const size_t prep = T > 0 ? replay_prep_lds_bytes(D, L, T) : 0;
  const size_t fold = replay_fold_lds_bytes(D, L) + 2 * 8 * (size_t)D * sizeof(float);
  return prep > fold ? prep : fold;
}

}  // namespace gdn
