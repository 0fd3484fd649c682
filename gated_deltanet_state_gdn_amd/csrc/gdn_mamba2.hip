// Mamba2 selective-state decode and its ReplaySSM form (AREX ReplaySSM
// article: "bottleneck" section, the (nheads, d, n) state read and written
// every step; "cache inputs, not state" section, a checkpoint plus a ring of
// the state-building inputs x, B and dt, C never cached; "numbers" section,
// the per-step figures were measured on Mamba2).  Per head h of group
// gr = h / (H / G), with dt' = softplus(dt + dt_bias[h]) and
// g = -exp(A_log[h]) dt' (Dao and Gu's selective state-space update):
//     S <- exp(g) S + dt' x B^T              (S is d x n, n fastest)
//     y  = S C + D[h] x
// Replay: with G_i the prefix sums of g over the live entries, window
// position t (last live entry e) outputs
//     y_t = e^{G_e} S0 C_t + sum_{j <= e} e^{G_e - G_j} dt'_j (B_j . C_t) x_j + D x_t
// (no delta-rule correction, so no back substitution), and a fold is one
// rank-n update  S0 <- e^{G_c} S0 + sum_j e^{G_c - G_j} dt'_j x_j B_j^T.
//
// Ring pointers are per slot: every head of a slot advances together.  The
// fold and step kernels only read them; a one-thread-per-row kernel moves
// them after the step, so no workgroup ever races another on them.
#include "gdn_device.h"
#include "gdn_launch.h"

#ifndef GDN_M2_NT_F32
#define GDN_M2_NT_F32 1
#endif

namespace gdn {

// d x n tile: each lane owns VEC consecutive columns of one row per pass; LPR
// lanes cover a row, a wave RPW rows per pass, NW waves, PASSES passes.
template <int DT, int ROWS, int COLS, int MAXW>
struct M2Geom {
  static constexpr int BYTES = StateElem<DT>::BYTES;
  static constexpr int VEC0 = 16 / BYTES;
  static constexpr int VEC = (64 / (COLS / VEC0) > ROWS) ? VEC0 / 2 : VEC0;
  static constexpr int LPR = COLS / VEC;
  static constexpr int RPW = 64 / LPR;
  static constexpr int NW = (ROWS / RPW) >= MAXW ? MAXW : (ROWS / RPW);
  static constexpr int PASSES = ROWS / (RPW * NW);
  static_assert(LPR * VEC == COLS && LPR * RPW == 64 && PASSES * RPW * NW == ROWS, "tile geometry");
};

template <int SDT, int P, int N>
using M2G = M2Geom<SDT, P, N, SDT == GDN_F32 ? 4 : 2>;

// Sum over the lanes of one row (lanes that differ only in bits < log2(LPR)).
template <int LPR>
__device__ __forceinline__ float row_sum(float x) {
#pragma unroll
  for (int off = 1; off < LPR; off <<= 1) x += __shfl_xor(x, off, 64);
  return x;
}

struct M2Pos {
  int st, cnt;  // pointers after any fold this step performs
  bool fold;
};

// Pointers as the step sees them: a fold (count + T > L; the flush, T == 0,
// folds any non-empty ring) empties the ring first.
__device__ __forceinline__ M2Pos m2_pos(const M2Args& a, int64_t slot) {
  const int L = a.L;
  int st = a.start[slot], cnt = a.count[slot];
  st = ((st % L) + L) % L;
  cnt = cnt < 0 ? 0 : (cnt > L ? L : cnt);
  const bool fold = a.T > 0 ? (cnt + a.T > L) : (cnt > 0);
  if (fold) return M2Pos{(st + cnt) % L, 0, true};
  return M2Pos{st, cnt, false};
}

// ---------------------------------------------------------------- decode
template <int SDT, int P, int N, bool NT>
__global__ void __launch_bounds__((M2G<SDT, P, N>::NW * 64)) gdn_m2_decode_kernel(const M2Args a) {
  using G = M2G<SDT, P, N>;
  constexpr int VEC = G::VEC, LPR = G::LPR, RPW = G::RPW, NW = G::NW, PASSES = G::PASSES;
  using IO = TileIO<SDT, VEC, NT>;
  using ST = typename StateElem<SDT>::T;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int b = blockIdx.x / a.H, h = blockIdx.x - (blockIdx.x / a.H) * a.H;
  const int gr = h / (a.H / a.G);
  const int c0 = (lane % LPR) * VEC;
  const int r0 = wave * RPW + lane / LPR;
  const int64_t yb = ((int64_t)b * a.H + h) * P;
  const int slot = a.slot_map[b];
  if (slot < 0 || (int64_t)slot >= a.num_slots) {  // padded row
    for (int i = threadIdx.x; i < P; i += NW * 64) store_elem(a.y, yb + i, 0.f, a.out_dt);
    return;
  }
  ST* tile = static_cast<ST*>(a.pool) + ((int64_t)slot * a.H + h) * (int64_t)(P * N);
  typename IO::Raw raw[PASSES];
#pragma unroll
  for (int pp = 0; pp < PASSES; ++pp) raw[pp] = IO::load_raw(tile + (r0 + pp * NW * RPW) * N + c0);

  const float dtp = softplus_f(load_elem(a.dt, (int64_t)b * a.H + h, a.in_dt) + a.dt_bias[h]);
  const float alpha = expf(-expf(a.A_log[h]) * dtp);
  const float Dh = a.Dskip[h];
  const int64_t bc = ((int64_t)b * a.G + gr) * N + c0;
  float Bc[VEC], Cc[VEC];
#pragma unroll
  for (int e = 0; e < VEC; ++e) {
    Bc[e] = dtp * load_elem(a.Bm, bc + e, a.in_dt);
    Cc[e] = load_elem(a.Cm, bc + e, a.in_dt);
  }
#pragma unroll
  for (int pp = 0; pp < PASSES; ++pp) {
    const int r = r0 + pp * NW * RPW;
    const float xr = load_elem(a.x, yb + r, a.in_dt);
    float s[VEC];
    IO::widen(raw[pp], s);
    float part = 0.f;
#pragma unroll
    for (int e = 0; e < VEC; ++e) {
      s[e] = fmaf(alpha, s[e], xr * Bc[e]);
      part = fmaf(s[e], Cc[e], part);
    }
    IO::store(tile + r * N + c0, s);
    part = row_sum<LPR>(part);
    if ((lane % LPR) == 0) store_elem(a.y, yb + r, fmaf(Dh, xr, part), a.out_dt);
  }
}

// ---------------------------------------------------------------- fold
// Persistent: workgroup w owns units w, w + Gd, ... (Gd the grid size), checks
// 64 at a time (one per lane of wave 0) and folds those whose slot folds this
// step, one after another.  Pointers are left to the advance kernel.
// Dynamic LDS (floats): x rows [L][P], B rows [L][N], weights [L].
template <int SDT, int P, int N, bool NT>
__global__ void __launch_bounds__((M2G<SDT, P, N>::NW * 64)) gdn_m2_fold_kernel(const M2Args a) {
  using G = M2G<SDT, P, N>;
  constexpr int VEC = G::VEC, LPR = G::LPR, RPW = G::RPW, NW = G::NW, PASSES = G::PASSES;
  constexpr int NTH = NW * 64;
  using IO = TileIO<SDT, VEC, NT>;
  using ST = typename StateElem<SDT>::T;
  extern __shared__ float s_dyn[];
  __shared__ int s_list[64];
  __shared__ int s_n;
  __shared__ float s_decay;
  const int L = a.L;
  float* ex = s_dyn;             // [L][P]
  float* eB = ex + L * P;        // [L][N]
  float* ew = eB + L * N;        // [L] e^{G_c - G_j} dt'_j
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int c0 = (lane % LPR) * VEC;
  const int r0 = wave * RPW + lane / LPR;
  const int units = a.B * a.H;
  const int grid_n = gridDim.x;

  for (int64_t j0 = 0; blockIdx.x + j0 * grid_n < units; j0 += 64) {
    if (wave == 0) {
      const int64_t xl = blockIdx.x + (j0 + lane) * grid_n;
      const int x = xl < units ? (int)xl : units;
      bool need = false;
      if (x < units) {
        const int slot = a.slot_map[x / a.H];
        if (slot >= 0 && (int64_t)slot < a.num_slots) {
          const int cnt = a.count[slot];
          need = a.T > 0 ? (cnt + a.T > L) : (cnt > 0);
        }
      }
      const uint64_t mask = __ballot(need);
      if (need) s_list[__builtin_amdgcn_mbcnt_hi((uint32_t)(mask >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)mask, 0))] = x;
      if (lane == 0) s_n = __popcll(mask);
    }
    __syncthreads();
    const int n_fold = s_n;
    for (int f = 0; f < n_fold; ++f) {
      const int x = s_list[f];
      const int b = x / a.H, h = x - (x / a.H) * a.H;
      const int gr = h / (a.H / a.G);
      const int64_t slot = a.slot_map[b];
      int st = a.start[slot], cnt = a.count[slot];
      st = ((st % L) + L) % L;
      cnt = cnt < 0 ? 0 : (cnt > L ? L : cnt);

      int lane_off = r0 * N + c0;
      asm volatile("" : "+v"(lane_off));
      ST* tile = static_cast<ST*>(a.pool) + (slot * a.H + h) * (int64_t)(P * N) + lane_off;
      typename IO::Raw raw[PASSES];
#pragma unroll
      for (int pp = 0; pp < PASSES; ++pp) raw[pp] = IO::load_raw(tile + pp * NW * RPW * N);

      // committed entries in live order, widened
      const int64_t rh = (slot * a.H + h) * L, rg = (slot * a.G + gr) * L;
      for (int i = tid; i < cnt * P; i += NTH) {
        const int e = i / P, c = i - e * P;
        ex[i] = load_elem(a.rx, (rh + (st + e) % L) * P + c, a.in_dt);
      }
      for (int i = tid; i < cnt * N; i += NTH) {
        const int e = i / N, c = i - e * N;
        eB[i] = load_elem(a.rB, (rg + (st + e) % L) * N + c, a.in_dt);
      }
      if (wave == 0) {  // weights e^{G_c - G_j} dt'_j from a suffix sum of g, and the decay e^{G_c}
        const int j = lane;
        const float gj = j < cnt ? a.rg[rh + (st + j) % L] : 0.f;
        float suf = gj;  // sum of g over entries j..cnt-1
#pragma unroll
        for (int off = 1; off < 64; off <<= 1) {
          const float y = __shfl_down(suf, off, 64);
          if (j + off < 64) suf += y;
        }
        if (j < cnt) ew[j] = expf(suf - gj) * a.rdtp[rh + (st + j) % L];
        const float total = __shfl(suf, 0, 64);
        if (j == 0) s_decay = expf(total);
      }
      __syncthreads();
      const float decay = s_decay;
#pragma unroll
      for (int pp = 0; pp < PASSES; ++pp) {
        const int r = r0 + pp * NW * RPW;
        float s[VEC];
        IO::widen(raw[pp], s);
#pragma unroll
        for (int e = 0; e < VEC; ++e) s[e] *= decay;
        for (int j = 0; j < cnt; ++j) {
          const float cx = ew[j] * ex[j * P + r];
#pragma unroll
          for (int e = 0; e < VEC; ++e) s[e] = fmaf(cx, eB[j * N + c0 + e], s[e]);
        }
        IO::store(tile + pp * NW * RPW * N, s);
      }
      __syncthreads();  // LDS staging is reused by the next unit
    }
    __syncthreads();  // s_list is rewritten by the next check
  }
}

// ---------------------------------------------------------------- step
// One workgroup per (sequence, head): outputs of the T window positions from
// the checkpoint and the ring, and the window appended to the ring (x, g, dt'
// per head; B once per group, by the group's first head).
// Dynamic LDS (floats): ring block x [L][P] and B [L][N] (ring order), window
// x [T][P], B [T][N], C [T][N], prefix sums G [L], dt' [L], weights [T][L].
__host__ __device__ inline size_t m2_step_floats(int P, int N, int L, int T) {
  return (size_t)L * P + (size_t)L * N + (size_t)T * P + 2 * (size_t)T * N + 2 * (size_t)L + (size_t)T * L;
}

template <int SDT, int P, int N, bool NT>
__global__ void __launch_bounds__((M2G<SDT, P, N>::NW * 64)) gdn_m2_step_kernel(const M2Args a) {
  using G = M2G<SDT, P, N>;
  constexpr int VEC = G::VEC, LPR = G::LPR, RPW = G::RPW, NW = G::NW, PASSES = G::PASSES;
  constexpr int NTH = NW * 64;
  using IO = TileIO<SDT, VEC, NT>;
  using ST = typename StateElem<SDT>::T;
  extern __shared__ float s_dyn[];
  const int L = a.L, T = a.T;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int b = blockIdx.x / a.H, h = blockIdx.x - (blockIdx.x / a.H) * a.H;
  const int gr = h / (a.H / a.G);
  const bool leader = (h % (a.H / a.G)) == 0;
  const int c0 = (lane % LPR) * VEC;
  const int r0 = wave * RPW + lane / LPR;
  const int slot = a.slot_map[b];
  if (slot < 0 || (int64_t)slot >= a.num_slots) {  // padded row
    for (int i = tid; i < T * P; i += NTH) {
      const int t = i / P, c = i - t * P;
      store_elem(a.y, (((int64_t)b * T + t) * a.H + h) * P + c, 0.f, a.out_dt);
    }
    return;
  }
  const ST* tile = static_cast<const ST*>(a.pool) + ((int64_t)slot * a.H + h) * (int64_t)(P * N);
  typename IO::Raw raw[PASSES];
#pragma unroll
  for (int pp = 0; pp < PASSES; ++pp) raw[pp] = IO::load_raw(tile + (r0 + pp * NW * RPW) * N + c0);

  float* rx = s_dyn;              // [L][P] ring order
  float* rB = rx + L * P;         // [L][N]
  float* wx = rB + L * N;         // [T][P]
  float* wB = wx + T * P;         // [T][N]
  float* wC = wB + T * N;         // [T][N]
  float* eG = wC + T * N;         // [L] prefix sums of g, live order
  float* ed = eG + L;             // [L] dt', live order
  float* ew = ed + L;             // [T][L] weights e^{G_e - G_j} dt'_j (B_j . C_t)

  const M2Pos pos = m2_pos(a, slot);
  const int st = pos.st, cnt = pos.cnt, n_all = cnt + T;  // n_all <= L
  const int64_t rh = ((int64_t)slot * a.H + h) * L, rgp = ((int64_t)slot * a.G + gr) * L;
  for (int i = tid; i < cnt * P; i += NTH) {
    const int e = i / P, c = i - e * P;
    const int j = (st + e) % L;
    rx[j * P + c] = load_elem(a.rx, (rh + j) * P + c, a.in_dt);
  }
  for (int i = tid; i < cnt * N; i += NTH) {
    const int e = i / N, c = i - e * N;
    const int j = (st + e) % L;
    rB[j * N + c] = load_elem(a.rB, (rgp + j) * N + c, a.in_dt);
  }
  for (int i = tid; i < T * P; i += NTH) {
    const int t = i / P, c = i - t * P;
    const int64_t src = (((int64_t)b * T + t) * a.H + h) * P + c;
    wx[i] = load_elem(a.x, src, a.in_dt);
    copy_elem(a.rx, (rh + (st + cnt + t) % L) * P + c, a.x, src, a.in_dt);  // append x
  }
  for (int i = tid; i < T * N; i += NTH) {
    const int t = i / N, c = i - t * N;
    const int64_t src = (((int64_t)b * T + t) * a.G + gr) * N + c;
    wB[i] = load_elem(a.Bm, src, a.in_dt);
    wC[i] = load_elem(a.Cm, src, a.in_dt);
    if (leader) copy_elem(a.rB, (rgp + (st + cnt + t) % L) * N + c, a.Bm, src, a.in_dt);  // append B
  }
  if (wave == 0) {
    // lane j takes live entry j: committed from ring position (st + j) % L, or window position j - cnt
    const int j = lane;
    float gj = 0.f, dj = 0.f;
    if (j < cnt) {
      gj = a.rg[rh + (st + j) % L];
      dj = a.rdtp[rh + (st + j) % L];
    } else if (j < n_all) {
      const int t = j - cnt;
      dj = softplus_f(load_elem(a.dt, ((int64_t)b * T + t) * a.H + h, a.in_dt) + a.dt_bias[h]);
      gj = -expf(a.A_log[h]) * dj;
      const int64_t dst = rh + (st + cnt + t) % L;  // append g and dt'
      a.rg[dst] = gj;
      a.rdtp[dst] = dj;
    }
    float G_ = gj;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
      const float y = __shfl_up(G_, off, 64);
      if (j >= off) G_ += y;
    }
    if (j < L) {
      eG[j] = G_;
      ed[j] = dj;
    }
  }
  __syncthreads();
  // weights: one thread per (t, j <= cnt + t)
  for (int i = tid; i < T * L; i += NTH) {
    const int t = i / L, j = i - t * L;
    const int e_last = cnt + t;
    float w = 0.f;
    if (j <= e_last) {
      const float* Bj = j < cnt ? rB + ((st + j) % L) * N : wB + (j - cnt) * N;
      const float* Ct = wC + t * N;
      float dot = 0.f;
      for (int c = 0; c < N; ++c) dot = fmaf(Bj[c], Ct[c], dot);
      w = expf(eG[e_last] - eG[j]) * ed[j] * dot;
    }
    ew[i] = w;
  }
  __syncthreads();
  // outputs: y_t[r] = e^{G_e} (S0 C_t)[r] + sum_j w_tj x_j[r] + D x_t[r]
  const float Dh = a.Dskip[h];
  for (int t = 0; t < T; ++t) {
    const int e_last = cnt + t;
    const float decay = expf(eG[e_last]);
    float Cc[VEC];
#pragma unroll
    for (int e = 0; e < VEC; ++e) Cc[e] = wC[t * N + c0 + e];
#pragma unroll
    for (int pp = 0; pp < PASSES; ++pp) {
      const int r = r0 + pp * NW * RPW;
      float s[VEC];
      IO::widen(raw[pp], s);
      float part = 0.f;
#pragma unroll
      for (int e = 0; e < VEC; ++e) part = fmaf(s[e], Cc[e], part);
      part = row_sum<LPR>(part);
      if ((lane % LPR) == 0) {
        float yv = decay * part;
        for (int j = 0; j <= e_last; ++j) {
          const float xj = j < cnt ? rx[((st + j) % L) * P + r] : wx[(j - cnt) * P + r];
          yv = fmaf(ew[t * L + j], xj, yv);
        }
        yv = fmaf(Dh, wx[t * P + r], yv);
        store_elem(a.y, (((int64_t)b * T + t) * a.H + h) * P + r, yv, a.out_dt);
      }
    }
  }
}

// ---------------------------------------------------------------- pointers
// One thread per batch row.  mode 0: a step of T tokens (fold if count + T > L,
// then count += T); mode 1: flush (fold any non-empty ring); mode 2: rollback.
__global__ void __launch_bounds__(256) gdn_m2_advance_kernel(const M2Args a, int mode) {
  const int b = blockIdx.x * blockDim.x + threadIdx.x;
  if (b >= a.B) return;
  const int slot = a.slot_map[b];
  if (slot < 0 || (int64_t)slot >= a.num_slots) return;
  if (mode == 2) {
    const int c = a.count[slot] - a.num_rejected[b];
    a.count[slot] = c > 0 ? c : 0;
    return;
  }
  const M2Pos pos = m2_pos(a, slot);
  a.start[slot] = pos.st;
  a.count[slot] = mode == 0 ? pos.cnt + a.T : pos.cnt;
}

// ---------------------------------------------------------------- launchers
template <int SDT, int P, int N>
static hipError_t m2_launch_t(const M2Args& a, int what, hipStream_t s) {
  using G = M2G<SDT, P, N>;
  constexpr bool NT = (SDT == GDN_F32) && (GDN_M2_NT_F32 != 0);
  const unsigned units = (unsigned)((int64_t)a.B * a.H);
  if (what == 0) {
    hipLaunchKernelGGL((gdn_m2_decode_kernel<SDT, P, N, NT>), dim3(units), dim3(G::NW * 64), 0, s, a);
    return hipGetLastError();
  }
  // fold (persistent, sized to the resident workgroups)
  const size_t fold_lds = ((size_t)a.L * (P + N + 1)) * sizeof(float);
  int per_cu = 0, cus = 0;
  hipError_t e = resident_blocks(reinterpret_cast<const void*>(&gdn_m2_fold_kernel<SDT, P, N, NT>), G::NW * 64,
                                 fold_lds, &per_cu);
  if (e == hipSuccess) e = device_cus(&cus);
  if (e != hipSuccess) return e;
  const int64_t fill = (int64_t)(per_cu > 0 ? per_cu : 1) * cus;
  hipLaunchKernelGGL((gdn_m2_fold_kernel<SDT, P, N, NT>), dim3((unsigned)(units < fill ? units : fill)),
                     dim3(G::NW * 64), fold_lds, s, a);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  if (a.T > 0) {
    hipLaunchKernelGGL((gdn_m2_step_kernel<SDT, P, N, NT>), dim3(units), dim3(G::NW * 64),
                       m2_step_floats(P, N, a.L, a.T) * sizeof(float), s, a);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  hipLaunchKernelGGL(gdn_m2_advance_kernel, dim3((unsigned)((a.B + 255) / 256)), dim3(256), 0, s, a,
                     a.T > 0 ? 0 : 1);
  return hipGetLastError();
}

template <int SDT, int P>
static hipError_t m2_launch_n(const M2Args& a, int N, int what, hipStream_t s) {
  switch (N) {
    case 16: return m2_launch_t<SDT, P, 16>(a, what, s);
    case 64: return m2_launch_t<SDT, P, 64>(a, what, s);
    case 128: return m2_launch_t<SDT, P, 128>(a, what, s);
    default: return hipErrorInvalidValue;
  }
}

template <int SDT>
static hipError_t m2_launch_sdt(const M2Args& a, int P, int N, int what, hipStream_t s) {
  switch (P) {
    case 16: return m2_launch_n<SDT, 16>(a, N, what, s);
    case 64: return m2_launch_n<SDT, 64>(a, N, what, s);
    case 128: return m2_launch_n<SDT, 128>(a, N, what, s);
    default: return hipErrorInvalidValue;
  }
}

static hipError_t m2_launch(const M2Args& a, int state_dt, int P, int N, int what, hipStream_t s) {
  if (a.B == 0) return hipSuccess;
  switch (state_dt) {
    case GDN_F32: return m2_launch_sdt<GDN_F32>(a, P, N, what, s);
    case GDN_BF16: return m2_launch_sdt<GDN_BF16>(a, P, N, what, s);
    case GDN_F16: return m2_launch_sdt<GDN_F16>(a, P, N, what, s);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_m2_decode(const M2Args& a, int state_dt, int P, int N, hipStream_t s) {
  return m2_launch(a, state_dt, P, N, 0, s);
}
hipError_t launch_m2_replay(const M2Args& a, int state_dt, int P, int N, hipStream_t s) {
  return m2_launch(a, state_dt, P, N, 1, s);
}
hipError_t launch_m2_rollback(const M2Args& a, hipStream_t s) {
  if (a.B == 0) return hipSuccess;
  hipLaunchKernelGGL(gdn_m2_advance_kernel, dim3((unsigned)((a.B + 255) / 256)), dim3(256), 0, s, a, 2);
  return hipGetLastError();
}
size_t m2_lds_bytes(int P, int N, int L, int T) {
  const size_t step = T > 0 ? m2_step_floats(P, N, L, T) * sizeof(float) : 0;
  const size_t fold = (size_t)L * (P + N + 1) * sizeof(float) + 64 * 4 + 8;
  return step > fold ? step : fold;
}

}  // namespace gdn
