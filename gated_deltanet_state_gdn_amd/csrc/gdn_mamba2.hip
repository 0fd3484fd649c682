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
// x (P values) is staged in LDS and the row outputs gathered there, so both
// move with one vector access per 8 elements, and B and C load VEC elements
// per access: per-element loads and stores cost the texture addresser an
// address pass each, which bounds these 32 KiB tiles as it does the 16-bit
// GDN ones.  Unaligned x, B, C or y take the per-element accesses.  The small
// loads (x, dt, B, C, as raw bits of the input dtype IDT) go out before the
// tile: loads complete in order, so their waits do not cover the tile.
template <int SDT, int P, int N, bool NT, int IDT>
__global__ void __launch_bounds__((M2G<SDT, P, N>::NW * 64)) gdn_m2_decode_kernel(const M2Args a) {
  using G = M2G<SDT, P, N>;
  constexpr int VEC = G::VEC, LPR = G::LPR, RPW = G::RPW, NW = G::NW, PASSES = G::PASSES;
  static_assert(P % 8 == 0 && P / 8 <= NW * 64, "x staged 8 values per lane");
  using IO = TileIO<SDT, VEC, NT>;
  using ST = typename StateElem<SDT>::T;
  __shared__ float s_x[P], s_y[P];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int b = blockIdx.x / a.H, h = blockIdx.x - (blockIdx.x / a.H) * a.H;
  const int gr = h / (a.H / a.G);
  const int c0 = (lane % LPR) * VEC;
  const int r0 = wave * RPW + lane / LPR;
  const int64_t yb = ((int64_t)b * a.H + h) * P;
  const int slot = a.slot_map[b];
  const bool vy = (reinterpret_cast<uintptr_t>(a.y) & 15) == 0;
  if (slot < 0 || (int64_t)slot >= a.num_slots) {  // padded row
    if (tid < P / 8) {
      const float z[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
      store_vec<8>(a.y, yb + 8 * tid, z, a.out_dt, vy);
    }
    return;
  }
  ST* tile = static_cast<ST*>(a.pool) + ((int64_t)slot * a.H + h) * (int64_t)(P * N);
  const bool vx = (reinterpret_cast<uintptr_t>(a.x) & 15) == 0;
  const bool vbc = ((reinterpret_cast<uintptr_t>(a.Bm) | reinterpret_cast<uintptr_t>(a.Cm)) & 15) == 0;
  const int xi = 8 * min(tid, P / 8 - 1);  // threads past P / 8 reload the last group (no branch)
  const int64_t bc = ((int64_t)b * a.G + gr) * N + c0;
  const uint32_t dtb = in_bits<IDT>(a.dt, (int64_t)b * a.H + h);
  const float dt_bias = a.dt_bias[h], A_log = a.A_log[h], Dh = a.Dskip[h];
  InVec<IDT, 8> xv;
  InVec<IDT, VEC> bv, cv;
  if (vx) xv.load(a.x, yb + xi);
  if (vbc) {
    bv.load(a.Bm, bc);
    cv.load(a.Cm, bc);
  }
  typename IO::Raw raw[PASSES];
#pragma unroll
  for (int pp = 0; pp < PASSES; ++pp) raw[pp] = IO::load_raw(tile + (r0 + pp * NW * RPW) * N + c0);

  if (tid < P / 8) {
    float f[8];
    if (vx) {
      xv.widen(f);
    } else {
#pragma unroll
      for (int e = 0; e < 8; ++e) f[e] = load_elem(a.x, yb + xi + e, IDT);
    }
#pragma unroll
    for (int e = 0; e < 8; ++e) s_x[xi + e] = f[e];
  }
  const float dtp = softplus_f(in_value<IDT>(dtb) + dt_bias);
  const float alpha = expf(-expf(A_log) * dtp);
  float Bc[VEC], Cc[VEC];
  if (vbc) {
    bv.widen(Bc);
    cv.widen(Cc);
  } else {
#pragma unroll
    for (int e = 0; e < VEC; ++e) {
      Bc[e] = load_elem(a.Bm, bc + e, IDT);
      Cc[e] = load_elem(a.Cm, bc + e, IDT);
    }
  }
#pragma unroll
  for (int e = 0; e < VEC; ++e) Bc[e] *= dtp;
  __syncthreads();
#pragma unroll
  for (int pp = 0; pp < PASSES; ++pp) {
    const int r = r0 + pp * NW * RPW;
    const float xr = s_x[r];
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
    if ((lane % LPR) == 0) s_y[r] = fmaf(Dh, xr, part);
  }
  __syncthreads();
  if (tid < P / 8) {
    float f[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) f[e] = s_y[8 * tid + e];
    store_vec<8>(a.y, yb + 8 * tid, f, a.out_dt, vy);
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
      float sv[PASSES][VEC];
#pragma unroll
      for (int pp = 0; pp < PASSES; ++pp) {
        IO::widen(raw[pp], sv[pp]);
#pragma unroll
        for (int e = 0; e < VEC; ++e) sv[pp][e] *= decay;
      }
      for (int j = 0; j < cnt; ++j) {  // rank-cnt update, B_j's columns held in registers
        const float wj = ew[j];
        float bj[VEC];
#pragma unroll
        for (int e = 0; e < VEC; ++e) bj[e] = eB[j * N + c0 + e];
#pragma unroll
        for (int pp = 0; pp < PASSES; ++pp) {
          const float cx = wj * ex[j * P + r0 + pp * NW * RPW];
#pragma unroll
          for (int e = 0; e < VEC; ++e) sv[pp][e] = fmaf(cx, bj[e], sv[pp][e]);
        }
      }
#pragma unroll
      for (int pp = 0; pp < PASSES; ++pp) IO::store(tile + pp * NW * RPW * N, sv[pp]);
      __syncthreads();  // LDS staging is reused by the next unit
    }
    __syncthreads();  // s_list is rewritten by the next check
  }
}

// ---------------------------------------------------------------- step
// One workgroup per (sequence, group): the B . C products are shared by the
// group's heads, so they are formed once; then the heads' checkpoint tiles
// stream through VGPRs one after another (the next tile's loads in flight
// while the current one is reduced).  Phase A stages the group's live B rows
// and the window's B and C, appends the window to the ring (B once per group;
// x, g and dt' per head), forms per head the prefix sums G of g and the weights
// w_tj = e^{G_e - G_j} dt'_j (B_j . C_t), and the ring part of every output,
// acc_t = sum_j w_tj x_j + D x_t.  Phase B adds e^{G_e} S0 C_t per head.
// Dynamic LDS (floats): ring B [L][N] (ring order), window B and C [T][N]
// each, dots [T][L], prefix sums and dt' [HPG][L] each, weights [HPG][T][L],
// decays [HPG][T], acc [HPG][T][P].
__host__ __device__ inline size_t m2_step_floats(int P, int N, int L, int T, int HPG) {
  return (size_t)L * N + 2 * (size_t)T * N + (size_t)T * L + 2 * (size_t)HPG * L + (size_t)HPG * T * L +
         (size_t)HPG * T + (size_t)HPG * T * P;
}

// Four consecutive input elements (16-byte aligned for f32, 8 for 16-bit) as floats.
__device__ __forceinline__ void load4(const void* p, int64_t i, int dt, float (&f)[4]) {
  if (dt == GDN_F32) {
    const f32x4 v = *reinterpret_cast<const f32x4*>(static_cast<const float*>(p) + i);
#pragma unroll
    for (int e = 0; e < 4; ++e) f[e] = v[e];
  } else {
    const u32x2 w = *reinterpret_cast<const u32x2*>(static_cast<const uint16_t*>(p) + i);
#pragma unroll
    for (int e = 0; e < 2; ++e) {
      const uint32_t lo = w[e] & 0xffffu, hi = w[e] >> 16;
      f[2 * e] = dt == GDN_BF16 ? bf16_bits_to_f32(lo) : f16_bits_to_f32(lo);
      f[2 * e + 1] = dt == GDN_BF16 ? bf16_bits_to_f32(hi) : f16_bits_to_f32(hi);
    }
  }
}

template <int SDT, int P, int N, bool NT>
__global__ void __launch_bounds__((M2G<SDT, P, N>::NW * 64)) gdn_m2_step_kernel(const M2Args a) {
  using G = M2G<SDT, P, N>;
  constexpr int VEC = G::VEC, LPR = G::LPR, RPW = G::RPW, NW = G::NW, PASSES = G::PASSES;
  constexpr int NTH = NW * 64;
  using IO = TileIO<SDT, VEC, NT>;
  using ST = typename StateElem<SDT>::T;
  extern __shared__ float s_dyn[];
  const int L = a.L, T = a.T, HPG = a.H / a.G;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int b = blockIdx.x / a.G, gr = blockIdx.x - (blockIdx.x / a.G) * a.G;
  const int h0 = gr * HPG;
  const int c0 = (lane % LPR) * VEC;
  const int r0 = wave * RPW + lane / LPR;
  const int slot = a.slot_map[b];
  if (slot < 0 || (int64_t)slot >= a.num_slots) {  // padded row
    for (int i = tid; i < T * HPG * P; i += NTH) {
      const int t = i / (HPG * P), rem = i - t * HPG * P;
      store_elem(a.y, (((int64_t)b * T + t) * a.H + h0) * P + rem, 0.f, a.out_dt);
    }
    return;
  }
  const ST* tiles = static_cast<const ST*>(a.pool) + ((int64_t)slot * a.H + h0) * (int64_t)(P * N);
  typename IO::Raw cur[PASSES];
#pragma unroll
  for (int pp = 0; pp < PASSES; ++pp) cur[pp] = IO::load_raw(tiles + (r0 + pp * NW * RPW) * N + c0);

  float* rB = s_dyn;               // [L][N] ring order
  float* wB = rB + L * N;          // [T][N]
  float* wC = wB + T * N;          // [T][N]
  float* dots = wC + T * N;        // [T][L] B_j . C_t, live order
  float* eG = dots + T * L;        // [HPG][L]
  float* ed = eG + HPG * L;        // [HPG][L]
  float* ew = ed + HPG * L;        // [HPG][T][L]
  float* edec = ew + HPG * T * L;  // [HPG][T] e^{G_e}
  float* acc = edec + HPG * T;     // [HPG][T][P]

  const M2Pos pos = m2_pos(a, slot);
  const int st = pos.st, cnt = pos.cnt, n_all = cnt + T;  // n_all <= L
  const int64_t rgp = ((int64_t)slot * a.G + gr) * L;
  // ---- phase A: group rows, appends, gates
  for (int i = tid; i < cnt * N; i += NTH) {
    const int e = i / N, c = i - e * N;
    const int j = (st + e) % L;
    rB[j * N + c] = load_elem(a.rB, (rgp + j) * N + c, a.in_dt);
  }
  for (int i = tid; i < T * N; i += NTH) {
    const int t = i / N, c = i - t * N;
    const int64_t src = (((int64_t)b * T + t) * a.G + gr) * N + c;
    wB[i] = load_elem(a.Bm, src, a.in_dt);
    wC[i] = load_elem(a.Cm, src, a.in_dt);
    copy_elem(a.rB, (rgp + (st + cnt + t) % L) * N + c, a.Bm, src, a.in_dt);  // append B
  }
  for (int i = tid; i < HPG * T * P; i += NTH) {  // append x
    const int hi = i / (T * P), rem = i - hi * T * P, t = rem / P, c = rem - t * P;
    const int64_t rh = ((int64_t)slot * a.H + h0 + hi) * L;
    copy_elem(a.rx, (rh + (st + cnt + t) % L) * P + c, a.x, (((int64_t)b * T + t) * a.H + h0 + hi) * P + c,
              a.in_dt);
  }
  for (int hi = wave; hi < HPG; hi += NW) {  // per head: lane j takes live entry j
    const int h = h0 + hi, j = lane;
    const int64_t rh = ((int64_t)slot * a.H + h) * L;
    float gj = 0.f, dj = 0.f;
    if (j < cnt) {
      gj = a.rg[rh + (st + j) % L];
      dj = a.rdtp[rh + (st + j) % L];
    } else if (j < n_all) {
      const int t = j - cnt;
      dj = softplus_f(load_elem(a.dt, ((int64_t)b * T + t) * a.H + h, a.in_dt) + a.dt_bias[h]);
      gj = -expf(a.A_log[h]) * dj;
      a.rg[rh + (st + cnt + t) % L] = gj;  // append g and dt'
      a.rdtp[rh + (st + cnt + t) % L] = dj;
    }
    float Gs = gj;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
      const float y = __shfl_up(Gs, off, 64);
      if (j >= off) Gs += y;
    }
    if (j < L) {
      eG[hi * L + j] = Gs;
      ed[hi * L + j] = dj;
    }
  }
  __syncthreads();
  for (int item = wave; item < T * L; item += NW) {  // B_j . C_t, one wave per pair, lanes over n
    const int t = item / L, j = item - t * L;
    if (j > cnt + t) continue;
    const float* Bj = j < cnt ? rB + ((st + j) % L) * N : wB + (j - cnt) * N;
    const float* Ct = wC + t * N;
    float d = 0.f;
    for (int c = lane; c < N; c += 64) d = fmaf(Bj[c], Ct[c], d);
    d = wave_sum(d);
    if (lane == 0) dots[item] = d;
  }
  __syncthreads();
  for (int i = tid; i < HPG * T * L; i += NTH) {  // weights per head
    const int hi = i / (T * L), rem = i - hi * T * L, t = rem / L, j = rem - t * L;
    const int e_last = cnt + t;
    ew[i] = j <= e_last ? expf(eG[hi * L + e_last] - eG[hi * L + j]) * ed[hi * L + j] * dots[t * L + j] : 0.f;
    if (j == 0) edec[hi * T + t] = expf(eG[hi * L + e_last]);
  }
  __syncthreads();
  // acc[hi][t][r..r+3] = sum_j w x_j + D x_t, four rows per thread, x read from the ring and the window
  for (int i = tid; i < HPG * T * (P / 4); i += NTH) {
    const int hi = i / (T * (P / 4)), rem = i - hi * T * (P / 4), t = rem / (P / 4), r = (rem - t * (P / 4)) * 4;
    const int h = h0 + hi;
    const int64_t rh = ((int64_t)slot * a.H + h) * L;
    const int64_t xw = ((int64_t)b * T * a.H + h) * P + r;  // window x of position 0
    float v[4], xt[4];
    load4(a.x, xw + (int64_t)t * a.H * P, a.in_dt, xt);
    const float Dh = a.Dskip[h];
#pragma unroll
    for (int e = 0; e < 4; ++e) v[e] = Dh * xt[e];
    const float* w = ew + (hi * T + t) * L;
    for (int j = 0; j <= cnt + t; ++j) {
      float xj[4];
      if (j < cnt)
        load4(a.rx, (rh + (st + j) % L) * P + r, a.in_dt, xj);
      else
        load4(a.x, xw + (int64_t)(j - cnt) * a.H * P, a.in_dt, xj);
#pragma unroll
      for (int e = 0; e < 4; ++e) v[e] = fmaf(w[j], xj[e], v[e]);
    }
#pragma unroll
    for (int e = 0; e < 4; ++e) acc[(hi * T + t) * P + r + e] = v[e];
  }
  __syncthreads();
  // ---- phase B: the heads' tiles in turn, the next one's loads in flight
  for (int hi = 0; hi < HPG; ++hi) {
    typename IO::Raw nxt[PASSES];
    const int hn = hi + 1 < HPG ? hi + 1 : hi;  // the last head re-reads itself (keeps the load count fixed)
#pragma unroll
    for (int pp = 0; pp < PASSES; ++pp)
      nxt[pp] = IO::load_raw(tiles + (int64_t)hn * (P * N) + (r0 + pp * NW * RPW) * N + c0);
    for (int t = 0; t < T; ++t) {
      float Cc[VEC];
#pragma unroll
      for (int e = 0; e < VEC; ++e) Cc[e] = wC[t * N + c0 + e];
      const float decay = edec[hi * T + t];
#pragma unroll
      for (int pp = 0; pp < PASSES; ++pp) {
        const int r = r0 + pp * NW * RPW;
        float sv[VEC];
        IO::widen(cur[pp], sv);
        float part = 0.f;
#pragma unroll
        for (int e = 0; e < VEC; ++e) part = fmaf(sv[e], Cc[e], part);
        part = row_sum<LPR>(part);
        if ((lane % LPR) == 0)
          store_elem(a.y, (((int64_t)b * T + t) * a.H + h0 + hi) * P + r, fmaf(decay, part, acc[(hi * T + t) * P + r]),
                     a.out_dt);
      }
    }
#pragma unroll
    for (int pp = 0; pp < PASSES; ++pp) cur[pp] = nxt[pp];
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
    void (*k)(const M2Args) = a.in_dt == GDN_F32    ? &gdn_m2_decode_kernel<SDT, P, N, NT, GDN_F32>
                              : a.in_dt == GDN_BF16 ? &gdn_m2_decode_kernel<SDT, P, N, NT, GDN_BF16>
                                                    : &gdn_m2_decode_kernel<SDT, P, N, NT, GDN_F16>;
    hipLaunchKernelGGL(k, dim3(units), dim3(G::NW * 64), 0, s, a);
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
    hipLaunchKernelGGL((gdn_m2_step_kernel<SDT, P, N, NT>), dim3((unsigned)((int64_t)a.B * a.G)), dim3(G::NW * 64),
                       m2_step_floats(P, N, a.L, a.T, a.H / a.G) * sizeof(float), s, a);
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
size_t m2_lds_bytes(int P, int N, int L, int T, int HPG) {
  const size_t step = T > 0 ? m2_step_floats(P, N, L, T, HPG) * sizeof(float) : 0;
  const size_t fold = (size_t)L * (P + N + 1) * sizeof(float) + 64 * 4 + 8;
  return step > fold ? step : fold;
}

}  // namespace gdn
