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
// one-shot decode workgroups over 16-bit tiles take their units in XCD-aware
// order (xcd_unit) when the tiles stream past the Infinity Cache both ways
// waves per workgroup of the decode over 16-bit tiles (the 16 KiB tile needs no
// cross-wave sums): eight, bf16 B = 512 0.407 -> 0.386 ms against two (four: 0.399)
#ifndef GDN_M2_DEC_WAVES_16
#define GDN_M2_DEC_WAVES_16 8
#endif
#ifndef GDN_M2_XCD
#define GDN_M2_XCD 1
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
// the decode kernel's own geometry (waves per workgroup for 16-bit tiles)
template <int SDT, int P, int N>
using M2DG = M2Geom<SDT, P, N, SDT == GDN_F32 ? 4 : GDN_M2_DEC_WAVES_16>;

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
__device__ __forceinline__ M2Pos m2_fix(int L, int T, int st, int cnt) {
  st = ((st % L) + L) % L;
  cnt = cnt < 0 ? 0 : (cnt > L ? L : cnt);
  const bool fold = T > 0 ? (cnt + T > L) : (cnt > 0);
  if (fold) return M2Pos{(st + cnt) % L, 0, true};
  return M2Pos{st, cnt, false};
}
__device__ __forceinline__ M2Pos m2_pos(const M2Args& a, int64_t slot) {
  return m2_fix(a.L, a.T, a.start[slot], a.count[slot]);
}

// ---------------------------------------------------------------- decode
// x (P values) is staged in LDS and the row outputs gathered there, so both
// move with one vector access per 8 elements, and B and C load VEC elements
// per access: per-element loads and stores cost the texture addresser an
// address pass each, which bounds these 32 KiB tiles as it does the 16-bit
// GDN ones.  Unaligned x, B, C or y take the per-element accesses.  The small
// loads (x, dt, B, C, as raw bits of the input dtype IDT) go out before the
// tile: loads complete in order, so their waits do not cover the tile.
template <int SDT, int P, int N, bool NT, int IDT, bool XO>
__global__ void __launch_bounds__((M2DG<SDT, P, N>::NW * 64)) gdn_m2_decode_kernel(const M2Args a) {
  using G = M2DG<SDT, P, N>;
  constexpr int VEC = G::VEC, LPR = G::LPR, RPW = G::RPW, NW = G::NW, PASSES = G::PASSES;
  static_assert(P % 8 == 0 && P / 8 <= NW * 64, "x staged 8 values per lane");
  using IO = TileIO<SDT, VEC, NT>;
  using ST = typename StateElem<SDT>::T;
  __shared__ float s_x[P], s_y[P];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int u = XO ? xcd_unit(blockIdx.x, gridDim.x) : (int)blockIdx.x;  // XO: XCD-aware order
  const int b = u / a.H, h = u - (u / a.H) * a.H;
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
template <int SDT, int P, int N, bool NT, int IDT>
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

      auto ring_at = [&](int e) { const int y = st + e; return y >= L ? y - L : y; };  // st < L, e < L
      const int64_t rh = (slot * a.H + h) * L, rg = (slot * a.G + gr) * L;
      // The committed entries (x rows, B rows, g and dt') go out first, 8
      // elements per access, as one batch (every thread loading, indices clamped
      // into the live entries), then the tile: loads return in order, so
      // waiting for the entries does not wait for the tile.  Element loops had
      // made each element a dependent round after the whole tile.  B rows as
      // vectors need a 16-byte aligned ring; rings past 16 entries loop after.
      constexpr int PV = P / 8, NV = N / 8;
      constexpr int KX = (16 * PV + NTH - 1) / NTH, KB = (16 * NV + NTH - 1) / NTH;
      const int nx = cnt * PV, nb = cnt * NV, clast = (cnt > 0 ? cnt : 1) - 1;
      const bool vB = (reinterpret_cast<uintptr_t>(a.rB) & 15) == 0;
      auto x_at = [&](int q) { const int e = q / PV; return (rh + ring_at(min(e, clast))) * P + (q - e * PV) * 8; };
      auto b_at = [&](int q) { const int e = q / NV; return (rg + ring_at(min(e, clast))) * N + (q - e * NV) * 8; };
      auto put8 = [&](float* d, const InVec<IDT, 8>& r) {
        float f[8];
        r.widen(f);
#pragma unroll
        for (int k = 0; k < 8; ++k) d[k] = f[k];
      };
      InVec<IDT, 8> xr[KX], br[KB];
#pragma unroll
      for (int u = 0; u < KX; ++u) xr[u].load(a.rx, x_at(min(u * NTH + tid, max(nx, 1) - 1)));
      if (vB) {
#pragma unroll
        for (int u = 0; u < KB; ++u) br[u].load(a.rB, b_at(min(u * NTH + tid, max(nb, 1) - 1)));
      }
      const int64_t gj_at = rh + ring_at(min(lane, clast));
      const float g_raw = a.rg[gj_at], d_raw = a.rdtp[gj_at];
      __builtin_amdgcn_sched_barrier(0);  // the entries' loads stay ahead of the tile's

      int lane_off = r0 * N + c0;
      asm volatile("" : "+v"(lane_off));
      ST* tile = static_cast<ST*>(a.pool) + (slot * a.H + h) * (int64_t)(P * N) + lane_off;
      typename IO::Raw raw[PASSES];
#pragma unroll
      for (int pp = 0; pp < PASSES; ++pp) raw[pp] = IO::load_raw(tile + pp * NW * RPW * N);
      __builtin_amdgcn_sched_barrier(0);

      // committed entries in live order, widened
#pragma unroll
      for (int u = 0; u < KX; ++u)
        if (u * NTH + tid < nx) put8(ex + 8 * (u * NTH + tid), xr[u]);
      for (int q = KX * NTH + tid; q < nx; q += NTH) {
        InVec<IDT, 8> r;
        r.load(a.rx, x_at(q));
        put8(ex + 8 * q, r);
      }
      if (vB) {
#pragma unroll
        for (int u = 0; u < KB; ++u)
          if (u * NTH + tid < nb) put8(eB + 8 * (u * NTH + tid), br[u]);
        for (int q = KB * NTH + tid; q < nb; q += NTH) {
          InVec<IDT, 8> r;
          r.load(a.rB, b_at(q));
          put8(eB + 8 * q, r);
        }
      } else {  // unaligned ring B rows: one element per access
        for (int i = tid; i < cnt * N; i += NTH) {
          const int e = i / N, c = i - e * N;
          eB[i] = load_elem(a.rB, (rg + ring_at(e)) * N + c, IDT);
        }
      }
      if (wave == 0) {  // weights e^{G_c - G_j} dt'_j from a suffix sum of g, and the decay e^{G_c}
        const int j = lane;
        const float gj = j < cnt ? g_raw : 0.f;
        float suf = gj;  // sum of g over entries j..cnt-1
#pragma unroll
        for (int off = 1; off < 64; off <<= 1) {
          const float y = __shfl_down(suf, off, 64);
          if (j + off < 64) suf += y;
        }
        if (j < cnt) ew[j] = expf(suf - gj) * d_raw;
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

template <int SDT, int P, int N, bool NT, int IDT>
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
  // Order of the loads: the ring pointers; the first batch of every phase-A
  // part (they need the pointers); the first head's tile.  Loads return in
  // order, so waiting for the phase-A loads does not wait for the tile.
  const int st_raw = a.start[slot], ct_raw = a.count[slot];
  const ST* tiles = static_cast<const ST*>(a.pool) + ((int64_t)slot * a.H + h0) * (int64_t)(P * N);

  float* rB = s_dyn;               // [L][N] ring order
  float* wB = rB + L * N;          // [T][N]
  float* wC = wB + T * N;          // [T][N]
  float* dots = wC + T * N;        // [T][L] B_j . C_t, live order
  float* eG = dots + T * L;        // [HPG][L]
  float* ed = eG + HPG * L;        // [HPG][L]
  float* ew = ed + HPG * L;        // [HPG][T][L]
  float* edec = ew + HPG * T * L;  // [HPG][T] e^{G_e}
  float* acc = edec + HPG * T;     // [HPG][T][P]

  const M2Pos pos = m2_fix(L, T, st_raw, ct_raw);
  const int st = pos.st, cnt = pos.cnt, n_all = cnt + T;  // n_all <= L
  auto ring_at = [&](int e) { const int x = st + e; return x >= L ? x - L : x; };  // st < L, e < L
  const int64_t rgp = ((int64_t)slot * a.G + gr) * L;
  // ---- phase A.  Each part issues all its loads (8 elements per access, every
  // thread loading, indices clamped) before its first store, so a part is one
  // memory round; one element per access, or a load whose value a branch waits
  // for, had made every element a round of its own.
  // Part 1, the group's rows: committed ring B rows to LDS (ring order), window
  // B and C rows to LDS with B appended to the ring, window x appended to the
  // heads' rings.  B rows as vectors need 16-byte aligned ring and inputs.  The
  // first batch is straight-line code, one source per load (a per-lane choice
  // among argument pointers compiles to a load of the pointer itself) and all
  // its loads before its first store; longer rings and windows loop after it.
  constexpr int NV = N / 8, PV = P / 8;
  constexpr int K1 = (16 * NV + NTH - 1) / NTH;  // ring B groups per thread in the first batch (up to 16 entries)
  const int n1 = cnt * NV, n2 = T * NV, n3 = HPG * T * PV;
  const bool vB = ((reinterpret_cast<uintptr_t>(a.rB) | reinterpret_cast<uintptr_t>(a.Bm) |
                    reinterpret_cast<uintptr_t>(a.Cm)) & 15) == 0;
  auto ring_b = [&](int q) { const int e = q / NV; return (rgp + ring_at(e)) * N + (q - e * NV) * 8; };
  auto win_bc = [&](int q) {
    const int t = q / NV;
    return (((int64_t)b * T + t) * a.G + gr) * N + (q - t * NV) * 8;
  };
  auto win_x = [&](int q) {
    const int hi = q / (T * PV), rem = q - hi * T * PV, t = rem / PV;
    return (((int64_t)b * T + t) * a.H + h0 + hi) * P + (rem - t * PV) * 8;
  };
  auto put_b = [&](int q, const InVec<IDT, 8>& r) {  // committed ring B row group q
    const int e = q / NV, c = (q - e * NV) * 8;
    float f[8];
    r.widen(f);
    float* d = rB + ring_at(e) * N + c;
#pragma unroll
    for (int k = 0; k < 8; ++k) d[k] = f[k];
  };
  auto put_bc = [&](int q, const InVec<IDT, 8>& rb, const InVec<IDT, 8>& rc) {  // window B and C group q
    const int t = q / NV, c = (q - t * NV) * 8;
    float f[8], g[8];
    rb.widen(f);
    rc.widen(g);
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      wB[t * N + c + k] = f[k];
      wC[t * N + c + k] = g[k];
    }
    rb.store(a.rB, (rgp + ring_at(cnt + t)) * N + c);  // append B
  };
  auto put_x = [&](int q, const InVec<IDT, 8>& r) {  // window x group q, appended to its head's ring
    const int hi = q / (T * PV), rem = q - hi * T * PV, t = rem / PV;
    r.store(a.rx, (((int64_t)slot * a.H + h0 + hi) * L + ring_at(cnt + t)) * P + (rem - t * PV) * 8);
  };
  // Part 2, gates: pair (head hi, live entry j); committed entries read g and
  // dt' from the ring, window ones form them from dt and append them.  Both
  // sources are read in every thread (the ring position is in range for any
  // pair) and selected.
  const int ng = HPG * n_all;
  struct GateIn {
    float g, d, dtb, al;
    uint32_t dt;
  };
  auto gate_ld = [&](int q) {
    const int hi = q / n_all, j = q - hi * n_all, h = h0 + hi;
    const int64_t rh = ((int64_t)slot * a.H + h) * L + ring_at(j);
    return GateIn{a.rg[rh], a.rdtp[rh], a.dt_bias[h], a.A_log[h],
                  in_bits<IDT>(a.dt, ((int64_t)b * T + max(j - cnt, 0)) * a.H + h)};
  };
  auto gate_put = [&](int q, const GateIn& x) {
    const int hi = q / n_all, j = q - hi * n_all;
    float gj = x.g, dj = x.d;
    if (j >= cnt) {
      dj = softplus_f(in_value<IDT>(x.dt) + x.dtb);
      gj = -expf(x.al) * dj;
      const int64_t rh = ((int64_t)slot * a.H + h0 + hi) * L + ring_at(j);
      a.rg[rh] = gj;  // append g and dt'
      a.rdtp[rh] = dj;
    }
    eG[hi * L + j] = gj;
    ed[hi * L + j] = dj;
  };
  typename IO::Raw cur[PASSES];
  {
    InVec<IDT, 8> r1[K1], r2b, r2c, r3;
    GateIn g2[2];
    if (vB) {
      if (n1 > 0) {
#pragma unroll
        for (int u = 0; u < K1; ++u) r1[u].load(a.rB, ring_b(min(u * NTH + tid, n1 - 1)));
      }
      r2b.load(a.Bm, win_bc(min(tid, n2 - 1)));
      r2c.load(a.Cm, win_bc(min(tid, n2 - 1)));
    }
    r3.load(a.x, win_x(min(tid, n3 - 1)));
#pragma unroll
    for (int u = 0; u < 2; ++u) g2[u] = gate_ld(min(u * NTH + tid, ng - 1));
    __builtin_amdgcn_sched_barrier(0);  // the batch's loads stay together, ahead of the tile's
#pragma unroll
    for (int pp = 0; pp < PASSES; ++pp) cur[pp] = IO::load_raw(tiles + (r0 + pp * NW * RPW) * N + c0);
    __builtin_amdgcn_sched_barrier(0);
    if (vB) {
#pragma unroll
      for (int u = 0; u < K1; ++u)
        if (u * NTH + tid < n1) put_b(u * NTH + tid, r1[u]);
      if (tid < n2) put_bc(tid, r2b, r2c);
    }
    if (tid < n3) put_x(tid, r3);
#pragma unroll
    for (int u = 0; u < 2; ++u)
      if (u * NTH + tid < ng) gate_put(u * NTH + tid, g2[u]);
  }
  if (vB) {  // beyond the first batch
    for (int q = K1 * NTH + tid; q < n1; q += NTH) {
      InVec<IDT, 8> r;
      r.load(a.rB, ring_b(q));
      put_b(q, r);
    }
    for (int q = NTH + tid; q < n2; q += NTH) {
      InVec<IDT, 8> rb, rc;
      rb.load(a.Bm, win_bc(q));
      rc.load(a.Cm, win_bc(q));
      put_bc(q, rb, rc);
    }
  } else {  // unaligned B rows: one element per access
    for (int i = tid; i < cnt * N; i += NTH) {
      const int e = i / N, c = i - e * N, j = ring_at(e);
      rB[j * N + c] = load_elem(a.rB, (rgp + j) * N + c, IDT);
    }
    for (int i = tid; i < T * N; i += NTH) {
      const int t = i / N, c = i - t * N;
      const int64_t src = (((int64_t)b * T + t) * a.G + gr) * N + c;
      wB[i] = load_elem(a.Bm, src, IDT);
      wC[i] = load_elem(a.Cm, src, IDT);
      copy_elem(a.rB, (rgp + ring_at(cnt + t)) * N + c, a.Bm, src, IDT);  // append B
    }
  }
  for (int q = NTH + tid; q < n3; q += NTH) {
    InVec<IDT, 8> r;
    r.load(a.x, win_x(q));
    put_x(q, r);
  }
  for (int q = 2 * NTH + tid; q < ng; q += NTH) gate_put(q, gate_ld(q));  // beyond the first batch
  __syncthreads();
  for (int hi = wave; hi < HPG; hi += NW) {  // prefix sums of g per head (lane j: entry j)
    const int j = lane;
    float Gs = j < n_all ? eG[hi * L + j] : 0.f;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
      const float y = __shfl_up(Gs, off, 64);
      if (j >= off) Gs += y;
    }
    if (j < L) {
      eG[hi * L + j] = Gs;
      if (j >= n_all) ed[hi * L + j] = 0.f;
    }
  }
  __syncthreads();
  for (int item = wave; item < T * L; item += NW) {  // B_j . C_t, one wave per pair, lanes over n
    const int t = item / L, j = item - t * L;
    if (j > cnt + t) continue;
    const float* Bj = j < cnt ? rB + ring_at(j) * N : wB + (j - cnt) * N;
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
  // acc[hi][t][r..r+3] = sum_j w x_j + D x_t, four rows per thread, x read from the
  // ring and the window.  Up to 16 live entries all of a thread's rows go out
  // before its sums (a pointer and an index selected per entry, no branch).
  for (int i = tid; i < HPG * T * (P / 4); i += NTH) {
    const int hi = i / (T * (P / 4)), rem = i - hi * T * (P / 4), t = rem / (P / 4), r = (rem - t * (P / 4)) * 4;
    const int h = h0 + hi, e_last = cnt + t;
    const int64_t rh = ((int64_t)slot * a.H + h) * L;
    const int64_t xw = ((int64_t)b * T * a.H + h) * P + r;  // window x of position 0
    const float* w = ew + (hi * T + t) * L;
    auto x_src = [&](int j, const void*& p) -> int64_t {
      p = j < cnt ? a.rx : a.x;
      return j < cnt ? (rh + ring_at(j)) * P + r : xw + (int64_t)(j - cnt) * a.H * P;
    };
    InVec<IDT, 4> xtr;
    xtr.load(a.x, xw + (int64_t)t * a.H * P);
    const float Dh = a.Dskip[h];
    float v[4], f[4];
    if (L <= 16) {
      InVec<IDT, 4> xr[16];
#pragma unroll
      for (int j = 0; j < 16; ++j) {
        const void* p = nullptr;
        const int64_t k = x_src(min(j, e_last), p);
        xr[j].load(p, k);
      }
      __builtin_amdgcn_sched_barrier(0);  // the rows' loads stay together
      xtr.widen(f);
#pragma unroll
      for (int e = 0; e < 4; ++e) v[e] = Dh * f[e];
#pragma unroll
      for (int j = 0; j < 16; ++j) {
        if (j <= e_last) {
          xr[j].widen(f);
          const float wj = w[j];
#pragma unroll
          for (int e = 0; e < 4; ++e) v[e] = fmaf(wj, f[e], v[e]);
        }
      }
    } else {
      xtr.widen(f);
#pragma unroll
      for (int e = 0; e < 4; ++e) v[e] = Dh * f[e];
      for (int j = 0; j <= e_last; ++j) {
        const void* p = nullptr;
        const int64_t k = x_src(j, p);
        InVec<IDT, 4> xj;
        xj.load(p, k);
        xj.widen(f);
#pragma unroll
        for (int e = 0; e < 4; ++e) v[e] = fmaf(w[j], f[e], v[e]);
      }
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
    // 16-bit tiles that stream past the Infinity Cache both ways: XCD-aware unit
    // order (bf16 B = 512: 0.416 -> 0.406 ms; fp32 tiles lost 3% to it)
    const bool xo = GDN_M2_XCD != 0 && SDT != GDN_F32 &&
                    stream_tile_writes((long long)units * P * N * (long long)sizeof(typename StateElem<SDT>::T));
    void (*k)(const M2Args);
    auto pick = [&](auto xo_c) {
      constexpr bool X = decltype(xo_c)::value;
      k = a.in_dt == GDN_F32    ? &gdn_m2_decode_kernel<SDT, P, N, NT, GDN_F32, X>
          : a.in_dt == GDN_BF16 ? &gdn_m2_decode_kernel<SDT, P, N, NT, GDN_BF16, X>
                                : &gdn_m2_decode_kernel<SDT, P, N, NT, GDN_F16, X>;
    };
    if (xo) pick(std::true_type{});
    else pick(std::false_type{});
    hipLaunchKernelGGL(k, dim3(units), dim3(M2DG<SDT, P, N>::NW * 64), 0, s, a);
    return hipGetLastError();
  }
  // fold (persistent, sized to the resident workgroups)
  const size_t fold_lds = ((size_t)a.L * (P + N + 1)) * sizeof(float);
  int per_cu = 0, cus = 0;
  void (*fold)(const M2Args) = a.in_dt == GDN_F32    ? &gdn_m2_fold_kernel<SDT, P, N, NT, GDN_F32>
                               : a.in_dt == GDN_BF16 ? &gdn_m2_fold_kernel<SDT, P, N, NT, GDN_BF16>
                                                     : &gdn_m2_fold_kernel<SDT, P, N, NT, GDN_F16>;
  hipError_t e = resident_blocks(reinterpret_cast<const void*>(fold), G::NW * 64, fold_lds, &per_cu);
  if (e == hipSuccess) e = device_cus(&cus);
  if (e != hipSuccess) return e;
  const int64_t fill = (int64_t)(per_cu > 0 ? per_cu : 1) * cus;
  hipLaunchKernelGGL(fold, dim3((unsigned)(units < fill ? units : fill)), dim3(G::NW * 64), fold_lds, s, a);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  if (a.T > 0) {
    void (*k)(const M2Args) = a.in_dt == GDN_F32    ? &gdn_m2_step_kernel<SDT, P, N, NT, GDN_F32>
                              : a.in_dt == GDN_BF16 ? &gdn_m2_step_kernel<SDT, P, N, NT, GDN_BF16>
                                                    : &gdn_m2_step_kernel<SDT, P, N, NT, GDN_F16>;
    hipLaunchKernelGGL(k, dim3((unsigned)((int64_t)a.B * a.G)), dim3(G::NW * 64),
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
