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

namespace gdn {

template <int SDT, int D>
using ReplayGeom = TileGeom<SDT, D, GDN_REPLAY_WAVES>;

constexpr int kStageRows = 16;  // entry rows staged per batch of loads
constexpr int kPrepThreads = 256;
constexpr int kStreamTB = 4;    // window positions reduced per pass over the tile

// Dynamic LDS of the prep kernel (floats): entries k, v [E][D+1] (E = L + T),
// window queries [T][D+1], gates (g, beta, prefix G, spare) [E] each, Gram
// matrix [E][E], key / query products [E][T], coefficients c and e^G c
// [T][E] each.
__host__ __device__ inline size_t replay_prep_lds_bytes(int D, int L, int T) {
  const size_t E = (size_t)L + (size_t)T;
  return (2 * E * (D + 1) + (size_t)T * (D + 1) + 4 * E + E * E + 3 * E * T) * sizeof(float);
}

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
template <int D, int EB>
__global__ void __launch_bounds__(kPrepThreads) gdn_replay_prep_kernel(const ReplayArgs P, float* __restrict__ ws) {
  constexpr int NTH = kPrepThreads, NW = NTH / 64;
  constexpr int LDE = D + 1;  // padded rows: the split dot products hit distinct banks
  using Stager = RowStager<D, kStageRows, NTH, EB>;
  extern __shared__ float s_dyn[];

  const DecodeArgs& p = P.d;
  const RingArgs& R = P.ring;
  const int T = P.T, L = R.L;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int b = blockIdx.x / p.Hv;
  const int h = blockIdx.x - b * p.Hv;
  const int hk = h / (p.Hv / p.Hk);
  const int slot = p.slot_map[b];
  if (slot < 0 || (int64_t)slot >= p.num_slots) return;  // the stream kernel writes the zeros
  const int64_t unit = (int64_t)slot * p.Hv + h;
  const RingPos rp = ring_pos(R, unit);
  const int st = rp.st;
  const int cnt = min(rp.cnt, L - T);  // the fold kernel left room for the window

  const int E = L + T;
  float* e_k = s_dyn;               // [E][LDE]
  float* e_v = e_k + E * LDE;       // [E][LDE]
  float* e_q = e_v + E * LDE;       // [T][LDE]
  float* e_g = e_q + T * LDE;       // [E] g
  float* e_b = e_g + E;             // [E] beta
  float* e_G = e_b + E;             // [E] prefix sums of g
  float* s_gram = e_G + 2 * E;      // [E][E] (one spare gate row before it)
  float* s_kq = s_gram + E * E;     // [E][T]
  float* s_c = s_kq + E * T;        // [T][E]
  float* s_ec = s_c + T * E;        // [T][E]

  const int64_t ring_e = unit * L;
  for (int t = tid; t < cnt + T; t += NTH) {
    if (t < cnt) {
      const int j = (st + t) % L;
      e_g[t] = R.g[ring_e + j];
      e_b[t] = R.beta[ring_e + j];
    } else {
      const int64_t gi = ((int64_t)b * T + (t - cnt)) * p.Hv + h;
      e_g[t] = gate_g(load_elem(p.a, gi, p.in_dt), p.A_log[h], p.dt_bias[h]);
      e_b[t] = sigmoid_f(load_elem(p.b, gi, p.in_dt));
    }
  }
  for (int r0s = 0; r0s < cnt; r0s += kStageRows) {  // committed entries
    Stager sk, sv;
    auto ring_row = [&](int r) { return (ring_e + (st + r0s + r) % L) * D; };
    const int nr = min(kStageRows, cnt - r0s);
    sk.issue(R.k, nr, ring_row);
    sv.issue(R.v, nr, ring_row);
    sk.commit(e_k + r0s * LDE, LDE, p.in_dt, nr);
    sv.commit(e_v + r0s * LDE, LDE, p.in_dt, nr);
  }
  for (int t0s = 0; t0s < T; t0s += kStageRows) {  // the window's keys, values and queries
    Stager sk, sv, sq;
    const int nr = min(kStageRows, T - t0s);
    auto key_row = [&](int t) { return (((int64_t)b * T + t0s + t) * p.Hk + hk) * D; };
    sk.issue(p.k, nr, key_row);
    sv.issue(p.v, nr, [&](int t) { return (((int64_t)b * T + t0s + t) * p.Hv + h) * D; });
    sq.issue(p.q, nr, key_row);
    sk.commit(e_k + (cnt + t0s) * LDE, LDE, p.in_dt, nr);
    sv.commit(e_v + (cnt + t0s) * LDE, LDE, p.in_dt, nr);
    sq.commit(e_q + t0s * LDE, LDE, p.in_dt, nr);
  }
  // append the window to the ring (raw input bytes); the slots written were
  // not live, so nothing staged above is overwritten
  const int base = (st + cnt) % L;
  for (int i = tid; i < T * D; i += NTH) {
    const int t = i / D, c = i - t * D;
    const int64_t j = ring_e + (base + t) % L;
    copy_elem(R.k, j * D + c, p.k, (((int64_t)b * T + t) * p.Hk + hk) * D + c, p.in_dt);
    copy_elem(R.v, j * D + c, p.v, (((int64_t)b * T + t) * p.Hv + h) * D + c, p.in_dt);
  }
  __syncthreads();
  for (int t = tid; t < T; t += NTH) {  // gates as fp32
    const int64_t j = ring_e + (base + t) % L;
    R.g[j] = e_g[cnt + t];
    R.beta[j] = e_b[cnt + t];
  }
  if (tid == 0) {
    R.start[unit] = st;
    R.count[unit] = cnt + T;
  }

  const int n_all = cnt + T;  // live entries of the last window position (<= L)
  if (wave == 0) {            // prefix sums of g over the live entries
    float x = (lane < n_all) ? e_g[lane] : 0.f;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
      const float y = __shfl_up(x, off, 64);
      if (lane >= off) x += y;
    }
    if (lane < n_all) e_G[lane] = x;
  }
  // Gram matrix (upper triangle) and key / query products, four lanes per dot product
  const int n_gram = n_all * (n_all - 1) / 2;
  const int n_dots = n_gram + n_all * T;
  for (int base4 = 0; base4 < n_dots * 4; base4 += NTH) {
    const int task = (base4 + tid) >> 2, part = tid & 3;
    const bool act = task < n_dots;
    const float* x0 = e_k;
    const float* x1 = e_k;
    float* dst = nullptr;
    if (act) {
      if (task < n_gram) {  // pair (i, j), i < j, row-major over the upper triangle
        int i = 0, rem = task;
        while (rem >= n_all - 1 - i) {
          rem -= n_all - 1 - i;
          ++i;
        }
        const int j = i + 1 + rem;
        x0 = e_k + i * LDE;
        x1 = e_k + j * LDE;
        dst = s_gram + i * E + j;
      } else {
        const int y = task - n_gram, i = y / T, t = y - i * T;
        x0 = e_k + i * LDE;
        x1 = e_q + t * LDE;
        dst = s_kq + i * T + t;
      }
    }
    float acc = 0.f;
    if (act) {
#pragma unroll 8
      for (int c = part; c < D; c += 4) acc = fmaf(x0[c], x1[c], acc);
    }
    acc += __shfl_xor(acc, 1, 64);
    acc += __shfl_xor(acc, 2, 64);
    if (act && part == 0) *dst = acc;
  }
  __syncthreads();

  // back substitution for the coefficients of each window position (one wave each)
  for (int t = wave; t < T; t += NW) {
    const int e_last = cnt + t;  // last live entry of position t
    const float Gn = e_G[e_last];
    const int j = lane;  // lane j holds the residual of live entry j
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
  // w_t = e^{G_n} q_t - sum_j e^{G_j} c_j k_j and acc_t = sum_j c_j v_j, to the workspace
  float* wsu = ws + ((int64_t)b * p.Hv + h) * T * 2 * D;
  for (int x = tid; x < T * D; x += NTH) {
    const int t = x / D, c = x - t * D;
    const int e_last = cnt + t;
    float w = expf(e_G[e_last]) * e_q[t * LDE + c];
    float acc = 0.f;
    for (int jj = 0; jj <= e_last; ++jj) {
      w = fmaf(-s_ec[t * E + jj], e_k[jj * LDE + c], w);
      acc = fmaf(s_c[t * E + jj], e_v[jj * LDE + c], acc);
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
  const size_t lds = replay_prep_lds_bytes(D, a.ring.L, a.T);
  if (f32_in)
    hipLaunchKernelGGL((gdn_replay_prep_kernel<D, 4>), dim3(grid), dim3(kPrepThreads), lds, s, a, ws);
  else
    hipLaunchKernelGGL((gdn_replay_prep_kernel<D, 2>), dim3(grid), dim3(kPrepThreads), lds, s, a, ws);
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
