// ReplaySSM-style GDN decode: a checkpoint S0 per (slot, value head) plus a
// ring of the last <= L state-building inputs (k, v, g, beta) replaces the
// per-step full-state write (AREX ReplaySSM article, "cache inputs, not state"
// section).  One workgroup owns one (sequence, value head) unit: its
// checkpoint tile, its ring entries and its ring pointers, so units never
// communicate.
//
// A step of T tokens:
//   1. if count + T > L, fold the committed entries into S0 (sequential
//      rank-1 updates on the tile held in VGPRs, one column reduction per
//      entry), write S0 back rounded once, and empty the ring;
//   2. append the T new entries at (start + count + t) mod L;
//   3. window position t outputs scale * S_t^T q_t, S_t being S0 advanced
//      over live entries first..e_t, without materialising S_t.
//
// Step 3 unrolls S_i = a_i (I - b_i k_i k_i^T) S_{i-1} + b_i k_i v_i^T
// (a_i = exp(g_i)).  Transposing gives S_n^T q = S0^T w + sum_j c_j v_j with
//     w   = e^{G_n} q - sum_j e^{G_j} c_j k_j
//     c_i = b_i (e^{G_n - G_i} (k_i . q) - sum_{j > i} e^{G_j - G_i} (k_i . k_j) c_j)
// where G_j is the sum of g over the live entries first..j (all exponents are
// <= 0).  The c are one small back substitution over the Gram matrix k_i . k_j
// and the products k_i . q_t, so every window position costs O(n (dk + dv))
// plus O(n^2) scalars, and all T positions share ONE read pass over S0:
// o = scale (S0^T W + ACC).  Everything before that pass depends only on the
// ring and the inputs, so it runs while the S0 loads are in flight.
#include "gdn_device.h"
#include "gdn_launch.h"

// streaming (non-temporal) checkpoint loads and stores for fp32 checkpoints
#ifndef GDN_REPLAY_NT_F32
#define GDN_REPLAY_NT_F32 1
#endif

namespace gdn {

constexpr int kStageRows = 16;  // entry rows staged per batch of loads

// Dynamic LDS (floats): staged entries k, v [E][D+1] (E = L + T), window
// queries [T][D+1], gates (exp(g), g, beta, prefix G) [E] each, Gram matrix
// [E][E], key / query products [E][T], coefficients [T][E], chain vectors w
// and acc [T][D].
__host__ __device__ inline size_t replay_lds_bytes(int D, int L, int T) {
  const size_t E = (size_t)L + (size_t)T;
  return (2 * E * (D + 1) + (size_t)T * (D + 1) + 4 * E + E * E + 2 * E * T + 2 * (size_t)T * D) * sizeof(float);
}

template <int SDT, int D, bool NT, int TB, int EB>
__global__ void __launch_bounds__((TileGeom<SDT, D>::NW * 64))
gdn_replay_kernel(const ReplayArgs P) {
  using G = TileGeom<SDT, D>;
  constexpr int VEC = G::VEC, LPR = G::LPR, RPW = G::RPW, NW = G::NW, PASSES = G::PASSES;
  constexpr int NTH = NW * 64;
  constexpr int LDE = D + 1;  // padded entry rows: per-thread dot products hit distinct banks
  using IO = TileIO<SDT, VEC, NT>;
  using ST = typename StateElem<SDT>::T;
  using Stager = RowStager<D, kStageRows, NTH, EB>;

  extern __shared__ float s_dyn[];
  __shared__ float s_red[2][NW][D];
  __shared__ float s_out[TB][NW][D];

  const DecodeArgs& p = P.d;
  const RingArgs& R = P.ring;
  const int T = P.T;  // 0: flush only
  const int L = R.L;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int b = blockIdx.x / p.Hv;
  const int h = blockIdx.x - b * p.Hv;
  const int hk = h / (p.Hv / p.Hk);
  const int slot = p.slot_map[b];

  if (slot < 0 || (int64_t)slot >= p.num_slots) {  // padded row
    for (int i = tid; i < T * D; i += NTH) {
      const int t = i / D, c = i - t * D;
      store_elem(p.out, (((int64_t)b * T + t) * p.Hv + h) * D + c, 0.f, p.out_dt);
    }
    return;
  }

  const int64_t unit = (int64_t)slot * p.Hv + h;
  // Ring pointers are clamped into range so that a corrupted pointer pair
  // cannot send an access outside this unit's entries.
  int st = R.start[unit];
  int cnt = R.count[unit];
  st = ((st % L) + L) % L;
  cnt = cnt < 0 ? 0 : (cnt > L ? L : cnt);
  const bool fold = (T > 0) ? (cnt + T > L) : (cnt > 0);
  if (T == 0 && !fold) return;  // flush of an empty ring

  ST* tile = static_cast<ST*>(p.pool) + unit * (int64_t)(D * D);
  const int c0 = (lane % LPR) * VEC;
  const int r0 = wave * RPW + lane / LPR;

  typename IO::Raw raw[PASSES];
#pragma unroll
  for (int pp = 0; pp < PASSES; ++pp) raw[pp] = IO::load_raw(tile + (r0 + pp * NW * RPW) * D + c0);

  // ---- stage live entries in LDS: committed ones (live order), then the window
  const int E = L + T;
  float* e_k = s_dyn;               // [E][LDE]
  float* e_v = e_k + E * LDE;       // [E][LDE]
  float* e_q = e_v + E * LDE;       // [T][LDE] window queries
  float* e_a = e_q + T * LDE;       // [E] exp(g)
  float* e_g = e_a + E;             // [E] g
  float* e_b = e_g + E;             // [E] beta
  float* e_G = e_b + E;             // [E] prefix sum of g over the live entries
  float* s_gram = e_G + E;          // [E][E]
  float* s_kq = s_gram + E * E;     // [E][T]
  float* s_c = s_kq + E * T;        // [T][E]
  float* s_w = s_c + T * E;         // [T][D]
  float* s_acc = s_w + T * D;       // [T][D]

  const int64_t ring_e = unit * L;  // first ring entry of this unit
  for (int t = tid; t < cnt + T; t += NTH) {
    if (t < cnt) {
      const int j = (st + t) % L;
      const float g = R.g[ring_e + j];
      e_g[t] = g;
      e_a[t] = expf(g);
      e_b[t] = R.beta[ring_e + j];
    } else {
      const int64_t gi = ((int64_t)b * T + (t - cnt)) * p.Hv + h;
      const float g = gate_g(load_elem(p.a, gi, p.in_dt), p.A_log[h], p.dt_bias[h]);
      e_g[t] = g;
      e_a[t] = expf(g);
      e_b[t] = sigmoid_f(load_elem(p.b, gi, p.in_dt));
    }
  }
  for (int r0s = 0; r0s < cnt; r0s += kStageRows) {  // committed entries, 16 rows per round trip
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
  __syncthreads();

  const int first = fold ? cnt : 0;  // first live entry after an eventual fold
  const int n_all = cnt + T - first;  // live entries of the last window position (<= L)
  if (T > 0) {
    // prefix sums of g over the live entries (one wave; n_all <= 64)
    if (wave == 0) {
      float x = (lane < n_all) ? e_g[first + lane] : 0.f;
#pragma unroll
      for (int off = 1; off < 64; off <<= 1) {
        const float y = __shfl_up(x, off, 64);
        if (lane >= off) x += y;
      }
      if (lane < n_all) e_G[first + lane] = x;
    }
    // Gram matrix of the live keys (upper triangle) and the key / query products
    const int n_gram = n_all * (n_all - 1) / 2;
    for (int task = tid; task < n_gram + n_all * T; task += NTH) {
      float acc = 0.f;
      if (task < n_gram) {  // pair (i, j), i < j, row-major over the upper triangle
        int i = 0, rem = task;
        while (rem >= n_all - 1 - i) {
          rem -= n_all - 1 - i;
          ++i;
        }
        const int j = i + 1 + rem;
        const float* ki = e_k + (first + i) * LDE;
        const float* kj = e_k + (first + j) * LDE;
#pragma unroll 8
        for (int c = 0; c < D; ++c) acc = fmaf(ki[c], kj[c], acc);
        s_gram[(first + i) * E + first + j] = acc;
      } else {
        const int x = task - n_gram, i = x / T, t = x - i * T;
        const float* ki = e_k + (first + i) * LDE;
        const float* qt = e_q + t * LDE;
#pragma unroll 8
        for (int c = 0; c < D; ++c) acc = fmaf(ki[c], qt[c], acc);
        s_kq[(first + i) * T + t] = acc;
      }
    }
  }
  __syncthreads();

  // ---- back substitution for the coefficients of each window position (one wave each)
  for (int t = wave; t < T; t += NW) {
    const int e_last = cnt + t;  // last live entry of position t
    const float Gn = e_G[e_last];
    const int j = first + lane;  // lane holds the residual of live entry j
    const bool live = j <= e_last;
    const float Gj = live ? e_G[j] : 0.f;
    float r = live ? expf(Gn - Gj) * s_kq[j * T + t] : 0.f;
    float cj = 0.f;
    for (int i = e_last; i >= first; --i) {
      // c_i = beta_i * residual_i, then every earlier entry drops its term
      const float ci = __builtin_bit_cast(
          float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, e_b[i] * r), i - first));
      if (j == i) cj = ci;
      if (live && j < i) r = fmaf(-expf(e_G[i] - Gj) * s_gram[j * E + i], ci, r);
    }
    if (live) s_c[t * E + j] = cj;
  }
  __syncthreads();
  // chain vectors: w_t = e^{G_n} q_t - sum_j e^{G_j} c_j k_j,  acc_t = sum_j c_j v_j
  for (int x = tid; x < T * D; x += NTH) {
    const int t = x / D, c = x - t * D;
    const int e_last = cnt + t;
    float w = expf(e_G[e_last]) * e_q[t * LDE + c];
    float acc = 0.f;
    for (int jj = first; jj <= e_last; ++jj) {
      const float cj = s_c[t * E + jj];
      w = fmaf(-expf(e_G[jj]) * cj, e_k[jj * LDE + c], w);
      acc = fmaf(cj, e_v[jj * LDE + c], acc);
    }
    s_w[t * D + c] = w;
    s_acc[t * D + c] = acc;
  }

  // ---- fold the committed entries into the tile, write the checkpoint back
  if (fold) {
    float s[PASSES][VEC];
#pragma unroll
    for (int pp = 0; pp < PASSES; ++pp) IO::widen(raw[pp], s[pp]);
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
      float* red = s_red[i & 1][0];
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
    // one rounding: the stored checkpoint and the tile the outputs read are the rounded values
#pragma unroll
    for (int pp = 0; pp < PASSES; ++pp) {
      raw[pp] = IO::pack_raw(s[pp]);
      IO::store(tile + (r0 + pp * NW * RPW) * D + c0, s[pp]);
    }
  }

  const int new_start = fold ? (st + cnt) % L : st;
  const int base_cnt = fold ? 0 : cnt;

  // ---- append the window to the ring (raw input bytes, gates as fp32)
  for (int i = tid; i < T * D; i += NTH) {
    const int t = i / D, c = i - t * D;
    const int64_t j = ring_e + (new_start + base_cnt + t) % L;
    copy_elem(R.k, j * D + c, p.k, (((int64_t)b * T + t) * p.Hk + hk) * D + c, p.in_dt);
    copy_elem(R.v, j * D + c, p.v, (((int64_t)b * T + t) * p.Hv + h) * D + c, p.in_dt);
  }
  for (int t = tid; t < T; t += NTH) {
    const int64_t j = ring_e + (new_start + base_cnt + t) % L;
    R.g[j] = e_g[cnt + t];
    R.beta[j] = e_b[cnt + t];
  }
  if (tid == 0) {
    R.start[unit] = new_start;
    R.count[unit] = base_cnt + T;
  }
  if (T == 0) return;
  __syncthreads();  // s_w / s_acc complete

  // ---- outputs: o_t = scale (S0^T w_t + acc_t), TB positions per pass over the tile
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
      float o = s_acc[(t0 + tb) * D + c];
#pragma unroll
      for (int w = 0; w < NW; ++w) o += s_out[tb][w][c];
      store_elem(p.out, (((int64_t)b * T + t0 + tb) * p.Hv + h) * D + c, p.scale * o, p.out_dt);
    }
    __syncthreads();
  }
}

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

template <int SDT, int D, int TB, int EB>
static hipError_t launch_replay_k(const ReplayArgs& a, hipStream_t s) {
  using G = TileGeom<SDT, D>;
  constexpr bool NT = (SDT == GDN_F32) && (GDN_REPLAY_NT_F32 != 0);
  const unsigned grid = (unsigned)((int64_t)a.d.B * a.d.Hv);
  const size_t lds = replay_lds_bytes(D, a.ring.L, a.T);
  hipLaunchKernelGGL((gdn_replay_kernel<SDT, D, NT, TB, EB>), dim3(grid), dim3(G::NW * 64), lds, s, a);
  return hipGetLastError();
}

template <int SDT, int D>
static hipError_t launch_replay_t(const ReplayArgs& a, hipStream_t s) {
  const bool f32_in = a.d.in_dt == GDN_F32;
  if (a.T <= 1)
    return f32_in ? launch_replay_k<SDT, D, 1, 4>(a, s) : launch_replay_k<SDT, D, 1, 2>(a, s);
  return f32_in ? launch_replay_k<SDT, D, 4, 4>(a, s) : launch_replay_k<SDT, D, 4, 2>(a, s);
}

template <int SDT>
static hipError_t launch_replay_sdt(const ReplayArgs& a, int D, hipStream_t s) {
  switch (D) {
    case 16: return launch_replay_t<SDT, 16>(a, s);
    case 32: return launch_replay_t<SDT, 32>(a, s);
    case 64: return launch_replay_t<SDT, 64>(a, s);
    case 128: return launch_replay_t<SDT, 128>(a, s);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_replay(const ReplayArgs& a, int state_dt, int D, hipStream_t s) {
  if (a.d.B == 0) return hipSuccess;
  switch (state_dt) {
    case GDN_F32: return launch_replay_sdt<GDN_F32>(a, D, s);
    case GDN_BF16: return launch_replay_sdt<GDN_BF16>(a, D, s);
    case GDN_F16: return launch_replay_sdt<GDN_F16>(a, D, s);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_replay_flush(const ReplayArgs& a, int state_dt, int D, hipStream_t s) {
  ReplayArgs f = a;
  f.T = 0;
  return launch_replay(f, state_dt, D, s);
}

hipError_t launch_replay_rollback(const ReplayArgs& a, hipStream_t s) {
  if (a.d.B == 0) return hipSuccess;
  const int64_t n = (int64_t)a.d.B * a.d.Hv;
  const unsigned grid = (unsigned)((n + 255) / 256);
  hipLaunchKernelGGL(gdn_replay_rollback_kernel, dim3(grid), dim3(256), 0, s, a);
  return hipGetLastError();
}

// static LDS of the widest instantiation (TB = 4)
template <int SDT, int D>
static size_t replay_static_lds() {
  using G = TileGeom<SDT, D>;
  return (size_t)(2 + 4) * G::NW * D * sizeof(float);
}

template <int SDT>
static size_t replay_static_lds_sdt(int D) {
  switch (D) {
    case 16: return replay_static_lds<SDT, 16>();
    case 32: return replay_static_lds<SDT, 32>();
    case 64: return replay_static_lds<SDT, 64>();
    default: return replay_static_lds<SDT, 128>();
  }
}

size_t replay_lds_total(int state_dt, int D, int L, int T) {
  const size_t st = state_dt == GDN_F32 ? replay_static_lds_sdt<GDN_F32>(D) : replay_static_lds_sdt<GDN_BF16>(D);
  return st + replay_lds_bytes(D, L, T);
}

}  // namespace gdn
