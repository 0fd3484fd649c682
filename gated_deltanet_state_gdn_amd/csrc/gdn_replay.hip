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
//   3. window position t outputs scale * S_t^T q_t with S_t = S0 advanced over
//      the live entries up to t, WITHOUT materialising S_t.  Unrolling
//      S_i = a_i (I - b_i k_i k_i^T) S_{i-1} + b_i k_i v_i^T and transposing
//      gives the adjoint chain
//          w <- q;  for i = n-1 .. 0:  c = b_i (k_i . w);  acc += c v_i;
//                                        w <- a_i (w - c k_i)
//          S_n^T q = S0^T w + acc
//      (a_i = exp(g_i)), so each position costs O(n (dk + dv)) for its chain
//      and all T positions share ONE read pass over S0: o = S0^T W + ACC.
// The chains depend only on the ring, so they run while the S0 loads are in
// flight.
#include "gdn_device.h"
#include "gdn_launch.h"

namespace gdn {

constexpr int kReplayTB = 4;  // window positions reduced per output pass

template <int DT>
__device__ __forceinline__ float storage_roundtrip(float x) {
  if constexpr (DT == GDN_F32) {
    return x;
  } else {
    return unpack_lo<DT>(pack2<DT>(x, 0.f));
  }
}

// Dynamic LDS: staged entries (k, v, alpha, g, beta) for E = L + T slots, then
// the chain results w and acc for T window positions.
__host__ __device__ inline size_t replay_lds_bytes(int D, int L, int T) {
  const size_t E = (size_t)L + (size_t)T;
  return (E * (2 * (size_t)D + 3) + 2 * (size_t)T * D) * sizeof(float);
}

template <int SDT, int D, bool NT>
__global__ void __launch_bounds__((TileGeom<SDT, D>::NW * 64))
gdn_replay_kernel(const ReplayArgs P) {
  using G = TileGeom<SDT, D>;
  constexpr int VEC = G::VEC, LPR = G::LPR, RPW = G::RPW, NW = G::NW, PASSES = G::PASSES;
  constexpr int NTH = NW * 64;
  constexpr int DL = (D + 63) / 64;  // chain elements per lane
  constexpr int TB = kReplayTB;
  using IO = TileIO<SDT, VEC, NT>;
  using ST = typename StateElem<SDT>::T;

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

  float s[PASSES][VEC];
#pragma unroll
  for (int pp = 0; pp < PASSES; ++pp) IO::load(tile + (r0 + pp * NW * RPW) * D + c0, s[pp]);

  // ---- stage live entries in LDS: committed ones (live order), then the window
  const int E = L + T;
  float* e_k = s_dyn;              // [E][D]
  float* e_v = e_k + E * D;        // [E][D]
  float* e_a = e_v + E * D;        // [E]  exp(g)
  float* e_g = e_a + E;            // [E]
  float* e_b = e_g + E;            // [E]
  float* s_w = e_b + E;            // [T][D]
  float* s_acc = s_w + T * D;      // [T][D]

  const int64_t ring_e = unit * L;  // first ring entry of this unit
  for (int i = tid; i < cnt * D; i += NTH) {
    const int e = i / D, c = i - e * D;
    const int j = (st + e) % L;
    e_k[e * D + c] = load_elem(R.k, (ring_e + j) * D + c, p.in_dt);
    e_v[e * D + c] = load_elem(R.v, (ring_e + j) * D + c, p.in_dt);
  }
  for (int e = tid; e < cnt; e += NTH) {
    const int j = (st + e) % L;
    const float g = R.g[ring_e + j];
    e_g[e] = g;
    e_a[e] = expf(g);
    e_b[e] = R.beta[ring_e + j];
  }
  for (int i = tid; i < T * D; i += NTH) {
    const int t = i / D, c = i - t * D;
    e_k[(cnt + t) * D + c] = load_elem(p.k, (((int64_t)b * T + t) * p.Hk + hk) * D + c, p.in_dt);
    e_v[(cnt + t) * D + c] = load_elem(p.v, (((int64_t)b * T + t) * p.Hv + h) * D + c, p.in_dt);
  }
  for (int t = tid; t < T; t += NTH) {
    const int64_t gi = ((int64_t)b * T + t) * p.Hv + h;
    const float g = gate_g(load_elem(p.a, gi, p.in_dt), p.A_log[h], p.dt_bias[h]);
    e_g[cnt + t] = g;
    e_a[cnt + t] = expf(g);
    e_b[cnt + t] = sigmoid_f(load_elem(p.b, gi, p.in_dt));
  }
  __syncthreads();

  // ---- window chains (independent of S0; overlap the tile loads)
  const int first = fold ? cnt : 0;  // first live entry after an eventual fold
  for (int t = wave; t < T; t += NW) {
    float w[DL], acc[DL];
#pragma unroll
    for (int j = 0; j < DL; ++j) {
      const int c = lane + 64 * j;
      w[j] = (c < D) ? load_elem(p.q, (((int64_t)b * T + t) * p.Hk + hk) * D + c, p.in_dt) : 0.f;
      acc[j] = 0.f;
    }
    for (int i = cnt + t; i >= first; --i) {
      float dot = 0.f;
#pragma unroll
      for (int j = 0; j < DL; ++j) {
        const int c = lane + 64 * j;
        if (c < D) dot = fmaf(e_k[i * D + c], w[j], dot);
      }
      const float cf = e_b[i] * wave_sum(dot);
      const float al = e_a[i];
#pragma unroll
      for (int j = 0; j < DL; ++j) {
        const int c = lane + 64 * j;
        if (c < D) {
          acc[j] = fmaf(cf, e_v[i * D + c], acc[j]);
          w[j] = al * fmaf(-cf, e_k[i * D + c], w[j]);
        }
      }
    }
#pragma unroll
    for (int j = 0; j < DL; ++j) {
      const int c = lane + 64 * j;
      if (c < D) {
        s_w[t * D + c] = w[j];
        s_acc[t * D + c] = acc[j];
      }
    }
  }

  // ---- fold the committed entries into the tile, write the checkpoint back
  if (fold) {
    for (int i = 0; i < cnt; ++i) {
      const float* ki = e_k + i * D;
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
        delta[e] = be * (e_v[i * D + c0 + e] - al * kv);
      }
#pragma unroll
      for (int pp = 0; pp < PASSES; ++pp) {
        const float kr = ki[r0 + pp * NW * RPW];
#pragma unroll
        for (int e = 0; e < VEC; ++e) s[pp][e] = fmaf(al, s[pp][e], kr * delta[e]);
      }
    }
#pragma unroll
    for (int pp = 0; pp < PASSES; ++pp) {
      IO::store(tile + (r0 + pp * NW * RPW) * D + c0, s[pp]);
#pragma unroll
      for (int e = 0; e < VEC; ++e) s[pp][e] = storage_roundtrip<SDT>(s[pp][e]);
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
#pragma unroll
      for (int tb = 0; tb < TB; ++tb) {
        if (tb < nt) {
          const float wr = s_w[(t0 + tb) * D + r];
#pragma unroll
          for (int e = 0; e < VEC; ++e) part[tb][e] = fmaf(s[pp][e], wr, part[tb][e]);
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

template <int SDT, int D>
static hipError_t launch_replay_t(const ReplayArgs& a, hipStream_t s) {
  using G = TileGeom<SDT, D>;
  const unsigned grid = (unsigned)((int64_t)a.d.B * a.d.Hv);
  const size_t lds = replay_lds_bytes(D, a.ring.L, a.T);
  hipLaunchKernelGGL((gdn_replay_kernel<SDT, D, false>), dim3(grid), dim3(G::NW * 64), lds, s, a);
  return hipGetLastError();
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

template <int SDT, int D>
static size_t replay_static_lds() {
  using G = TileGeom<SDT, D>;
  return (size_t)(2 + kReplayTB) * G::NW * D * sizeof(float);
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
