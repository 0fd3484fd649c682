// Speculative decode that keeps one full state per window position: the
// per-draft-token baseline that ReplaySSM's speculative replay replaces (vLLM
// PR #52191 page, the speculative update kernel with templated source and
// destination state pointers; AREX ReplaySSM article, "bottleneck" section:
// (1 + num_spec) full states per step, written whether or not the drafts are
// accepted).
//
// One workgroup per (sequence, value head).  The source state is read once
// into VGPRs as fp32 and advanced token by token:
//     kv_t = S^T k_t,  qs_t = S^T q_t,  delta_t = beta_t (v_t - alpha_t kv_t)
//     S   <- alpha_t S + k_t delta_t^T          (written, rounded once, to dst[t])
//     o_t  = scale (alpha_t qs_t + (k_t . q_t) delta_t)
// The chain carries the unrounded fp32 state, so each destination holds the
// state after its token rounded exactly once.  Per token the column sums need
// one cross-wave reduction (double-buffered, one barrier per token); the
// source is read once and each of the T destination tiles is written once.
#include "gdn_device.h"
#include "gdn_launch.h"

// fp32 tiles are read and written non-temporally; 16-bit source tiles are
// read non-temporally when the launch's tiles exceed the Infinity Cache, and
// 16-bit tiles are written so when the T destinations exceed twice that
#ifndef GDN_SPEC_NT_F32
#define GDN_SPEC_NT_F32 1
#endif

// one-shot workgroups take their units in XCD-aware order (xcd_unit) when the
// tiles stream past the Infinity Cache both ways (fp32 B = 512, T = 5: 1.311 ->
// 1.259 ms; bf16 unchanged within the noise)
#ifndef GDN_SPEC_XCD
#define GDN_SPEC_XCD 1
#endif

namespace gdn {

// Four waves for every state dtype: the working tile is fp32 in VGPRs, so a
// 16-bit tile needs as many lanes as an fp32 one.
template <int SDT, int D>
using SpecGeom = TileGeom<SDT, D, 4>;

// Dynamic LDS (floats): k, q, v [T][D] each, then alpha, beta, k.q [T] each.
size_t spec_lds_bytes(int D, int T) { return ((size_t)3 * T * D + 3 * (size_t)T) * sizeof(float); }

template <int SDT, int D, bool NT, bool NTL>
__global__ void __launch_bounds__((SpecGeom<SDT, D>::NW * 64)) gdn_spec_kernel(const SpecArgs P) {
  using G = SpecGeom<SDT, D>;
  constexpr int VEC = G::VEC, LPR = G::LPR, RPW = G::RPW, NW = G::NW, PASSES = G::PASSES;
  constexpr int NTH = NW * 64;
  using IO = TileIO<SDT, VEC, NT>;
  using ST = typename StateElem<SDT>::T;
  extern __shared__ float s_dyn[];
  __shared__ float s_red[2][2][NW][D];

  const DecodeArgs& p = P.d;
  const int T = P.T;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  constexpr bool XO = GDN_SPEC_XCD != 0 && NT && NTL;  // tiles streamed both ways: XCD-aware order
  const int u = XO ? xcd_unit(blockIdx.x, gridDim.x) : (int)blockIdx.x;
  const int b = u / p.Hv;
  const int h = u - b * p.Hv;
  const int hk = h / (p.Hv / p.Hk);
  const int src = p.slot_map[b];

  if (src < 0 || (int64_t)src >= p.num_slots) {  // padded row: zero outputs, nothing written
    for (int i = tid; i < T * D; i += NTH) {
      const int t = i / D, c = i - t * D;
      store_elem(p.out, (((int64_t)b * T + t) * p.Hv + h) * D + c, 0.f, p.out_dt);
    }
    return;
  }

  const int c0 = (lane % LPR) * VEC;
  const int r0 = wave * RPW + lane / LPR;  // row of pass 0; pass pp adds pp * NW * RPW
  const ST* stile = static_cast<const ST*>(p.pool) + ((int64_t)src * p.Hv + h) * (int64_t)(D * D);
  float s[PASSES][VEC];
  {
    typename IO::Raw raw[PASSES];
#pragma unroll
    for (int pp = 0; pp < PASSES; ++pp) raw[pp] = TileIO<SDT, VEC, NT || NTL>::load_raw(stile + (r0 + pp * NW * RPW) * D + c0);
#pragma unroll
    for (int pp = 0; pp < PASSES; ++pp) IO::widen(raw[pp], s[pp]);
  }

  float* s_k = s_dyn;           // [T][D]
  float* s_q = s_k + T * D;     // [T][D]
  float* s_v = s_q + T * D;     // [T][D]
  float* s_al = s_v + T * D;    // [T] exp(g)
  float* s_be = s_al + T;       // [T]
  float* s_kq = s_be + T;       // [T]
  for (int i = tid; i < T * D; i += NTH) {
    const int t = i / D, c = i - t * D;
    const int64_t kq = (((int64_t)b * T + t) * p.Hk + hk) * D + c;
    s_k[i] = load_elem(p.k, kq, p.in_dt);
    s_q[i] = load_elem(p.q, kq, p.in_dt);
    s_v[i] = load_elem(p.v, (((int64_t)b * T + t) * p.Hv + h) * D + c, p.in_dt);
  }
  if (tid < T) {
    const int64_t gi = ((int64_t)b * T + tid) * p.Hv + h;
    s_al[tid] = expf(gate_g(load_elem(p.a, gi, p.in_dt), p.A_log[h], p.dt_bias[h]));
    s_be[tid] = sigmoid_f(load_elem(p.b, gi, p.in_dt));
  }
  __syncthreads();
  for (int t = wave; t < T; t += NW) {
    float x = 0.f;
    for (int i = lane; i < D; i += 64) x = fmaf(s_k[t * D + i], s_q[t * D + i], x);
    x = wave_sum(x);
    if (lane == 0) s_kq[t] = x;
  }
  // (s_kq is read after the first reduction barrier below)

  for (int t = 0; t < T; ++t) {
    const float* kt = s_k + t * D;
    const float* qt = s_q + t * D;
    float kvp[VEC], qsp[VEC];
#pragma unroll
    for (int e = 0; e < VEC; ++e) kvp[e] = qsp[e] = 0.f;
#pragma unroll
    for (int pp = 0; pp < PASSES; ++pp) {
      const int r = r0 + pp * NW * RPW;
      const float kr = kt[r], qr = qt[r];
#pragma unroll
      for (int e = 0; e < VEC; ++e) {
        kvp[e] = fmaf(s[pp][e], kr, kvp[e]);
        qsp[e] = fmaf(s[pp][e], qr, qsp[e]);
      }
    }
#pragma unroll
    for (int e = 0; e < VEC; ++e) {
      kvp[e] = xor_sum_from<LPR>(kvp[e]);
      qsp[e] = xor_sum_from<LPR>(qsp[e]);
    }
    float(*red)[NW][D] = s_red[t & 1];  // double-buffered: one barrier per token
    if (lane < LPR) {
#pragma unroll
      for (int e = 0; e < VEC; ++e) {
        red[0][wave][c0 + e] = kvp[e];
        red[1][wave][c0 + e] = qsp[e];
      }
    }
    __syncthreads();

    const float alpha = s_al[t], beta = s_be[t], kq = s_kq[t];
    float delta[VEC];
#pragma unroll
    for (int e = 0; e < VEC; ++e) {
      float kv = 0.f, qs = 0.f;
#pragma unroll
      for (int w = 0; w < NW; ++w) {
        kv += red[0][w][c0 + e];
        qs += red[1][w][c0 + e];
      }
      delta[e] = beta * (s_v[t * D + c0 + e] - alpha * kv);
      if (wave == 0 && lane < LPR)
        store_elem(p.out, (((int64_t)b * T + t) * p.Hv + h) * D + c0 + e, p.scale * fmaf(alpha, qs, kq * delta[e]),
                   p.out_dt);
    }
#pragma unroll
    for (int pp = 0; pp < PASSES; ++pp) {
      const float kr = kt[r0 + pp * NW * RPW];
#pragma unroll
      for (int e = 0; e < VEC; ++e) s[pp][e] = fmaf(alpha, s[pp][e], kr * delta[e]);
    }
    const int dst = P.dst_slots[(int64_t)b * T + t];
    if (dst >= 0 && (int64_t)dst < p.num_slots) {
      ST* dtile = static_cast<ST*>(p.pool) + ((int64_t)dst * p.Hv + h) * (int64_t)(D * D);
#pragma unroll
      for (int pp = 0; pp < PASSES; ++pp) IO::store(dtile + (r0 + pp * NW * RPW) * D + c0, s[pp]);
    }
  }
}

template <int SDT, int D>
static hipError_t launch_spec_t(const SpecArgs& a, hipStream_t s) {
  using G = SpecGeom<SDT, D>;
  constexpr bool NT = (SDT == GDN_F32) && (GDN_SPEC_NT_F32 != 0);
  const unsigned grid = (unsigned)((int64_t)a.d.B * a.d.Hv);
  const long long tile_bytes = (long long)grid * D * D * (long long)sizeof(typename StateElem<SDT>::T);
  if (!NT && stream_tile_writes(tile_bytes * a.T))  // the T destination tiles
    hipLaunchKernelGGL((gdn_spec_kernel<SDT, D, true, true>), dim3(grid), dim3(G::NW * 64), spec_lds_bytes(D, a.T), s, a);
  else if (stream_tile_reads(tile_bytes))
    hipLaunchKernelGGL((gdn_spec_kernel<SDT, D, NT, true>), dim3(grid), dim3(G::NW * 64), spec_lds_bytes(D, a.T), s, a);
  else
    hipLaunchKernelGGL((gdn_spec_kernel<SDT, D, NT, false>), dim3(grid), dim3(G::NW * 64), spec_lds_bytes(D, a.T), s, a);
  return hipGetLastError();
}

template <int SDT>
static hipError_t launch_spec_sdt(const SpecArgs& a, int D, hipStream_t s) {
  switch (D) {
    case 16: return launch_spec_t<SDT, 16>(a, s);
    case 32: return launch_spec_t<SDT, 32>(a, s);
    case 64: return launch_spec_t<SDT, 64>(a, s);
    case 128: return launch_spec_t<SDT, 128>(a, s);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_spec(const SpecArgs& a, int state_dt, int D, hipStream_t s) {
  if (a.d.B == 0 || a.T == 0) return hipSuccess;
  switch (state_dt) {
    case GDN_F32: return launch_spec_sdt<GDN_F32>(a, D, s);
    case GDN_BF16: return launch_spec_sdt<GDN_BF16>(a, D, s);
    case GDN_F16: return launch_spec_sdt<GDN_F16>(a, D, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace gdn
