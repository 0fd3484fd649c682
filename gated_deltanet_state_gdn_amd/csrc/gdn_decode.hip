// Single-token GDN decode: one workgroup per (sequence, value head) streams the
// dk x dv state tile once in and once out.
//
// Operation (vLLM PR #52191 page, implementation item 3, the fused
// sigmoid-gating delta-rule update; item 4, FP32 math with one rounding per
// write-back): with alpha = exp(g),
//     kv    = S^T k,  qs = S^T q            (one read pass over S)
//     delta = beta (v - alpha kv)
//     S'    = alpha S + k delta^T            (written back, rounded once)
//     o     = scale S'^T q = scale (alpha qs + (k.q) delta)
// The identity for o lets both column sums come from the single read pass, so
// the state is read once and written once (the whole-state read and write per
// step that the AREX ReplaySSM article's "bottleneck" section names as the
// dominant traffic).
//
// Memory: a wave reads RPW full rows per pass with 8/16-byte lane accesses
// (coalesced; a 128-float row is 512 contiguous bytes), all passes are issued
// before any arithmetic so the tile is in flight at once, and the tile stays
// in VGPRs between the read and the write.
#include "gdn_device.h"
#include "gdn_launch.h"

// Launch tuning (measured on MI355X): waves per workgroup (4 for fp32 tiles,
// 2 for 16-bit ones, which then carry as many bytes per lane); fp32 tiles are
// read and written non-temporally (+7%), 16-bit ones read non-temporally when
// the launch's tiles exceed the Infinity Cache (stream_tile_reads) and also
// written so past twice that (stream_tile_writes).
#ifndef GDN_DECODE_WAVES
#define GDN_DECODE_WAVES 4
#endif
#ifndef GDN_DECODE_WAVES_16
#define GDN_DECODE_WAVES_16 2
#endif
#ifndef GDN_DECODE_NT_F32
#define GDN_DECODE_NT_F32 1
#endif
#ifndef GDN_DECODE_NT_16
#define GDN_DECODE_NT_16 0
#endif

namespace gdn {

template <int SDT, int D>
using DecodeGeom = TileGeom<SDT, D, SDT == GDN_F32 ? GDN_DECODE_WAVES : GDN_DECODE_WAVES_16>;

// NT: non-temporal stores (and loads); NTL: non-temporal loads
template <int SDT, int D, bool NT, bool NTL>
__global__ void __launch_bounds__((DecodeGeom<SDT, D>::NW * 64))
gdn_decode_kernel(const DecodeArgs p) {
  using G = DecodeGeom<SDT, D>;
  constexpr int VEC = G::VEC, LPR = G::LPR, RPW = G::RPW, NW = G::NW, PASSES = G::PASSES;
  constexpr int NT_THREADS = NW * 64;
  using IO = TileIO<SDT, VEC, NT>;
  using ST = typename StateElem<SDT>::T;

  __shared__ float s_k[D], s_q[D];
  __shared__ float s_red[2][NW][D];
  __shared__ float s_kq;

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int b = blockIdx.x / p.Hv;
  const int h = blockIdx.x - b * p.Hv;
  const int hk = h / (p.Hv / p.Hk);
  const int slot = p.slot_map[b];
  const int64_t row_bh = (int64_t)b * p.Hv + h;

  if (slot < 0 || (int64_t)slot >= p.num_slots) {  // padded row
    for (int i = tid; i < D; i += NT_THREADS) store_elem(p.out, row_bh * D + i, 0.f, p.out_dt);
    return;
  }

  ST* tile = static_cast<ST*>(p.pool) + ((int64_t)slot * p.Hv + h) * (int64_t)(D * D);
  const int c0 = (lane % LPR) * VEC;
  const int r0 = wave * RPW + lane / LPR;  // row of pass 0; pass pp adds pp * NW * RPW

  typename IO::Raw raw[PASSES];
#pragma unroll
  for (int pp = 0; pp < PASSES; ++pp) raw[pp] = TileIO<SDT, VEC, NT || NTL>::load_raw(tile + (r0 + pp * NW * RPW) * D + c0);

  // gates (uniform over the workgroup)
  const float g = gate_g(load_elem(p.a, row_bh, p.in_dt), p.A_log[h], p.dt_bias[h]);
  const float beta = sigmoid_f(load_elem(p.b, row_bh, p.in_dt));
  const float alpha = expf(g);

  const int64_t kq_base = ((int64_t)b * p.Hk + hk) * D;
  for (int i = tid; i < D; i += NT_THREADS) {
    s_k[i] = load_elem(p.k, kq_base + i, p.in_dt);
    s_q[i] = load_elem(p.q, kq_base + i, p.in_dt);
  }
  float vv[VEC];
#pragma unroll
  for (int e = 0; e < VEC; ++e) vv[e] = load_elem(p.v, row_bh * D + c0 + e, p.in_dt);
  __syncthreads();

  float kvp[VEC], qsp[VEC];
#pragma unroll
  for (int e = 0; e < VEC; ++e) kvp[e] = qsp[e] = 0.f;
#pragma unroll
  for (int pp = 0; pp < PASSES; ++pp) {
    const int r = r0 + pp * NW * RPW;
    const float kr = s_k[r], qr = s_q[r];
    float sv[VEC];
    IO::widen(raw[pp], sv);
#pragma unroll
    for (int e = 0; e < VEC; ++e) {
      kvp[e] = fmaf(sv[e], kr, kvp[e]);
      qsp[e] = fmaf(sv[e], qr, qsp[e]);
    }
  }
#pragma unroll
  for (int e = 0; e < VEC; ++e) {
    kvp[e] = xor_sum_from<LPR>(kvp[e]);
    qsp[e] = xor_sum_from<LPR>(qsp[e]);
  }
  if (lane < LPR) {
#pragma unroll
    for (int e = 0; e < VEC; ++e) {
      s_red[0][wave][c0 + e] = kvp[e];
      s_red[1][wave][c0 + e] = qsp[e];
    }
  }
  if (wave == 0) {
    float t = 0.f;
    for (int i = lane; i < D; i += 64) t = fmaf(s_k[i], s_q[i], t);
    t = wave_sum(t);
    if (lane == 0) s_kq = t;
  }
  __syncthreads();

  // Keep only the packed tile live across the barrier: without this the
  // compiler reuses the widened values of the first pass (twice the VGPRs for
  // a 16-bit tile, half the tiles in flight per CU).
  if constexpr (SDT != GDN_F32) {
#pragma unroll
    for (int pp = 0; pp < PASSES; ++pp)
#pragma unroll
      for (int w = 0; w < IO::WORDS; ++w) asm volatile("" : "+v"(raw[pp][w]));
  }
  const float kq = s_kq;
  float delta[VEC];
#pragma unroll
  for (int e = 0; e < VEC; ++e) {
    float kv = 0.f, qs = 0.f;
#pragma unroll
    for (int w = 0; w < NW; ++w) {
      kv += s_red[0][w][c0 + e];
      qs += s_red[1][w][c0 + e];
    }
    delta[e] = beta * (vv[e] - alpha * kv);
    if (wave == 0 && lane < LPR)
      store_elem(p.out, row_bh * D + c0 + e, p.scale * fmaf(alpha, qs, kq * delta[e]), p.out_dt);
  }

#pragma unroll
  for (int pp = 0; pp < PASSES; ++pp) {
    const int r = r0 + pp * NW * RPW;
    const float kr = s_k[r];
    float sv[VEC];
    IO::widen(raw[pp], sv);
#pragma unroll
    for (int e = 0; e < VEC; ++e) sv[e] = fmaf(alpha, sv[e], kr * delta[e]);
    IO::store(tile + r * D + c0, sv);
  }
}

template <int SDT, int D>
static hipError_t launch_decode_t(const DecodeArgs& a, hipStream_t s) {
  using G = DecodeGeom<SDT, D>;
  const unsigned grid = (unsigned)((int64_t)a.B * a.Hv);
  constexpr bool NT = (SDT == GDN_F32) ? (GDN_DECODE_NT_F32 != 0) : (GDN_DECODE_NT_16 != 0);
  const long long tile_bytes = (long long)grid * D * D * (long long)sizeof(typename StateElem<SDT>::T);
  if (!NT && stream_tile_writes(tile_bytes))
    hipLaunchKernelGGL((gdn_decode_kernel<SDT, D, true, true>), dim3(grid), dim3(G::NW * 64), 0, s, a);
  else if (stream_tile_reads(tile_bytes))
    hipLaunchKernelGGL((gdn_decode_kernel<SDT, D, NT, true>), dim3(grid), dim3(G::NW * 64), 0, s, a);
  else
    hipLaunchKernelGGL((gdn_decode_kernel<SDT, D, NT, false>), dim3(grid), dim3(G::NW * 64), 0, s, a);
  return hipGetLastError();
}

template <int SDT>
static hipError_t launch_decode_sdt(const DecodeArgs& a, int D, hipStream_t s) {
  switch (D) {
    case 16: return launch_decode_t<SDT, 16>(a, s);
    case 32: return launch_decode_t<SDT, 32>(a, s);
    case 64: return launch_decode_t<SDT, 64>(a, s);
    case 128: return launch_decode_t<SDT, 128>(a, s);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_decode(const DecodeArgs& a, int state_dt, int D, hipStream_t s) {
  if (a.B == 0) return hipSuccess;
  switch (state_dt) {
    case GDN_F32: return launch_decode_sdt<GDN_F32>(a, D, s);
    case GDN_BF16: return launch_decode_sdt<GDN_BF16>(a, D, s);
    case GDN_F16: return launch_decode_sdt<GDN_F16>(a, D, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace gdn
