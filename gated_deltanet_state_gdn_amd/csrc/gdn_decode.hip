// Single-token GDN decode: each (sequence, value head) streams its dk x dv
// state tile once in and once out, one workgroup per tile (the one-shot
// kernel) or, for fp32 128 x 128 tiles, one workgroup per CU walking the tiles
// (the persistent kernel below).
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

// Launch tuning (measured on MI355X): waves per workgroup (4 for fp32 tiles;
// for 16-bit ones 2, which then carry as many bytes per lane, 4 once the
// launch's tiles exceed the Infinity Cache, and 8 once its stores stream too);
// fp32 tiles are
// read and written non-temporally (+7%), 16-bit ones read non-temporally when
// the launch's tiles exceed the Infinity Cache (stream_tile_reads) and also
// written so past twice that (stream_tile_writes).
#ifndef GDN_DECODE_WAVES
#define GDN_DECODE_WAVES 4
#endif
#ifndef GDN_DECODE_WAVES_16
#define GDN_DECODE_WAVES_16 2
#endif
// 16-bit tiles streamed both ways (non-temporal reads and stores): one-shot
// workgroups take their units in XCD-aware order (xcd_unit), bf16 B = 512
// 0.2025 -> 0.1968 ms, f16 0.2016 -> 0.1973.  Where the tiles stay in the
// Infinity Cache between steps the plain order stays ahead (bf16 B = 256
// 0.0897 against 0.0931, fp32 B = 64 0.0501 against 0.0520).
#ifndef GDN_DECODE_XCD
#define GDN_DECODE_XCD 1
#endif
// 16-bit tiles read past the Infinity Cache (stream_tile_reads): bf16 B = 256
// 0.0939 -> 0.0897 ms, B = 512 0.2059 -> 0.2017 ms against two waves; at B = 64
// (cache-resident) two waves stay ahead, 0.0228 against 0.0248 ms
#ifndef GDN_DECODE_WAVES_16_STREAM
#define GDN_DECODE_WAVES_16_STREAM 4
#endif
// 16-bit tiles streamed both ways (B = 512): eight waves, whose column sums take
// two levels (one thread per column adds the waves' partials, then every lane
// reads its totals): bf16 0.1962 -> 0.1924 ms, f16 0.1966 -> 0.1929 (with the
// sums in one level, as four waves take them, eight waves ran 0.207)
#ifndef GDN_DECODE_WAVES_16_STREAM2
#define GDN_DECODE_WAVES_16_STREAM2 8
#endif
#ifndef GDN_DECODE_RED2
#define GDN_DECODE_RED2 1
#endif
#ifndef GDN_DECODE_NT_F32
#define GDN_DECODE_NT_F32 1
#endif
#ifndef GDN_DECODE_NT_16
#define GDN_DECODE_NT_16 0
#endif
// fp32 128 x 128 tiles go through the persistent 16-wave kernel
#ifndef GDN_DECODE_PERSIST
#define GDN_DECODE_PERSIST 1
#endif
// 16-bit 128 x 128 tiles through the persistent 8-wave kernel (measured slower)
#ifndef GDN_DECODE_PERSIST_16
#define GDN_DECODE_PERSIST_16 0
#endif

namespace gdn {

template <int SDT, int D, int NWG = (SDT == GDN_F32 ? GDN_DECODE_WAVES : GDN_DECODE_WAVES_16)>
using DecodeGeom = TileGeom<SDT, D, NWG>;

// NT: non-temporal stores (and loads); NTL: non-temporal loads; IDT: the input dtype;
// NWG: waves per workgroup
template <int SDT, int D, bool NT, bool NTL, int IDT, int NWG>
__global__ void __launch_bounds__(NWG * 64)
gdn_decode_kernel(const DecodeArgs p) {
  using G = DecodeGeom<SDT, D, NWG>;
  constexpr int VEC = G::VEC, LPR = G::LPR, RPW = G::RPW, NW = G::NW, PASSES = G::PASSES;
  constexpr int NT_THREADS = NW * 64;
  using IO = TileIO<SDT, VEC, NT>;
  using ST = typename StateElem<SDT>::T;

  __shared__ float s_k[D], s_q[D];
  __shared__ float s_red[2][NW][D];
  __shared__ float s_kq;

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  constexpr bool XO = GDN_DECODE_XCD != 0 && SDT != GDN_F32 && NT && NTL;
  const int u = XO ? xcd_unit(blockIdx.x, gridDim.x) : (int)blockIdx.x;
  const int b = u / p.Hv;
  const int h = u - b * p.Hv;
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

  // The small loads go out first, as raw bits: both gate inputs in one access
  // (lane 0 reads a, lane 1 b), k and q for staging (8 elements per lane, one
  // access each) and this lane's VEC values (one access).  Loads complete in
  // order, so the waits for them do not cover the tile loads issued after.
  const uint32_t gab = in_bits<IDT>(lane == 1 ? p.b : p.a, row_bh);
  const float A_log = p.A_log[h], dt_bias = p.dt_bias[h];
  const int64_t kq_base = ((int64_t)b * p.Hk + hk) * D;
  const bool stager = tid < 2 * (D / 8);
  const int which = tid / (D / 8), kq_i = (tid - which * (D / 8)) * 8;
  InVec<IDT, 8> kqr;
  if (stager) kqr.load(which ? p.q : p.k, kq_base + kq_i);
  InVec<IDT, VEC> vr;
  vr.load(p.v, row_bh * D + c0);

  typename IO::Raw raw[PASSES];
#pragma unroll
  for (int pp = 0; pp < PASSES; ++pp) raw[pp] = TileIO<SDT, VEC, NT || NTL>::load_raw(tile + (r0 + pp * NW * RPW) * D + c0);

  // gates (uniform over the workgroup)
  const float g = gate_g(in_value<IDT>(__builtin_amdgcn_readlane(gab, 0)), A_log, dt_bias);
  const float beta = sigmoid_f(in_value<IDT>(__builtin_amdgcn_readlane(gab, 1)));
  const float alpha = expf(g);

  if (stager) {
    float f[8];
    kqr.widen(f);
    float* dst = (which ? s_q : s_k) + kq_i;
#pragma unroll
    for (int e = 0; e < 8; ++e) dst[e] = f[e];
  }
  float vv[VEC];
  vr.widen(vv);
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
  // eight or more waves: one thread per (sum, column) adds the waves' partials
  // (one barrier more, a sixteenth of the LDS reads per lane)
  constexpr bool RED2 = GDN_DECODE_RED2 != 0 && NW >= 8;
  __shared__ float s_tot[RED2 ? 2 : 1][RED2 ? D : 1];
  if constexpr (RED2) {
    if (tid < 2 * D) {
      const int kind = tid / D, c = tid - kind * D;
      float t = 0.f;
#pragma unroll
      for (int w = 0; w < NW; ++w) t += s_red[kind][w][c];
      s_tot[kind][c] = t;
    }
    __syncthreads();
  }
  const float kq = s_kq;
  float delta[VEC], o[VEC];
#pragma unroll
  for (int e = 0; e < VEC; ++e) {
    float kv = 0.f, qs = 0.f;
    if constexpr (RED2) {
      kv = s_tot[0][c0 + e];
      qs = s_tot[1][c0 + e];
    } else {
#pragma unroll
      for (int w = 0; w < NW; ++w) {
        kv += s_red[0][w][c0 + e];
        qs += s_red[1][w][c0 + e];
      }
    }
    delta[e] = beta * (vv[e] - alpha * kv);
    o[e] = p.scale * fmaf(alpha, qs, kq * delta[e]);
  }
  if (wave == 0 && lane < LPR)  // the row's outputs, one access per 16 bytes when out is 16-byte aligned
    store_vec<VEC>(p.out, row_bh * D + c0, o, p.out_dt, (reinterpret_cast<uintptr_t>(p.out) & 15) == 0);

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

// Persistent decode for fp32 128 x 128 states.  One workgroup of 16 waves
// per compute unit walks the tiles t = blockIdx.x + i G; the loads of the next
// tile (its state rows, the key and query elements of this lane's rows, the
// values of its columns and the gate inputs) are in flight while the current
// tile is reduced, updated and written back, and slot indices are fetched two
// tiles ahead so no load waits on another.  Lane l of wave w holds VEC = 4
// (fp32) or 8 (16-bit) columns from VEC (l mod LPR) of rows RPW w + l / LPR
// + 16 RPW pp (LPR = 128 / VEC lanes per row, RPW = 64 / LPR rows per wave).  Column sums of
// S^T k and S^T q go through LDS in two levels (double-buffered by tile
// parity, two barriers per tile).  Copies with this shape (64 KiB per
// 16-wave workgroup, next loads issued before the current stores) run at
// 5.95 TB/s on MI355X against 5.26 for one-shot 4-wave workgroups; the
// decode went from 5.25 to 5.70-5.76 TB/s at B = 256 and from 5.40 to 5.93
// at B = 512.
constexpr int kPersistNW = 16;
constexpr int kPersistMaxIter = 512;  // tiles per workgroup whose slot and head scalars sit in LDS

// NTL / NTS: non-temporal tile loads / stores.
// Waves per workgroup: 16 for fp32 tiles (one workgroup per CU), 8 for 16-bit
// ones (two per CU, four 16-byte loads per lane either way).
template <int SDT>
constexpr int persist_waves() { return SDT == GDN_F32 ? kPersistNW : kPersistNW / 2; }

template <int SDT, bool NTL, bool NTS, int IDT>
__global__ void __launch_bounds__(persist_waves<SDT>() * 64, 4) gdn_decode_persist_kernel(const DecodeArgs p) {
  // 16-byte accesses: 4 fp32 or 8 16-bit columns per lane
  constexpr int D = 128, NW = persist_waves<SDT>(), VEC = SDT == GDN_F32 ? 4 : 8, LPR = D / VEC, RPW = 64 / LPR;
  constexpr int PASSES = D / (RPW * NW);
  static_assert(PASSES * RPW * NW == D, "whole rows per pass");
  using IO = TileIO<SDT, VEC, NTS>;
  typedef typename IO::Raw Raw;
  static_assert(sizeof(Raw) == 16, "16-byte tile accesses");
  using ST = typename StateElem<SDT>::T;
  typedef typename std::conditional<IDT == GDN_F32, uint32_t, uint16_t>::type IT;  // input element bits

  __shared__ __attribute__((aligned(16))) float s_red[2][2][NW][D];  // [parity][S^T k | S^T q][wave][column]
  __shared__ __attribute__((aligned(16))) float s_sum[2][2][D];      // [parity][S^T k | S^T q][column]
  __shared__ __attribute__((aligned(16))) float s_kqw[2][NW];        // [parity][wave] partial k . q
  __shared__ int s_slot[kPersistMaxIter];                            // per tile of this workgroup:
  __shared__ float s_al[kPersistMaxIter], s_db[kPersistMaxIter];     // slot, A_log and dt_bias of its head

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int c0 = (lane % LPR) * VEC, r0 = wave * RPW + lane / LPR;
  const int units = p.B * p.Hv, G = gridDim.x;
  int t = blockIdx.x;
  if (t >= units) return;
  // The scalars of every tile this workgroup visits go to LDS first (one wait
  // here), so no load inside the loop waits behind the tile traffic.
  const int n_iter = (units - t + G - 1) / G;  // <= kPersistMaxIter (launcher)
  for (int i = tid; i < n_iter; i += NW * 64) {
    const int u = t + i * G, hh = u % p.Hv;
    s_slot[i] = p.slot_map[u / p.Hv];
    s_al[i] = p.A_log[hh];
    s_db[i] = p.dt_bias[hh];
  }
  __syncthreads();

  // Loads of a tile in flight behind the current one keep their raw bits and
  // are widened only when the tile becomes current, so nothing waits on them
  // early; the per-element input index is made opaque so that the uniform ones
  // (gates) go through vector loads, which complete in order with the tile.
  int zl = 0;
  asm volatile("" : "+v"(zl));
  const IT* kin = static_cast<const IT*>(p.k);
  const IT* qin = static_cast<const IT*>(p.q);
  const IT* vin = static_cast<const IT*>(p.v);
  const IT* ain = static_cast<const IT*>(p.a);
  const IT* bin = static_cast<const IT*>(p.b);
  auto widen = [](uint32_t x) -> float {
    if constexpr (IDT == GDN_F32) return __uint_as_float(x);
    else if constexpr (IDT == GDN_BF16) return bf16_bits_to_f32(x);
    else return f16_bits_to_f32(x);
  };
  auto valid = [&](int slot) { return slot >= 0 && (int64_t)slot < p.num_slots; };
  const bool out_vec = (reinterpret_cast<uintptr_t>(p.out) & 15) == 0;
  // the values of this lane's columns, packed as loaded (VEC inputs in one access)
  typedef unsigned int VRaw __attribute__((ext_vector_type(VEC * sizeof(IT) / 4)));
  // The RPW key (or query) elements of one pass's rows of this wave, adjacent
  // in memory, in one access: lane j < PASSES holds the keys of pass j, lane
  // PASSES + j the queries (the other lanes repeat lane 0's).  One load per
  // wave replaces 2 PASSES per-element ones; each lane takes its row's element
  // with a lane read.
  constexpr int KQWORDS = RPW * (int)sizeof(IT) / 4;
  static_assert(RPW * sizeof(IT) % 4 == 0 && KQWORDS <= 4 && 2 * PASSES <= 64, "row-group key loads");
  typedef unsigned int KQW __attribute__((ext_vector_type(KQWORDS)));
  struct In {
    Raw raw[PASSES];
    VRaw vv;
    KQW kq;
    uint32_t ga, gb;
  };
  // Every load is issued unconditionally (a branch around them would make the
  // compiler wait for all loads in flight where the paths join): a padded row's
  // tile goes through a zero-size buffer, whose reads return zeros and touch no
  // memory.
  auto fetch = [&](int u, int slot, In& x) {
    const int b = u / p.Hv, h = u - b * p.Hv, hk = h / (p.Hv / p.Hk);
    const int64_t row_bh = (int64_t)b * p.Hv + h, kq_base = ((int64_t)b * p.Hk + hk) * D;
    const bool ok = valid(slot);
    const ST* tile = static_cast<const ST*>(p.pool) + (ok ? ((int64_t)slot * p.Hv + h) * (int64_t)(D * D) : 0);
    const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<ST*>(tile), 0, ok ? D * D * (int)sizeof(ST) : 0, 0x00020000);
#pragma unroll
    for (int pp = 0; pp < PASSES; ++pp)
      x.raw[pp] = __builtin_bit_cast(Raw, __builtin_amdgcn_raw_buffer_load_b128(
                                              rs, (r0 * D + c0) * (int)sizeof(ST),
                                              pp * NW * RPW * D * (int)sizeof(ST), NTL ? 2 : 0));
    {
      const bool isq = lane >= PASSES && lane < 2 * PASSES;
      const int jp = lane < 2 * PASSES ? lane % PASSES : 0;
      x.kq = *reinterpret_cast<const KQW*>((isq ? qin : kin) + kq_base + RPW * wave + NW * RPW * jp);
    }
    x.vv = *reinterpret_cast<const VRaw*>(vin + row_bh * D + c0);
    x.ga = ain[row_bh + zl];
    x.gb = bin[row_bh + zl];
  };

  // LDS parity flips on live tiles only.  A padded tile passes no barrier, so
  // a wave may run ahead through it to the next live tile while a slower wave
  // still reads the k . q partials of the previous one: the two live tiles
  // must use different buffers, whatever the padded tiles between them.
  // element of this lane's row (lane / LPR within the group) from lane j's row group
  auto kq_at = [&](const KQW& w, int j) -> uint32_t {
    const int i = lane / LPR;
    uint32_t word[KQWORDS];
#pragma unroll
    for (int q = 0; q < KQWORDS; ++q) word[q] = __builtin_amdgcn_readlane(w[q], j);
    if constexpr (IDT == GDN_F32) {
      return word[i];
    } else {
      const uint32_t v = word[i >> 1];
      return (i & 1) ? (v >> 16) : (v & 0xffffu);
    }
  };

  In cur, nxt;
  fetch(t, s_slot[0], cur);
  for (int it = 0, par = 0; t < units; t += G, ++it) {
    const int tn = t + G;
    // past the last tile the loads repeat this tile's inputs, with no state
    fetch(tn < units ? tn : t, tn < units ? s_slot[it + 1] : -1, nxt);
    const int slot_c = s_slot[it];

    const int b = t / p.Hv, h = t - b * p.Hv;
    const int64_t row_bh = (int64_t)b * p.Hv + h;
    if (!valid(slot_c)) {  // padded row: zero output, no state access (uniform over the workgroup)
      if (tid < D) store_elem(p.out, row_bh * D + tid, 0.f, p.out_dt);
    } else {
      const float g = gate_g(widen(cur.ga), s_al[it], s_db[it]);
      const float beta = sigmoid_f(widen(cur.gb));
      const float alpha = expf(g);
      float kr[PASSES], kvp[VEC], qsp[VEC], kqp = 0.f;
#pragma unroll
      for (int e = 0; e < VEC; ++e) kvp[e] = qsp[e] = 0.f;
#pragma unroll
      for (int pp = 0; pp < PASSES; ++pp) {
        kr[pp] = widen(kq_at(cur.kq, pp));
        const float qr = widen(kq_at(cur.kq, PASSES + pp));
        float sv[VEC];
        IO::widen(cur.raw[pp], sv);
#pragma unroll
        for (int e = 0; e < VEC; ++e) {
          kvp[e] = fmaf(sv[e], kr[pp], kvp[e]);
          qsp[e] = fmaf(sv[e], qr, qsp[e]);
        }
        kqp = fmaf(kr[pp], qr, kqp);
      }
#pragma unroll
      for (int e = 0; e < VEC; ++e) {
        kvp[e] = xor_sum_from<LPR>(kvp[e]);
        qsp[e] = xor_sum_from<LPR>(qsp[e]);
      }
      // this wave's rows: lane group l / LPR holds rows RPW w + l / LPR + 16 RPW pp
      // (summed with every lane active: a cross-lane read inside the lane-0 branch
      // would see an operand the compiler computed for lane 0 only)
      kqp = xor_sum_from<LPR>(kqp);
      if (lane < LPR) {
#pragma unroll
        for (int e4 = 0; e4 < VEC; e4 += 4) {
          *reinterpret_cast<f32x4*>(&s_red[par][0][wave][c0 + e4]) = f32x4{kvp[e4], kvp[e4 + 1], kvp[e4 + 2], kvp[e4 + 3]};
          *reinterpret_cast<f32x4*>(&s_red[par][1][wave][c0 + e4]) = f32x4{qsp[e4], qsp[e4 + 1], qsp[e4 + 2], qsp[e4 + 3]};
        }
      }
      if (lane == 0) s_kqw[par][wave] = kqp;
      __syncthreads();
      if (tid < 2 * D) {  // one (kind, column) per thread
        const int kind = tid / D, col = tid - kind * D;
        float acc = 0.f;
#pragma unroll
        for (int w = 0; w < NW; ++w) acc += s_red[par][kind][w][col];
        s_sum[par][kind][col] = acc;
      }
      __syncthreads();
      float kv[VEC], qs[VEC];
#pragma unroll
      for (int e4 = 0; e4 < VEC; e4 += 4) {
        const f32x4 k4 = *reinterpret_cast<const f32x4*>(&s_sum[par][0][c0 + e4]);
        const f32x4 q4 = *reinterpret_cast<const f32x4*>(&s_sum[par][1][c0 + e4]);
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          kv[e4 + j] = k4[j];
          qs[e4 + j] = q4[j];
        }
      }
      float kq = 0.f;
#pragma unroll
      for (int w = 0; w < NW; ++w) kq += s_kqw[par][w];
      float delta[VEC], o[VEC];
#pragma unroll
      for (int e = 0; e < VEC; ++e) {
        float ve;
        if constexpr (IDT == GDN_F32) ve = __uint_as_float(cur.vv[e]);
        else ve = widen((e & 1) ? (cur.vv[e >> 1] >> 16) : (cur.vv[e >> 1] & 0xffffu));
        delta[e] = beta * (ve - alpha * kv[e]);
        o[e] = p.scale * fmaf(alpha, qs[e], kq * delta[e]);
      }
      if (wave == 0 && lane < LPR) store_vec<VEC>(p.out, row_bh * D + c0, o, p.out_dt, out_vec);
      ST* tile = static_cast<ST*>(p.pool) + ((int64_t)slot_c * p.Hv + h) * (int64_t)(D * D);
#pragma unroll
      for (int pp = 0; pp < PASSES; ++pp) {
        float sv[VEC];
        IO::widen(cur.raw[pp], sv);
#pragma unroll
        for (int e = 0; e < VEC; ++e) sv[e] = fmaf(alpha, sv[e], kr[pp] * delta[e]);
        IO::store(tile + (r0 + pp * NW * RPW) * D + c0, sv);
      }
      par ^= 1;
    }
    cur = nxt;
  }
}

template <int SDT, int D>
static hipError_t launch_decode_t(const DecodeArgs& a, hipStream_t s) {
  using G = DecodeGeom<SDT, D>;
  const unsigned grid = (unsigned)((int64_t)a.B * a.Hv);
  constexpr bool NT = (SDT == GDN_F32) ? (GDN_DECODE_NT_F32 != 0) : (GDN_DECODE_NT_16 != 0);
  const long long tile_bytes = (long long)grid * D * D * (long long)sizeof(typename StateElem<SDT>::T);
  // fp32 by default: 16-bit tiles (32 KiB) ran at 3.66-3.83 TB/s with 16-wave
  // workgroups and 4.16-4.72 with 8-wave ones (two per CU) against 4.62-5.14
  // for the one-shot two-wave kernel, which keeps eight such tiles in flight
  // per CU
  if constexpr (D == 128 && GDN_DECODE_PERSIST != 0 && (SDT == GDN_F32 || GDN_DECODE_PERSIST_16 != 0)) {
    // fp32: streamed both ways; 16-bit: the cache rules of the one-shot kernel
    const bool ntl = SDT == GDN_F32 ? NT : stream_tile_reads(tile_bytes);
    const bool nts = SDT == GDN_F32 ? NT : stream_tile_writes(tile_bytes);
    void (*kern)(const DecodeArgs) = nullptr;
    auto pick = [&](auto ntl_c, auto nts_c) {
      constexpr bool L = decltype(ntl_c)::value, S = decltype(nts_c)::value;
      kern = a.in_dt == GDN_F32    ? &gdn_decode_persist_kernel<SDT, L, S, GDN_F32>
             : a.in_dt == GDN_BF16 ? &gdn_decode_persist_kernel<SDT, L, S, GDN_BF16>
                                   : &gdn_decode_persist_kernel<SDT, L, S, GDN_F16>;
    };
    if (ntl && nts) pick(std::true_type{}, std::true_type{});
    else if (ntl) pick(std::true_type{}, std::false_type{});
    else pick(std::false_type{}, std::false_type{});
    int per_cu = 0, cus = 0;
    constexpr int nth = persist_waves<SDT>() * 64;
    hipError_t e = resident_blocks(reinterpret_cast<const void*>(kern), nth, 0, &per_cu);
    if (e == hipSuccess) e = device_cus(&cus);
    if (e != hipSuccess) return e;
    const int64_t fill = (int64_t)(per_cu > 0 ? per_cu : 1) * cus;
    const unsigned pgrid = (unsigned)((int64_t)grid < fill ? (int64_t)grid : fill);
    // with 8 or fewer tiles per workgroup the pipeline has too little to overlap
    // (fp32 at B = 64: 5.06-5.25 TB/s against 5.28-5.30 for the one-shot kernel)
    if ((int64_t)grid > 8 * (int64_t)pgrid && (int64_t)grid <= (int64_t)pgrid * kPersistMaxIter) {
      hipLaunchKernelGGL(kern, dim3(pgrid), dim3(nth), 0, s, a);
      return hipGetLastError();
    }
  }
  auto one_shot = [&](auto nt_c, auto ntl_c) {
    constexpr bool N = decltype(nt_c)::value, L = decltype(ntl_c)::value;
    // 16-bit tiles streamed from HBM: more waves per workgroup
    constexpr int W = (SDT != GDN_F32 && L) ? (N ? GDN_DECODE_WAVES_16_STREAM2 : GDN_DECODE_WAVES_16_STREAM) : G::NW;
    void (*k)(const DecodeArgs) = a.in_dt == GDN_F32    ? &gdn_decode_kernel<SDT, D, N, L, GDN_F32, W>
                                  : a.in_dt == GDN_BF16 ? &gdn_decode_kernel<SDT, D, N, L, GDN_BF16, W>
                                                        : &gdn_decode_kernel<SDT, D, N, L, GDN_F16, W>;
    hipLaunchKernelGGL(k, dim3(grid), dim3(W * 64), 0, s, a);
  };
  if (!NT && stream_tile_writes(tile_bytes)) one_shot(std::true_type{}, std::true_type{});
  else if (stream_tile_reads(tile_bytes)) one_shot(std::integral_constant<bool, NT>{}, std::true_type{});
  else one_shot(std::integral_constant<bool, NT>{}, std::false_type{});
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
