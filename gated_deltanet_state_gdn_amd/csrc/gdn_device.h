// Device-side helpers shared by the GDN kernels (gfx950, wave64).
//
// Storage types: the state and the inputs are f32, bf16 or f16 in memory and
// always FP32 in registers (vLLM PR #52191 page, implementation item 4: FP32
// math, narrow storage, one rounding per write-back).  Narrowing uses the
// gfx950 packed converts (v_cvt_pk_bf16_f32 / v_cvt_pk_f16_f32), which round
// to nearest-even under the default mode.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

#include "gdn.h"

namespace gdn {

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));

// ------------------------------------------------------------------ scalars
__device__ __forceinline__ float bf16_bits_to_f32(uint32_t h) { return __uint_as_float(h << 16); }
__device__ __forceinline__ float f16_bits_to_f32(uint32_t h) {
  return (float)__builtin_bit_cast(_Float16, (uint16_t)h);
}

// Two floats -> one packed word of two 16-bit values (element 0 in the low half).
template <int DT>
__device__ __forceinline__ uint32_t pack2(float x0, float x1);
template <>
__device__ __forceinline__ uint32_t pack2<GDN_BF16>(float x0, float x1) {
  typedef __bf16 bf2 __attribute__((ext_vector_type(2)));
  bf2 r = {(__bf16)x0, (__bf16)x1};
  return __builtin_bit_cast(uint32_t, r);
}
template <>
__device__ __forceinline__ uint32_t pack2<GDN_F16>(float x0, float x1) {
  typedef _Float16 h2 __attribute__((ext_vector_type(2)));
  h2 r = {(_Float16)x0, (_Float16)x1};
  return __builtin_bit_cast(uint32_t, r);
}

template <int DT>
__device__ __forceinline__ float unpack_lo(uint32_t w) {
  return DT == GDN_BF16 ? bf16_bits_to_f32(w & 0xffffu) : f16_bits_to_f32(w & 0xffffu);
}
template <int DT>
__device__ __forceinline__ float unpack_hi(uint32_t w) {
  return DT == GDN_BF16 ? __uint_as_float(w & 0xffff0000u) : f16_bits_to_f32(w >> 16);
}

// Element i of a tensor whose dtype is only known at run time (inputs, outputs,
// small per-token vectors: never the state stream).
__device__ __forceinline__ float load_elem(const void* p, int64_t i, int dt) {
  if (dt == GDN_F32) return static_cast<const float*>(p)[i];
  const uint32_t h = static_cast<const uint16_t*>(p)[i];
  return dt == GDN_BF16 ? bf16_bits_to_f32(h) : f16_bits_to_f32(h);
}

__device__ __forceinline__ void store_elem(void* p, int64_t i, float x, int dt) {
  if (dt == GDN_F32) {
    static_cast<float*>(p)[i] = x;
  } else if (dt == GDN_BF16) {
    static_cast<__bf16*>(p)[i] = (__bf16)x;
  } else {
    static_cast<_Float16*>(p)[i] = (_Float16)x;
  }
}

// N = 4 or 8 consecutive elements from element i of a run-time-dtype tensor,
// in one vector access per 16 bytes: the caller guarantees N x element bytes
// alignment of element i (a 16-byte-aligned array and i a multiple of N).  A
// per-element loop issues N memory instructions, each an address pass of the
// texture addresser, which bounds the 16-bit decode tiles' kernels.
template <int N>
__device__ __forceinline__ void load_vec(const void* p, int64_t i, int dt, float (&f)[N]) {
  static_assert(N == 4 || N == 8, "4 or 8 elements");
  if (dt == GDN_F32) {
    const float* q = static_cast<const float*>(p) + i;
#pragma unroll
    for (int e = 0; e < N; e += 4) {
      const f32x4 w = *reinterpret_cast<const f32x4*>(q + e);
#pragma unroll
      for (int j = 0; j < 4; ++j) f[e + j] = w[j];
    }
    return;
  }
  const uint16_t* q = static_cast<const uint16_t*>(p) + i;
  uint32_t w[N / 2];
  if constexpr (N == 8) {
    const u32x4 v = *reinterpret_cast<const u32x4*>(q);
#pragma unroll
    for (int j = 0; j < 4; ++j) w[j] = v[j];
  } else {
    const u32x2 v = *reinterpret_cast<const u32x2*>(q);
    w[0] = v[0];
    w[1] = v[1];
  }
#pragma unroll
  for (int j = 0; j < N / 2; ++j) {
    f[2 * j] = dt == GDN_BF16 ? unpack_lo<GDN_BF16>(w[j]) : unpack_lo<GDN_F16>(w[j]);
    f[2 * j + 1] = dt == GDN_BF16 ? unpack_hi<GDN_BF16>(w[j]) : unpack_hi<GDN_F16>(w[j]);
  }
}

// N = 4 or 8 consecutive input elements of compile-time dtype IDT kept as raw
// bits: the load is issued early and widened later, with no wait between the
// load and the loads issued after it (a run-time dtype switch widens inside
// its branches, where the compiler waits for every load issued so far).
template <int IDT, int N>
struct InVec {
  static_assert(N == 4 || N == 8, "4 or 8 elements");
  static constexpr int W = IDT == GDN_F32 ? N : N / 2;
  uint32_t w[W];
  __device__ __forceinline__ void load(const void* p, int64_t i) {
    if constexpr (IDT == GDN_F32) {
      const u32x4* q = reinterpret_cast<const u32x4*>(static_cast<const float*>(p) + i);
#pragma unroll
      for (int c = 0; c < N / 4; ++c) {
        const u32x4 v = q[c];
#pragma unroll
        for (int j = 0; j < 4; ++j) w[4 * c + j] = v[j];
      }
    } else if constexpr (N == 8) {
      const u32x4 v = *reinterpret_cast<const u32x4*>(static_cast<const uint16_t*>(p) + i);
#pragma unroll
      for (int j = 0; j < 4; ++j) w[j] = v[j];
    } else {
      const u32x2 v = *reinterpret_cast<const u32x2*>(static_cast<const uint16_t*>(p) + i);
      w[0] = v[0];
      w[1] = v[1];
    }
  }
  // the raw bits back to memory (a bit-exact copy of the input)
  __device__ __forceinline__ void store(void* p, int64_t i) const {
    if constexpr (IDT == GDN_F32) {
      u32x4* q = reinterpret_cast<u32x4*>(static_cast<float*>(p) + i);
#pragma unroll
      for (int c = 0; c < N / 4; ++c) q[c] = u32x4{w[4 * c], w[4 * c + 1], w[4 * c + 2], w[4 * c + 3]};
    } else if constexpr (N == 8) {
      *reinterpret_cast<u32x4*>(static_cast<uint16_t*>(p) + i) = u32x4{w[0], w[1], w[2], w[3]};
    } else {
      *reinterpret_cast<u32x2*>(static_cast<uint16_t*>(p) + i) = u32x2{w[0], w[1]};
    }
  }
  __device__ __forceinline__ void widen(float (&f)[N]) const {
    if constexpr (IDT == GDN_F32) {
#pragma unroll
      for (int e = 0; e < N; ++e) f[e] = __uint_as_float(w[e]);
    } else {
#pragma unroll
      for (int j = 0; j < N / 2; ++j) {
        f[2 * j] = unpack_lo<IDT>(w[j]);
        f[2 * j + 1] = unpack_hi<IDT>(w[j]);
      }
    }
  }
};

// One input element of compile-time dtype IDT as raw bits, and its value.
template <int IDT>
__device__ __forceinline__ uint32_t in_bits(const void* p, int64_t i) {
  if constexpr (IDT == GDN_F32) return static_cast<const uint32_t*>(p)[i];
  else return static_cast<const uint16_t*>(p)[i];
}
template <int IDT>
__device__ __forceinline__ float in_value(uint32_t bits) {
  if constexpr (IDT == GDN_F32) return __uint_as_float(bits);
  else return unpack_lo<IDT>(bits);
}

// N = 4 or 8 consecutive elements stored at element i of a run-time-dtype
// tensor, rounded once: one vector access per 16 bytes when that is aligned
// (`vec`, uniform), else one access per element.
template <int N>
__device__ __forceinline__ void store_vec(void* p, int64_t i, const float (&f)[N], int dt, bool vec) {
  static_assert(N == 4 || N == 8, "4 or 8 elements");
  if (!vec) {
#pragma unroll
    for (int e = 0; e < N; ++e) store_elem(p, i + e, f[e], dt);
    return;
  }
  if (dt == GDN_F32) {
    float* q = static_cast<float*>(p) + i;
#pragma unroll
    for (int e = 0; e < N; e += 4) *reinterpret_cast<f32x4*>(q + e) = f32x4{f[e], f[e + 1], f[e + 2], f[e + 3]};
    return;
  }
  uint32_t w[N / 2];
#pragma unroll
  for (int j = 0; j < N / 2; ++j)
    w[j] = dt == GDN_BF16 ? pack2<GDN_BF16>(f[2 * j], f[2 * j + 1]) : pack2<GDN_F16>(f[2 * j], f[2 * j + 1]);
  uint16_t* q = static_cast<uint16_t*>(p) + i;
  if constexpr (N == 8) *reinterpret_cast<u32x4*>(q) = u32x4{w[0], w[1], w[2], w[3]};
  else *reinterpret_cast<u32x2*>(q) = u32x2{w[0], w[1]};
}

// Raw copy of one element (ring append keeps the input bytes bit-exact).
__device__ __forceinline__ void copy_elem(void* dst, int64_t di, const void* src, int64_t si, int dt) {
  if (dt == GDN_F32) {
    static_cast<uint32_t*>(dst)[di] = static_cast<const uint32_t*>(src)[si];
  } else {
    static_cast<uint16_t*>(dst)[di] = static_cast<const uint16_t*>(src)[si];
  }
}

// ------------------------------------------------------------------ gates
// g = -exp(A_log) * softplus(a + dt_bias), beta = sigmoid(b); softplus is the
// exact max(x,0) + log1p(exp(-|x|)) (no threshold linearisation).
//
// log1p(t) for t in [0, 1] by Goldberg's identity (D. Goldberg, "What every
// computer scientist should know about floating-point arithmetic", 1991, Theorem
// 4): with u = 1 + t rounded, log1p(t) = log(u) t / (u - 1) to a few ulps, since
// the ratio t / (u - 1) undoes the rounding of u (u - 1 is exact).  u == 1 means
// t is below half an ulp of 1, where log1p(t) rounds to t.  This replaces the
// library log1p, whose double-float evaluation cost about 100 instructions per
// lane in the kernels that form gates per lane.
__device__ __forceinline__ float log1p_unit(float t) {
  const float u = 1.f + t;
  return u == 1.f ? t : logf(u) * (t * __builtin_amdgcn_rcpf(u - 1.f));
}
__device__ __forceinline__ float softplus_f(float x) { return fmaxf(x, 0.f) + log1p_unit(expf(-fabsf(x))); }
// the hardware reciprocal (1 ulp) in place of a correctly rounded division
__device__ __forceinline__ float sigmoid_f(float x) { return __builtin_amdgcn_rcpf(1.f + expf(-x)); }
__device__ __forceinline__ float gate_g(float a, float A_log, float dt_bias) {
  return -expf(A_log) * softplus_f(a + dt_bias);
}

// ------------------------------------------------------------------ state tiles
// Storage element type per state dtype.
template <int DT> struct StateElem { typedef uint16_t T; static constexpr int BYTES = 2; };
template <> struct StateElem<GDN_F32> { typedef float T; static constexpr int BYTES = 4; };

// VEC consecutive state elements <-> VEC floats, one 8- or 16-byte access.
// NT selects non-temporal (streaming) loads and stores.
template <int DT, int VEC, bool NT>
struct TileIO {
  static_assert(VEC * StateElem<DT>::BYTES == 16 || VEC * StateElem<DT>::BYTES == 8, "8/16-byte vectors");
  static constexpr int WORDS = VEC * StateElem<DT>::BYTES / 4;
  typedef unsigned int Raw __attribute__((ext_vector_type(WORDS)));

  // Raw (still packed) access: a 16-bit tile stays packed in registers and is
  // widened on use, halving the registers that hold it.
  __device__ __forceinline__ static Raw load_raw(const void* p) {
    return NT ? __builtin_nontemporal_load(static_cast<const Raw*>(p)) : *static_cast<const Raw*>(p);
  }
  __device__ __forceinline__ static void widen(const Raw& w, float (&f)[VEC]) { unpack<WORDS>(w, f); }
  __device__ __forceinline__ static Raw pack_raw(const float (&f)[VEC]) {
    Raw w;
    pack<WORDS>(f, w);
    return w;
  }

  __device__ __forceinline__ static void load(const void* p, float (&f)[VEC]) {
    if constexpr (WORDS == 4) {
      u32x4 w = NT ? __builtin_nontemporal_load(static_cast<const u32x4*>(p)) : *static_cast<const u32x4*>(p);
      unpack<4>(w, f);
    } else {
      u32x2 w = NT ? __builtin_nontemporal_load(static_cast<const u32x2*>(p)) : *static_cast<const u32x2*>(p);
      unpack<2>(w, f);
    }
  }
  __device__ __forceinline__ static void store(void* p, const float (&f)[VEC]) {
    if constexpr (WORDS == 4) {
      u32x4 w;
      pack<4>(f, w);
      if (NT) __builtin_nontemporal_store(w, static_cast<u32x4*>(p));
      else *static_cast<u32x4*>(p) = w;
    } else {
      u32x2 w;
      pack<2>(f, w);
      if (NT) __builtin_nontemporal_store(w, static_cast<u32x2*>(p));
      else *static_cast<u32x2*>(p) = w;
    }
  }

 private:
  template <int N, typename W>
  __device__ __forceinline__ static void unpack(const W& w, float (&f)[VEC]) {
#pragma unroll
    for (int i = 0; i < N; ++i) {
      if constexpr (DT == GDN_F32) {
        f[i] = __uint_as_float(w[i]);
      } else {
        f[2 * i] = unpack_lo<DT>(w[i]);
        f[2 * i + 1] = unpack_hi<DT>(w[i]);
      }
    }
  }
  template <int N, typename W>
  __device__ __forceinline__ static void pack(const float (&f)[VEC], W& w) {
#pragma unroll
    for (int i = 0; i < N; ++i) {
      if constexpr (DT == GDN_F32) {
        w[i] = __float_as_uint(f[i]);
      } else {
        w[i] = pack2<DT>(f[2 * i], f[2 * i + 1]);
      }
    }
  }
};

// ------------------------------------------------------------------ batched row staging
// Stages MAXR rows of ROWLEN elements (element size EB bytes: 4 for f32, 2 for
// bf16/f16) from global memory into LDS as floats.  issue() starts every
// 16-byte load of the block at once (one memory round trip for the whole
// block; rows >= nrows read as zero); commit() waits for them, widens and
// stores to LDS.  Keeping the two apart lets a caller overlap the loads of
// the next block with work on the current one.  Row r starts at element
// row_off(r) of the source, which must be 16-byte aligned.
template <int ROWLEN, int MAXR, int NTH, int EB>
struct RowStager {
  static constexpr int VE = 16 / EB;               // elements per 16-byte load
  static_assert(ROWLEN % VE == 0, "rows are whole 16-byte vectors");
  static constexpr int CPR = ROWLEN / VE;          // loads per row
  static constexpr int TOTAL = MAXR * CPR;
  static constexpr int IT = (TOTAL + NTH - 1) / NTH;
  u32x4 v[IT];

  template <class RowOff>
  __device__ __forceinline__ void issue(const void* src, int nrows, const RowOff& row_off) {
    const int tid = threadIdx.x;
#pragma unroll
    for (int it = 0; it < IT; ++it) {
      const int idx = tid + it * NTH;
      const int r = idx / CPR, c = (idx - r * CPR) * VE;
      u32x4 x = {0u, 0u, 0u, 0u};
      if (idx < TOTAL && r < nrows)
        x = *reinterpret_cast<const u32x4*>(static_cast<const char*>(src) + ((int64_t)row_off(r) + c) * EB);
      v[it] = x;
    }
  }

  // dt selects bf16 or f16 widening when EB == 2; rows >= nrows are not written.
  __device__ __forceinline__ void commit(float* dst, int ldd, int dt, int nrows = MAXR) const {
    const int tid = threadIdx.x;
#pragma unroll
    for (int it = 0; it < IT; ++it) {
      const int idx = tid + it * NTH;
      const int r = idx / CPR, c = (idx - r * CPR) * VE;
      if (idx >= TOTAL || r >= nrows) continue;
      float* d = dst + r * ldd + c;
      if constexpr (EB == 4) {
#pragma unroll
        for (int e = 0; e < 4; ++e) d[e] = __uint_as_float(v[it][e]);
      } else if (dt == GDN_BF16) {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          d[2 * e] = unpack_lo<GDN_BF16>(v[it][e]);
          d[2 * e + 1] = unpack_hi<GDN_BF16>(v[it][e]);
        }
      } else {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          d[2 * e] = unpack_lo<GDN_F16>(v[it][e]);
          d[2 * e + 1] = unpack_hi<GDN_F16>(v[it][e]);
        }
      }
    }
  }
};

// ------------------------------------------------------------------ cache policy
// 16-bit state tiles are read non-temporally only when the tiles one launch
// reads exceed what the 256 MiB Infinity Cache keeps from one step to the next
// (+5% for bf16 decode at 268 MB, +11% for a bf16 replay step at 537 MB); a
// smaller set stays cache-resident across steps and is read normally (bf16
// decode at 67 MB lost 15% to non-temporal reads).
constexpr long long kCacheResidentBytes = 192ll << 20;
inline bool stream_tile_reads(long long bytes) { return bytes > kCacheResidentBytes; }
// 16-bit tiles are also written non-temporally once one launch writes more
// than twice that (bf16 and f16 decode at 537 MB: +3%; a 5-token window of
// 16-bit destination states, 1.3 GB: +5 to +8%); at 268 MB such stores cost
// 1 to 5%.  fp32 tiles are always streamed.
inline bool stream_tile_writes(long long bytes) { return bytes > 2 * kCacheResidentBytes; }

// ------------------------------------------------------------------ XCD-aware order
// MI355X hands workgroup i of a launch to XCD i mod 8.  A one-shot launch whose
// workgroups first fetch a small index (a slot) before their tile maps workgroup
// i to unit u so that each XCD takes one contiguous run of units, about G / 8
// long: the units of one sequence (its heads) then run on one XCD, whose L2 and
// scalar caches hold that sequence's index line as its heads go by.  A
// bijection of [0, G) for every G.
__device__ __forceinline__ int xcd_unit(int i, int G) {
  const int x = i & 7, k = i >> 3, q = G >> 3, r = G & 7;
  return x * q + (x < r ? x : r) + k;
}

// ------------------------------------------------------------------ wave64 reductions
template <int CTRL>
__device__ __forceinline__ float dpp_mov(float x) {
  return __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, x), CTRL, 0xf, 0xf, false));
}

// Sum over the lanes that differ only in bits >= log2(OFF_FROM), returned to
// every lane, all on the VALU: bits 0-1 by DPP quad permutes, bits 2-3 by DPP
// rotates within 16-lane rows (by 8, then by 4 over the pair sums), bits 4 and
// 5 by the gfx950 16- and 32-lane swaps (v_permlane16/32_swap with both
// operands x: the two results hold the two halves, so their sum is the
// all-reduce).  No LDS-crossbar permutes.
template <int OFF_FROM>
__device__ __forceinline__ float xor_sum_from(float x) {
  static_assert(OFF_FROM >= 1 && OFF_FROM <= 32 && (OFF_FROM & (OFF_FROM - 1)) == 0, "power of two lane offset");
  if constexpr (OFF_FROM <= 1) x += dpp_mov<0xB1>(x);   // quad_perm [1, 0, 3, 2]: lane ^ 1
  if constexpr (OFF_FROM <= 2) x += dpp_mov<0x4E>(x);   // quad_perm [2, 3, 0, 1]: lane ^ 2
  if constexpr (OFF_FROM <= 8) x += dpp_mov<0x128>(x);  // row_ror:8: lane ^ 8 within a row
  if constexpr (OFF_FROM <= 4) x += dpp_mov<0x124>(x);  // row_ror:4 over the pair sums: bits 2-3 complete
  // Both swap results pass through an empty asm: when they are added directly
  // this compiler takes the first result for both operands of the add.
  if constexpr (OFF_FROM <= 16) {
    const unsigned a = __builtin_bit_cast(unsigned, x);
    const auto r = __builtin_amdgcn_permlane16_swap(a, a, false, false);
    unsigned r0 = r[0], r1 = r[1];
    asm volatile("" : "+v"(r0), "+v"(r1));
    x = __builtin_bit_cast(float, r0) + __builtin_bit_cast(float, r1);
  }
  const unsigned a = __builtin_bit_cast(unsigned, x);
  const auto r = __builtin_amdgcn_permlane32_swap(a, a, false, false);
  unsigned r0 = r[0], r1 = r[1];
  asm volatile("" : "+v"(r0), "+v"(r1));
  return __builtin_bit_cast(float, r0) + __builtin_bit_cast(float, r1);
}

__device__ __forceinline__ float wave_sum(float x) { return xor_sum_from<1>(x); }

// Sum over the 64 lanes of a wave on the DPP path (row shifts within 16-lane
// rows, then row broadcasts), result returned uniformly from lane 63.  A
// handful of dependent VALU ops instead of six LDS-crossbar permutes.
__device__ __forceinline__ float wave_sum_dpp(float x) {
  auto dpp = [](float v, auto ctrl, auto rmask) {
    return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), decltype(ctrl)::value,
                                                                 decltype(rmask)::value, 0xf, true));
  };
  using c_shr1 = std::integral_constant<int, 0x111>;
  using c_shr2 = std::integral_constant<int, 0x112>;
  using c_shr4 = std::integral_constant<int, 0x114>;
  using c_shr8 = std::integral_constant<int, 0x118>;
  using c_bc15 = std::integral_constant<int, 0x142>;
  using c_bc31 = std::integral_constant<int, 0x143>;
  using all_rows = std::integral_constant<int, 0xf>;
  using rows_13 = std::integral_constant<int, 0xa>;
  using rows_23 = std::integral_constant<int, 0xc>;
  x += dpp(x, c_shr1{}, all_rows{});
  x += dpp(x, c_shr2{}, all_rows{});
  x += dpp(x, c_shr4{}, all_rows{});
  x += dpp(x, c_shr8{}, all_rows{});   // lane 16r + 15 holds the sum of row r
  x += dpp(x, c_bc15{}, rows_13{});    // lane 31 / 63: rows 0+1 / 2+3
  x += dpp(x, c_bc31{}, rows_23{});    // lane 63: all four rows
  return __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, x), 63));
}

// ------------------------------------------------------------------ tile geometry
// A workgroup of NW waves streams one dk x dv tile (dk == dv == D).  Each lane
// owns VEC consecutive columns of a row; LPR lanes cover a row, a wave covers
// RPW rows per pass and the workgroup NW * RPW rows per pass.  Lanes with equal
// (lane % LPR) own the same columns, so column sums over the rows need a
// butterfly over lane bits >= log2(LPR) and then a sum over the NW waves.
template <int DT, int D, int MAXW = 4>
struct TileGeom {
  static constexpr int BYTES = StateElem<DT>::BYTES;
  // widest vector (16 B) that still leaves at least one row per wave
  static constexpr int VEC0 = 16 / BYTES;
  static constexpr int VEC = (64 / (D / VEC0) > D) ? VEC0 / 2 : VEC0;
  static constexpr int LPR = D / VEC;
  static constexpr int RPW = 64 / LPR;
  static constexpr int NW = (D / RPW) >= MAXW ? MAXW : (D / RPW);
  static constexpr int PASSES = D / (RPW * NW);
  static_assert(LPR * VEC == D && LPR * RPW == 64 && PASSES * RPW * NW == D, "tile geometry");
};

// ------------------------------------------------------------------ packed rows on MFMA
// Rows of keys / queries kept packed in LDS in their input dtype (row stride
// ldw words) and widened on use.
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

}  // namespace gdn
