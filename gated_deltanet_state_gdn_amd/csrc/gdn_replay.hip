// ReplaySSM-style GDN decode: a checkpoint S0 per (slot, value head) plus a
// ring of the last <= L state-building inputs (k, v, g, beta) replaces the
// per-step full-state write (AREX ReplaySSM article, "cache inputs, not state"
// section).  Every kernel works on independent (sequence, value head) units:
// a unit owns its checkpoint tile, its ring entries and its ring pointers.
//
// A step of T tokens runs three kernels:
//   fold   - if count + T > L, fold the committed entries into S0 (on the tile
//            held in VGPRs), write S0 back rounded once and empty the ring; a
//            persistent grid lists the folding sequences from the ring counts
//            and spreads their units evenly, so a step without folds costs one
//            pass over the counts;
//   prep   - stage the live entries and the window, compute per window
//            position t the vectors w_t and acc_t below, append the window
//            to the ring;
//   stream - o_t = scale (S0^T w_t + acc_t): one read pass over S0 for all T
//            positions, a plain batched matrix-vector product that runs at
//            high occupancy.
// With 16-bit inputs, rings of at most 16 entries and D = 64 (or 128 with fp32
// checkpoints) the order is prep, fold, stream instead (fused fold): the prep
// takes each unit's fold decision itself and forms w and acc against the
// folded ring, the fold also writes the outputs of the units it folds from
// the new S0 it holds in registers, and the stream skips those units' tiles,
// so a fold step reads each folded tile once instead of twice.
//
// prep unrolls S_i = a_i (I - b_i k_i k_i^T) S_{i-1} + b_i k_i v_i^T
// (a_i = exp(g_i)).  Transposing gives S_n^T q = S0^T w + acc with
//     w   = e^{G_n} q - sum_j e^{G_j} c_j k_j,    acc = sum_j c_j v_j,
//     c_i = b_i (e^{G_n - G_i} (k_i . q) - sum_{j > i} e^{G_j - G_i} (k_i . k_j) c_j)
// where G_j is the sum of g over the live entries up to j (every exponent is
// <= 0).  The c are one small back substitution over the Gram matrix of the
// live keys and their products with q, so a window position costs
// O(n (dk + dv)) plus O(n^2) scalars and S_n itself is never materialised.
#include <map>
#include <mutex>

#include "gdn_device.h"
#include "gdn_launch.h"

// streaming (non-temporal) checkpoint loads and stores for fp32 checkpoints
// (the stream kernel reads 16-bit checkpoints non-temporally when they exceed
// the Infinity Cache, stream_tile_reads: bf16 T = 1 steps 0.178 -> 0.159 ms)
#ifndef GDN_REPLAY_NT_F32
#define GDN_REPLAY_NT_F32 1
#endif
// fp32 128 x 128 one-token windows go through the persistent stream kernel
#ifndef GDN_REPLAY_STREAM_PERSIST
#define GDN_REPLAY_STREAM_PERSIST 1
#endif
// waves per workgroup of the stream kernel, every checkpoint dtype (for 16-bit
// tiles two waves ran T = 5 windows 10% slower on MI355X, eight no faster)
#ifndef GDN_REPLAY_WAVES
#define GDN_REPLAY_WAVES 4
#endif
// XCD-aware unit order (xcd_unit) of the one-shot stream over 16-bit
// checkpoints read past the Infinity Cache, and of the one-wave prep (whose
// two value heads of a key head then fetch its ring keys through one L2): bf16
// T = 1 steps at B = 512 0.150 -> 0.144 ms, the prep's share 0.146 -> 0.144
#ifndef GDN_REPLAY_XCD
#define GDN_REPLAY_XCD 1
#endif
#ifndef GDN_REPLAY_PREP_XCD
#define GDN_REPLAY_PREP_XCD 1
#endif
// waves per workgroup of the two-wave prep kernel (one unit per workgroup;
// 1 leaves its phases serial, 4 halves the units in flight)
#ifndef GDN_REPLAY_PREP_WAVES
#define GDN_REPLAY_PREP_WAVES 2
#endif

namespace gdn {

template <int SDT, int D>
using ReplayGeom = TileGeom<SDT, D, GDN_REPLAY_WAVES>;

constexpr int kStageRows = 16;  // entry rows staged per batch of loads
constexpr int kStreamTB = 4;    // window positions reduced per pass over the tile

// Dynamic LDS of the fold kernel (floats): committed entries k, v [L][D+1], exp(g) and beta [L].
__host__ __device__ inline size_t replay_fold_lds_bytes(int D, int L) {
  return (size_t)L * (2 * ((size_t)D + 1) + 2) * sizeof(float);
}

// Workspace: w and acc per (unit, window position) as floats, then one
// 16-byte record per unit (see ReplayArgs::rec).
size_t replay_vectors_bytes(int64_t B, int Hv, int T, int D) {
  return (size_t)B * (size_t)Hv * (size_t)T * 2 * (size_t)D * sizeof(float);
}
size_t replay_workspace_bytes(int64_t B, int Hv, int T, int D) {
  return replay_vectors_bytes(B, Hv, T, D) + (size_t)B * (size_t)Hv * 4 * sizeof(int32_t);
}

// The no-allocation variant's workspace.  In host code `scratch` names a
// host-side stand-in, not device memory: only the address hipGetSymbolAddress
// returns for the current device may reach a kernel.  Every call on one GPU
// shares its copy; nothing in it is read before the same call writes it.
static __device__ __align__(256) unsigned char scratch[kReplayScratchBytes];

hipError_t replay_scratch(void** ptr) {
  static std::mutex mu;
  static std::map<int, void*> addr;  // device -> address of that device's copy
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  std::lock_guard<std::mutex> lock(mu);
  auto it = addr.find(dev);
  if (it == addr.end()) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (p == nullptr) return hipErrorInvalidSymbol;
    it = addr.emplace(dev, p).first;
  }
  *ptr = it->second;
  return hipSuccess;
}

struct RingPos {
  int st, cnt;
};

// Ring pointers are kept per slot: every value head of a slot takes the same
// windows, folds and rollbacks, so one pair serves them all, and the heads
// cannot disagree about where the entries they share (the keys) sit.  They are
// clamped into range so that a corrupted pair cannot send an access outside
// the slot's entries.  Within a step no kernel writes a pair that another
// kernel of the same step reads: the fold's check records each unit's pointers
// after any fold, the prep reads only those records and the first value head's
// prep writes the slot's new pair (fused fold: the prep reads the pairs and
// records them, the fold reads the records, the stream writes the new pairs);
// a flush moves the pairs in a kernel of its own after the fold.
__device__ __forceinline__ RingPos ring_pos(const RingArgs& R, int64_t slot) {
  const int L = R.L;
  int st = R.start[slot], cnt = R.count[slot];
  st = ((st % L) + L) % L;
  cnt = cnt < 0 ? 0 : (cnt > L ? L : cnt);
  return RingPos{st, cnt};
}

// ---------------------------------------------------------------- ring keys
// Ring keys are stored once per key head: the value heads of a key head share
// its entries (their ring pointers always advance together), and the first of
// them appends the keys of a window.  First key row of the ring entries of
// value head h of `slot`:
__device__ __forceinline__ int64_t ring_key_base(const DecodeArgs& p, int64_t slot, int h, int L) {
  return (slot * p.Hk + h / (p.Hv / p.Hk)) * L;
}
__device__ __forceinline__ bool appends_keys(const DecodeArgs& p, int h) { return h % (p.Hv / p.Hk) == 0; }

// ---------------------------------------------------------------- fold plan
// Which units a fold workgroup folds.  A sequence folds when its slot is mapped
// and its ring would overflow (count + T > L), or, in a flush (T == 0), when
// its ring holds entries (every mapped slot in a dual flush).  Workgroup w
// first writes the records of units w, w + G, ... (the pointers the prep will
// see).  Then, for each window of up to kFoldPlanSeqs sequences, every
// workgroup builds the same list of the window's folding sequences from the
// ring counts (bit b of a mask word per 64 sequences, with prefix counts) and
// folds units f = w, w + G, ... of it: sequence f / Hv of the list, head
// f mod Hv.  The folds of a step are so spread evenly over the grid whichever
// sequences they belong to (staggered rings fold about 1/L of the sequences
// on every step), and no counter has to start at zero.
constexpr int kFoldPlanSeqs = 4096;
constexpr int kFoldPlanWords = kFoldPlanSeqs / 64;

struct FoldPlanLds {
  uint64_t mask[kFoldPlanWords];
  int pref[kFoldPlanWords + 1];
};

// FUSED: the prep ran first and wrote every unit's record (slot, pointers
// before the step, fold flag); the plan reads the flag of each sequence's first
// unit and writes nothing.
template <bool DUAL, class F, bool FUSED = false>
__device__ __forceinline__ void fold_units(const ReplayArgs& P, FoldPlanLds& sh, F&& fold_unit,
                                           std::integral_constant<bool, FUSED> = {}) {
  const DecodeArgs& p = P.d;
  const RingArgs& R = P.ring;
  const int T = P.T, L = R.L;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, nth = blockDim.x;
  const int units = p.B * p.Hv, G = gridDim.x;
  // whether sequence b folds, and the record of its units
  auto plan_of = [&](int b, int4& rc) -> bool {
    if constexpr (FUSED) {
      rc = reinterpret_cast<const int4*>(P.rec)[(int64_t)b * p.Hv];
      return rc.x >= 0 && rc.w != 0;
    }
    const int slot = p.slot_map[b];
    rc = int4{-1, 0, 0, 0};
    if (slot < 0 || (int64_t)slot >= p.num_slots) return false;
    const RingPos rp = ring_pos(R, slot);
    const bool need = (T > 0) ? (rp.cnt + T > L) : (rp.cnt > 0 || DUAL);
    rc = need ? int4{slot, (rp.st + rp.cnt) % L, 0, 0} : int4{slot, rp.st, rp.cnt, 0};
    return need;
  };
  if (!FUSED && P.rec != nullptr) {
    for (int64_t j = tid; blockIdx.x + j * G < units; j += nth) {
      const int x = (int)(blockIdx.x + j * G);
      int4 rc;
      plan_of(x / p.Hv, rc);
      reinterpret_cast<int4*>(P.rec)[x] = rc;
    }
  }
  // every value of the list walk is the same in all lanes: scalar registers
  auto uni = [](int v) { return __builtin_amdgcn_readfirstlane(v); };
  for (int b0 = 0; b0 < p.B; b0 += kFoldPlanSeqs) {
    const int nwords = (min(kFoldPlanSeqs, p.B - b0) + 63) / 64;
    for (int q0 = 0; q0 < nwords; q0 += nth / 64) {
      const int q = q0 + wave, b = b0 + 64 * q + lane;
      int4 rc;
      const bool need = q < nwords && b < p.B && plan_of(b, rc);
      const uint64_t m = __ballot(need);
      if (q < nwords && lane == 0) sh.mask[q] = m;
    }
    __syncthreads();
    if (tid == 0) {
      int acc = 0;
      for (int q = 0; q < nwords; ++q) {
        sh.pref[q] = acc;
        acc += __popcll(sh.mask[q]);
      }
      sh.pref[nwords] = acc;
    }
    __syncthreads();
    const int64_t total = (int64_t)uni(sh.pref[nwords]) * p.Hv;
    int q = 0;
    for (int64_t f = blockIdx.x; f < total; f += G) {
      const int i = (int)(f / p.Hv), h = (int)(f - (int64_t)i * p.Hv);
      while (uni(sh.pref[q + 1]) <= i) ++q;
      const uint64_t mw = sh.mask[q];
      uint64_t m = ((uint64_t)(uint32_t)uni((int)(mw >> 32)) << 32) | (uint32_t)uni((int)(uint32_t)mw);
      for (int k = i - uni(sh.pref[q]); k > 0; --k) m &= m - 1;  // drop the set bits before the i-th
      fold_unit((b0 + 64 * q + __builtin_ctzll(m)) * p.Hv + h);
    }
    __syncthreads();  // the masks are rewritten for the next window
  }
}

// ---------------------------------------------------------------- fold
// Persistent (G workgroups, the resident count): each workgroup folds the
// units the fold plan above gives it, one after another with the whole
// workgroup, so a step without folds costs one pass over the ring counts.
// A unit folds when count + T > L; the flush (T == 0) folds every non-empty
// ring.  CDT >= 0 selects the dual-precision checkpoint: the fp32 result is
// also written, rounded once, to the CDT read copy (the flush then refreshes
// the copy of every unit).  Two variants: by columns for D >= 32 (below the
// prep section), by rows for D = 16 (here).
template <int SDT, int D>
using FoldGeom = TileGeom<SDT, D, 4>;  // fp32 working tile: four waves for every state dtype

template <int SDT, int D, bool NT, int EB, int CDT>
__global__ void __launch_bounds__((FoldGeom<SDT, D>::NW * 64))
gdn_replay_fold_rows_kernel(const ReplayArgs P) {
  using G = FoldGeom<SDT, D>;
  constexpr int VEC = G::VEC, LPR = G::LPR, RPW = G::RPW, NW = G::NW, PASSES = G::PASSES;
  constexpr int NTH = NW * 64;
  constexpr int LDE = D + 1;
  using IO = TileIO<SDT, VEC, NT>;
  using ST = typename StateElem<SDT>::T;
  using Stager = RowStager<D, kStageRows, NTH, EB>;

  extern __shared__ float s_dyn[];
  __shared__ float s_red[2][NW][D];
  __shared__ FoldPlanLds s_plan;

  const DecodeArgs& p = P.d;
  const RingArgs& R = P.ring;
  const int L = R.L;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int c0 = (lane % LPR) * VEC;
  const int r0 = wave * RPW + lane / LPR;
  float* e_k = s_dyn;           // [L][LDE]
  float* e_v = e_k + L * LDE;   // [L][LDE]
  float* e_a = e_v + L * LDE;   // [L] exp(g)
  float* e_b = e_a + L;         // [L] beta

  fold_units<(CDT >= 0)>(P, s_plan, [&](const int x) {
    const int b = x / p.Hv, h = x - (x / p.Hv) * p.Hv;
    const int64_t unit = (int64_t)p.slot_map[b] * p.Hv + h;
    const RingPos rp = ring_pos(R, p.slot_map[b]);
    const int st = rp.st, cnt = rp.cnt;

    // the lane offset is made opaque per unit so that the per-pass addresses
    // are not hoisted out of the unit loop (they would hold registers)
    int lane_off = r0 * D + c0;
    asm volatile("" : "+v"(lane_off));
    ST* tile = static_cast<ST*>(p.pool) + unit * (int64_t)(D * D) + lane_off;
    float s[PASSES][VEC];
#pragma unroll
    for (int pp = 0; pp < PASSES; ++pp) IO::widen(IO::load_raw(tile + pp * NW * RPW * D), s[pp]);

    const int64_t ring_e = unit * L;
    const int64_t kring_e = ring_key_base(p, p.slot_map[b], h, L);
    for (int t = tid; t < cnt; t += NTH) {
      const int j = (st + t) % L;
      e_a[t] = expf(R.g[ring_e + j]);
      e_b[t] = R.beta[ring_e + j];
    }
    for (int r0s = 0; r0s < cnt; r0s += kStageRows) {
      Stager sk, sv;
      auto ring_row = [&](int r) { return (ring_e + (st + r0s + r) % L) * D; };
      auto key_row = [&](int r) { return (kring_e + (st + r0s + r) % L) * D; };
      const int nr = min(kStageRows, cnt - r0s);
      sk.issue(R.k, nr, key_row);
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
    if (cnt > 0) {
#pragma unroll
      for (int pp = 0; pp < PASSES; ++pp) IO::store(tile + pp * NW * RPW * D, s[pp]);
    }
    if constexpr (CDT >= 0) {
      using CIO = TileIO<CDT, VEC, false>;
      uint16_t* copy = static_cast<uint16_t*>(P.read_pool) + unit * (int64_t)(D * D) + lane_off;
#pragma unroll
      for (int pp = 0; pp < PASSES; ++pp) CIO::store(copy + pp * NW * RPW * D, s[pp]);
    }
    __syncthreads();  // LDS staging is reused by the next unit
  });
}

// The fold for D >= 32, with the tile split by columns: wave w holds columns
// w D / 4 .. (w + 1) D / 4 - 1 of every row, four per lane, so the key
// products S^T k of its columns reduce within the wave.  The columns of S
// are independent under the recurrence, so each wave runs all cnt steps on
// its own with no barrier between them: two barriers per unit (staging,
// reuse) instead of one per entry.  Keys are staged permuted so that a lane
// reads the key rows it multiplies as one contiguous run.
constexpr int kFoldColThreads = 256;

template <int SDT, int D, bool NT, int EB, int CDT>
__global__ void __launch_bounds__(kFoldColThreads) gdn_replay_fold_kernel(const ReplayArgs P) {
  constexpr int NW = kFoldColThreads / 64, VEC = 4;
  constexpr int CW = D / NW;      // columns per wave
  constexpr int CG = CW / VEC;    // column groups per wave
  constexpr int RS = 64 / CG;     // row lanes per column group
  constexpr int PASSES = D / RS;  // rows per lane: pp * RS + rs
  static_assert(D >= 32 && CG * RS == 64 && PASSES * RS == D, "fold geometry");
  constexpr int NTH = kFoldColThreads;
  using IO = TileIO<SDT, VEC, NT>;
  using ST = typename StateElem<SDT>::T;

  extern __shared__ float s_dyn[];
  __shared__ FoldPlanLds s_plan;

  const DecodeArgs& p = P.d;
  const RingArgs& R = P.ring;
  const int L = R.L;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int cg = lane % CG, rs = lane / CG;
  const int c0 = wave * CW + cg * VEC;
  float* e_kp = s_dyn;           // [L][RS][PASSES]: element (j, row pp * RS + r) at j D + r PASSES + pp
  float* e_v = e_kp + L * D;     // [L][D]
  float* e_a = e_v + L * D;      // [L] exp(g)
  float* e_b = e_a + L;          // [L] beta
  constexpr int VE = 16 / EB, CPR = D / VE;  // ring row elements per 16-byte load, loads per row

  fold_units<(CDT >= 0)>(P, s_plan, [&](const int x) {
    const int b = x / p.Hv, h = x - (x / p.Hv) * p.Hv;
    const int64_t unit = (int64_t)p.slot_map[b] * p.Hv + h;
    const RingPos rp = ring_pos(R, p.slot_map[b]);
    const int st = rp.st, cnt = rp.cnt;

    // the lane offset is made opaque per unit so that the per-pass addresses
    // are not hoisted out of the unit loop (they would hold registers)
    int lane_off = rs * D + c0;
    asm volatile("" : "+v"(lane_off));
    ST* tile = static_cast<ST*>(p.pool) + unit * (int64_t)(D * D) + lane_off;
    typename IO::Raw raw[PASSES];
#pragma unroll
    for (int pp = 0; pp < PASSES; ++pp) raw[pp] = IO::load_raw(tile + pp * RS * D);

    const int64_t ring_e = unit * L;
    const int64_t kring_e = ring_key_base(p, p.slot_map[b], h, L);
    for (int t = tid; t < cnt; t += NTH) {
      const int j = (st + t) % L;
      e_a[t] = expf(R.g[ring_e + j]);
      e_b[t] = R.beta[ring_e + j];
    }
    for (int q = tid; q < cnt * CPR; q += NTH) {  // keys (permuted) and values, widened
      const int t = q / CPR, cc = (q - t * CPR) * VE;
      const int64_t row = (ring_e + (st + t) % L) * D + cc, krow = (kring_e + (st + t) % L) * D + cc;
      const u32x4 kw = *reinterpret_cast<const u32x4*>(static_cast<const char*>(R.k) + krow * EB);
      const u32x4 vw = *reinterpret_cast<const u32x4*>(static_cast<const char*>(R.v) + row * EB);
#pragma unroll
      for (int e = 0; e < VE; ++e) {
        float kf, vf;
        if constexpr (EB == 4) {
          kf = __uint_as_float(kw[e]);
          vf = __uint_as_float(vw[e]);
        } else {
          const uint32_t kh = (e & 1) ? (kw[e >> 1] >> 16) : (kw[e >> 1] & 0xffffu);
          const uint32_t vh = (e & 1) ? (vw[e >> 1] >> 16) : (vw[e >> 1] & 0xffffu);
          kf = p.in_dt == GDN_BF16 ? bf16_bits_to_f32(kh) : f16_bits_to_f32(kh);
          vf = p.in_dt == GDN_BF16 ? bf16_bits_to_f32(vh) : f16_bits_to_f32(vh);
        }
        const int r = cc + e;
        e_kp[t * D + (r % RS) * PASSES + r / RS] = kf;
        e_v[t * D + r] = vf;
      }
    }
    float s[PASSES][VEC];
#pragma unroll
    for (int pp = 0; pp < PASSES; ++pp) IO::widen(raw[pp], s[pp]);
    __syncthreads();

    // the cnt steps S <- e^{g} S;  d = beta (v - S^T k);  S <- S + k d^T, per column.
    // The tile is held as S = sc * S' with the decays in the scalar sc, so a
    // step costs one FMA per element: S' <- S' + k (d / sc).  When sc falls
    // below 2^-64 (an underflowed decay included) it is folded into S' before
    // the step, so 1/sc stays finite and the tile far from fp32 range.
    float sc = 1.f;
    for (int j = 0; j < cnt; ++j) {
      const float be = e_b[j];
      sc *= e_a[j];
      if (sc < 0x1p-64f) {  // uniform over the workgroup
#pragma unroll
        for (int pp = 0; pp < PASSES; ++pp)
#pragma unroll
          for (int e = 0; e < VEC; ++e) s[pp][e] *= sc;
        sc = 1.f;
      }
      float kr[PASSES];
      const float* kp = e_kp + j * D + rs * PASSES;
#pragma unroll
      for (int pp = 0; pp < PASSES; ++pp) kr[pp] = kp[pp];
      float xs[VEC];
#pragma unroll
      for (int e = 0; e < VEC; ++e) xs[e] = 0.f;
#pragma unroll
      for (int pp = 0; pp < PASSES; ++pp)
#pragma unroll
        for (int e = 0; e < VEC; ++e) xs[e] = fmaf(s[pp][e], kr[pp], xs[e]);
      const float inv = 1.f / sc;
      float dl[VEC];
#pragma unroll
      for (int e = 0; e < VEC; ++e) dl[e] = inv * be * (e_v[j * D + c0 + e] - sc * xor_sum_from<CG>(xs[e]));
#pragma unroll
      for (int pp = 0; pp < PASSES; ++pp)
#pragma unroll
        for (int e = 0; e < VEC; ++e) s[pp][e] = fmaf(kr[pp], dl[e], s[pp][e]);
    }
    if (sc != 1.f) {
#pragma unroll
      for (int pp = 0; pp < PASSES; ++pp)
#pragma unroll
        for (int e = 0; e < VEC; ++e) s[pp][e] *= sc;
    }
    if (cnt > 0) {
#pragma unroll
      for (int pp = 0; pp < PASSES; ++pp) IO::store(tile + pp * RS * D, s[pp]);
    }
    if constexpr (CDT >= 0) {
      using CIO = TileIO<CDT, VEC, false>;
      uint16_t* copy = static_cast<uint16_t*>(P.read_pool) + unit * (int64_t)(D * D) + lane_off;
#pragma unroll
      for (int pp = 0; pp < PASSES; ++pp) CIO::store(copy + pp * RS * D, s[pp]);
    }
    __syncthreads();  // LDS staging is reused by the next unit
  });
}

// e^x for x <= 0 on the hardware base-2 exponential (underflows to zero)
__device__ __forceinline__ float exp_neg(float x) { return __builtin_amdgcn_exp2f(x * 1.4426950408889634f); }

// ---------------------------------------------------------------- fold on MFMA
// The fold in its chunked (WY) form for D = 64 or 128 and rings of at most 16
// entries.  With G_i the prefix sums of g over the n committed entries,
//     d = (I + diag(beta) F)^-1 diag(beta) (V - diag(e^G) K S0),
//     F[i][j] = e^{G_i - G_j} k_i . k_j  (j < i),
//     S_n = e^{G_n} S0 + K^T diag(e^{G_n - G}) d,
// which is the sequential recurrence unrolled (the chunked form of the GDN
// paper's section on hardware-efficient training, with one chunk of n rows).
// K S0 and the rank-n update are fp32 MFMA chains (v_mfma_f32_16x16x4_f32):
// wave w holds columns 16 J .. 16 J + 15 (J = NJ w .. NJ w + NJ - 1) of every
// row in the accumulator layout (block (I, J), element r of lane (c, g): row
// 16 I + 4 g + r, column 16 J + c).  Both chains take their checkpoint or
// update operand straight from those registers by running the reduction over
// rows {16 I + 4 g + r : g} at step (I, r), the same permutation on both
// sides.  Each wave forms the 16 x 16 factor (I + diag(beta) F)^-1 diag(beta)
// itself from its own K K^T, so the waves never wait for one another after
// staging.  Entries past n are zero rows with zero gates and drop out.
constexpr int kFoldKTS = 20;  // LDS stride of the transposed keys: 16 entries + 4 (conflict-free reads)

// The fused fold (windows of up to TW positions) adds the window's w
// transposed [D][kFoldKTS] and its acc rows [TW][D].
__host__ __device__ inline size_t replay_fold_mfma_lds_bytes(int D, int TW = 0) {
  const size_t fused = TW > 0 ? (size_t)D * kFoldKTS + (size_t)TW * D : 0;
  return ((size_t)D * kFoldKTS + 2 * 16 * ((size_t)D + 4) + 2 * 16 + 4 * 16 * 17 + fused) * sizeof(float);
}

// Built for three workgroups per CU: at four (128 VGPRs) the kernel spilled
// registers to scratch, and at three it folds as fast or faster (fp32 fold
// steps 453-467 us against 454-482, bf16 373-396 against 372-407).
// TW > 0, fused (the prep ran first, see the prep): each folded unit also writes
// its window's outputs, o_t = scale (S^T w_t + acc_t) from the tile as stored, so
// the stream kernel skips its tile; windows of up to TW <= 16 positions.  W S for
// all positions at once is the K S0 product's shape (positions in place of
// entries): one pass of MFMAs whatever the window.
template <int SDT, int D, bool NT, int EB, int CDT, int TW = 0>
__global__ void __launch_bounds__(256, 3) gdn_replay_fold_mfma_kernel(const ReplayArgs P) {
  constexpr bool FUSED = TW > 0;
  static_assert(D == 64 || D == 128, "four waves of 16-column blocks");
  constexpr int NI = D / 16;  // row blocks
  constexpr int NJ = D / 64;  // column blocks per wave
  constexpr int KTS = kFoldKTS, VS = D + 4;
  constexpr int NTH = 256;
  using ST = typename StateElem<SDT>::T;

  extern __shared__ float s_dyn[];
  __shared__ FoldPlanLds s_plan;

  const DecodeArgs& p = P.d;
  const RingArgs& R = P.ring;
  const int L = R.L;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int c = lane & 15, g = lane >> 4;
  float* e_kt = s_dyn;                  // [D][KTS]: key element (entry e, row r) at r KTS + e
  float* e_k = e_kt + D * KTS;          // [16][VS]: key rows
  float* e_v = e_k + 16 * VS;           // [16][VS]: value rows
  float* e_G = e_v + 16 * VS;           // [16] prefix sums of g
  float* e_b = e_G + 16;                // [16] beta
  float* s_m = e_b + 16 + wave * 16 * 17;  // this wave's [16][17] factor
  float* e_wt = e_b + 16 + 4 * 16 * 17;    // FUSED: [D][KTS] w transposed: w_t[r] at r KTS + t
  float* e_acc = e_wt + D * KTS;           // FUSED: [TW][D] acc rows
  constexpr int VE = 16 / EB, CPR = D / VE;  // ring row elements per 16-byte load, loads per row
  const int T = P.T;
  // FUSED: the prep's vectors, [B Hv][T][2][D] floats right before the records in the workspace
  const float* ws_vec = FUSED ? reinterpret_cast<const float*>(P.rec) - (int64_t)p.B * p.Hv * T * 2 * D : nullptr;

  // Tile elements go through buffer instructions: one per-lane byte offset and
  // a scalar offset per element, so the 4 NI NJ accesses of a lane need no
  // address registers of their own.
  constexpr int SB = (int)sizeof(ST);
  auto ld_state = [&](__amdgpu_buffer_rsrc_t rs, int voff, int soff) -> float {
    if constexpr (SDT == GDN_F32) return __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(rs, voff, soff, 0));
    else if constexpr (SDT == GDN_BF16) return bf16_bits_to_f32(__builtin_amdgcn_raw_buffer_load_b16(rs, voff, soff, 0));
    else return f16_bits_to_f32(__builtin_amdgcn_raw_buffer_load_b16(rs, voff, soff, 0));
  };
  auto st_state = [&](__amdgpu_buffer_rsrc_t rs, int voff, int soff, float x, auto dt) {
    constexpr int DT = decltype(dt)::value;
    if constexpr (DT == GDN_F32)
      __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(x), rs, voff, soff, 0);
    else
      __builtin_amdgcn_raw_buffer_store_b16((unsigned short)(pack2<DT>(x, 0.f) & 0xffffu), rs, voff, soff, 0);
  };

  fold_units<(CDT >= 0)>(P, s_plan, [&](const int x) {
    const int b = x / p.Hv, h = x - (x / p.Hv) * p.Hv;
    // the slot as a scalar: with it in a vector register (where per-lane ring
    // addresses below put it) the tile's buffer descriptor would not be known
    // uniform, and every tile access would become a loop over distinct values
    int slot, st, cnt;
    if constexpr (FUSED) {  // the prep's record: slot and the pointers before the step
      const int4 rc = reinterpret_cast<const int4*>(P.rec)[x];
      slot = __builtin_amdgcn_readfirstlane(rc.x);
      st = __builtin_amdgcn_readfirstlane(rc.y);
      cnt = min(__builtin_amdgcn_readfirstlane(rc.z), 16);
    } else {
      slot = __builtin_amdgcn_readfirstlane(p.slot_map[b]);
      const RingPos rp = ring_pos(R, slot);
      st = rp.st;
      cnt = rp.cnt < 16 ? rp.cnt : 16;
    }
    const int64_t unit = (int64_t)slot * p.Hv + h;

    // ---- the checkpoint tile in the accumulator layout.  Element (16 I + r,
    // 16 jj) of a lane takes the row block's offset as the scalar offset (NI
    // values) and lane offset + (r D + 16 jj) as the vector one.  The lane
    // offset is made opaque here and again before the write-back, so those
    // NJ 4 vector offsets live only around the loads and around the stores
    // (as 4 NI NJ scalar offsets the constants spilled).
    // ---- first the committed entries' rows and gates, as raw bits: loads
    // complete in order, so waiting for them does not wait for the tile issued
    // after them.  Every thread loads a ring row in range (entry min(t, cnt - 1),
    // entry 0 of an empty ring) and the rows past cnt are zeroed when widened.
    const int64_t ring_e = unit * L;
    const int64_t kring_e = ring_key_base(p, slot, h, L);
    constexpr int QN = (16 * CPR + NTH - 1) / NTH;  // entry-row loads per thread
    const int clast = (cnt > 0 ? cnt : 1) - 1;
    auto ring_at = [&](int t) { const int x = st + t; return x >= L ? x - L : x; };  // st < L, t < L
    u32x4 kw[QN], vw[QN];
#pragma unroll
    for (int u = 0; u < QN; ++u) {
      const int q = min(tid + u * NTH, 16 * CPR - 1), t = q / CPR, cc = (q - t * CPR) * VE;
      const int pos = ring_at(min(t, clast));
      kw[u] = *reinterpret_cast<const u32x4*>(static_cast<const char*>(R.k) + ((kring_e + pos) * D + cc) * EB);
      vw[u] = *reinterpret_cast<const u32x4*>(static_cast<const char*>(R.v) + ((ring_e + pos) * D + cc) * EB);
    }
    float gg, be;
    {
      const int64_t j = ring_e + ring_at(min(lane & 15, clast));
      gg = R.g[j];
      be = R.beta[j];
    }
    // FUSED: the window's w and acc, 4 floats per load, all before the tile.  w
    // chunk q is rows 4 (q / TW).. of position q mod TW (consecutive lanes take
    // consecutive positions, so the transposed LDS writes below do not conflict);
    // acc chunk q is columns 4 (q mod D/4).. of position q / (D/4).  Positions
    // past T load position T - 1 (their w is zeroed, their acc never read).
    constexpr int QW = FUSED ? (TW * D / 4 + NTH - 1) / NTH : 1;
    f32x4 wq[QW], aq[QW];
    const float* wsu = FUSED ? ws_vec + (int64_t)x * T * 2 * D : nullptr;
    if constexpr (FUSED) {
#pragma unroll
      for (int u = 0; u < QW; ++u) {
        const int q = min(tid + u * NTH, TW * D / 4 - 1);
        const int tw = min(q % TW, T - 1), ta = min(q / (D / 4), T - 1);
        wq[u] = *reinterpret_cast<const f32x4*>(wsu + 2 * tw * D + 4 * (q / TW));
        aq[u] = *reinterpret_cast<const f32x4*>(wsu + (2 * ta + 1) * D + 4 * (q % (D / 4)));
      }
    }

    int lane_off = (4 * g * D + NJ * 16 * wave + c) * SB;
    asm volatile("" : "+v"(lane_off));
    const __amdgpu_buffer_rsrc_t rs_tile = __builtin_amdgcn_make_buffer_rsrc(
        static_cast<ST*>(p.pool) + unit * (int64_t)(D * D), 0, D * D * SB, 0x00020000);
    float s0[NI][NJ][4];
#pragma unroll
    for (int I = 0; I < NI; ++I)
#pragma unroll
      for (int jj = 0; jj < NJ; ++jj)
#pragma unroll
        for (int r = 0; r < 4; ++r) s0[I][jj][r] = ld_state(rs_tile, lane_off + (r * D + 16 * jj) * SB, 16 * I * D * SB);

    // ---- committed entries, widened: keys twice (transposed and by rows), values by rows
#pragma unroll
    for (int u = 0; u < QN; ++u) {
      const int q = tid + u * NTH, t = q / CPR, cc = (q - t * CPR) * VE;
      if (q < 16 * CPR) {
        const bool live = t < cnt;
#pragma unroll
        for (int e = 0; e < VE; ++e) {
          float kf, vf;
          if constexpr (EB == 4) {
            kf = __uint_as_float(kw[u][e]);
            vf = __uint_as_float(vw[u][e]);
          } else {
            const uint32_t kh = (e & 1) ? (kw[u][e >> 1] >> 16) : (kw[u][e >> 1] & 0xffffu);
            const uint32_t vh = (e & 1) ? (vw[u][e >> 1] >> 16) : (vw[u][e >> 1] & 0xffffu);
            kf = p.in_dt == GDN_BF16 ? bf16_bits_to_f32(kh) : f16_bits_to_f32(kh);
            vf = p.in_dt == GDN_BF16 ? bf16_bits_to_f32(vh) : f16_bits_to_f32(vh);
          }
          kf = live ? kf : 0.f;
          vf = live ? vf : 0.f;
          e_kt[(cc + e) * KTS + t] = kf;
          e_k[t * VS + cc + e] = kf;
          e_v[t * VS + cc + e] = vf;
        }
      }
    }
    if constexpr (FUSED) {
#pragma unroll
      for (int u = 0; u < QW; ++u) {
        const int q = tid + u * NTH;
        // used here, so the loads stay ahead of the tile's instead of sinking into the test
        asm volatile("" ::"v"(wq[u]), "v"(aq[u]));
        if (QW * NTH == TW * D / 4 || q < TW * D / 4) {
          const int t = q % TW, r0 = 4 * (q / TW);
#pragma unroll
          for (int k = 0; k < 4; ++k) e_wt[(r0 + k) * KTS + t] = t < T ? wq[u][k] : 0.f;
          *reinterpret_cast<f32x4*>(e_acc + 4 * q) = aq[u];  // position q / (D/4), columns 4 (q mod D/4)..
        }
      }
    }
    if (wave == 0 && lane < 16) {  // gates in live order, zero past cnt; prefix sums within the row
      gg = lane < cnt ? gg : 0.f;
      be = lane < cnt ? be : 0.f;
#pragma unroll
      for (int off = 1; off < 16; off <<= 1) {
        const float y = __shfl_up(gg, off, 16);
        if (lane >= off) gg += y;
      }
      e_G[lane] = gg;
      e_b[lane] = be;
    }
    __syncthreads();

    // (FUSED: a folding unit has entries; with none the update below would return S0
    // unchanged, and without the test the tile's loads are known complete before
    // the outputs read it, so no wait there also covers the write-back)
    if (FUSED || cnt > 0) {
      const float Gn = e_G[15];  // gates past cnt are zero: entry 15 carries G_cnt
      // ---- K K^T; element r of lane (c, g) is (4 g + r, c)
      f32x4 kk = {0.f, 0.f, 0.f, 0.f};
#pragma unroll 8
      for (int s4 = 0; s4 < D / 4; ++s4) {
        const float a = e_kt[(4 * s4 + g) * KTS + c];
        kk = __builtin_amdgcn_mfma_f32_16x16x4f32(a, a, kk, 0, 0, 0);
      }
      // M = I + diag(beta) F, strictly lower part (the unit diagonal is implicit)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int i = 4 * g + r;
        s_m[i * 17 + c] = c < i ? e_b[i] * exp_neg(e_G[i] - e_G[c]) * kk[r] : 0.f;
      }
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
      __builtin_amdgcn_wave_barrier();
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
      // X = M^-1 by forward substitution (lane c < 16 owns column c), then
      // the factor X diag(beta) replaces M in place
      if (lane < 16) {
        int cz = c;  // opaque: keeps the 16 identity entries from being held across units
        asm volatile("" : "+v"(cz));
        float xc[16];
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          float v = i == cz ? 1.f : 0.f;
#pragma unroll
          for (int k = 0; k < i; ++k) v = fmaf(-s_m[i * 17 + k], xc[k], v);
          xc[i] = v;
        }
        const float bc = e_b[c];
#pragma unroll
        for (int i = 0; i < 16; ++i) s_m[i * 17 + c] = xc[i] * bc;
      }
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
      __builtin_amdgcn_wave_barrier();
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");

      // ---- K S0 for this wave's columns, reduction over rows {16 I + 4 g + r}
      f32x4 ks[NJ];
#pragma unroll
      for (int jj = 0; jj < NJ; ++jj) ks[jj] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int I = 0; I < NI; ++I)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const float a = e_kt[(16 * I + 4 * g + r) * KTS + c];
#pragma unroll
          for (int jj = 0; jj < NJ; ++jj) ks[jj] = __builtin_amdgcn_mfma_f32_16x16x4f32(a, s0[I][jj][r], ks[jj], 0, 0, 0);
        }
      // ---- R = V - diag(e^G) K S0, then d = factor . R (reduction over entries
      // {4 g + r}), each row scaled by e^{G_n - G_e} for the update
      f32x4 u[NJ];
      float eGe[4], wGe[4];
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const float Ge = e_G[4 * g + r];
        eGe[r] = exp_neg(Ge);
        wGe[r] = exp_neg(Gn - Ge);
      }
#pragma unroll
      for (int jj = 0; jj < NJ; ++jj) {
        const int col = 16 * (NJ * wave + jj) + c;
#pragma unroll
        for (int r = 0; r < 4; ++r) ks[jj][r] = e_v[(4 * g + r) * VS + col] - eGe[r] * ks[jj][r];
        u[jj] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int r = 0; r < 4; ++r)
          u[jj] = __builtin_amdgcn_mfma_f32_16x16x4f32(s_m[c * 17 + 4 * g + r], ks[jj][r], u[jj], 0, 0, 0);
#pragma unroll
        for (int r = 0; r < 4; ++r) u[jj][r] *= wGe[r];
      }
      // ---- S_n = e^{G_n} S0 + K^T (scaled d), reduction over entries {4 g + r}
      const float eGn = exp_neg(Gn);
#pragma unroll
      for (int I = 0; I < NI; ++I) {
        f32x4 acc[NJ];
#pragma unroll
        for (int jj = 0; jj < NJ; ++jj)
#pragma unroll
          for (int r = 0; r < 4; ++r) acc[jj][r] = eGn * s0[I][jj][r];
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const float a = e_k[(4 * g + r) * VS + 16 * I + c];
#pragma unroll
          for (int jj = 0; jj < NJ; ++jj) acc[jj] = __builtin_amdgcn_mfma_f32_16x16x4f32(a, u[jj][r], acc[jj], 0, 0, 0);
        }
#pragma unroll
        for (int jj = 0; jj < NJ; ++jj)
#pragma unroll
          for (int r = 0; r < 4; ++r) s0[I][jj][r] = acc[jj][r];
      }
      constexpr int NC = 2;  // FUSED: MFMA chains per column block of the outputs
      [[maybe_unused]] f32x4 o[NC][NJ];
      if constexpr (FUSED) {
        // the window's outputs from the tile as stored (formed here, stored after
        // the write-back):
        // O = W S with W [positions][rows] as the MFMA's A operand (lane (c, g)
        // gives w_c at rows 16 I + 4 g + r) and the tile as B, two chains per
        // column block; element r of lane (c, g) is position 4 g + r, column c
        if constexpr (SDT != GDN_F32) {  // rounded in place (the write-back's rounding then changes nothing)
#pragma unroll
          for (int I = 0; I < NI; ++I)
#pragma unroll
            for (int jj = 0; jj < NJ; ++jj)
#pragma unroll
              for (int r = 0; r < 4; ++r) s0[I][jj][r] = unpack_lo<SDT>(pack2<SDT>(s0[I][jj][r], 0.f));
        }
#pragma unroll
        for (int hh = 0; hh < NC; ++hh)
#pragma unroll
          for (int jj = 0; jj < NJ; ++jj) o[hh][jj] = f32x4{0.f, 0.f, 0.f, 0.f};
        if (TW <= 4 && T == 1) {
          // one position: lane (c, g) sums its rows {16 I + 4 g + r} on the vector
          // ALU (a short chain per row block) and the four row groups meet in two
          // lane exchanges; the MFMA would form 16 positions for the one
          float part[NJ][NI];
#pragma unroll
          for (int I = 0; I < NI; ++I) {
            float w[4];
#pragma unroll
            for (int r = 0; r < 4; ++r) w[r] = e_wt[(16 * I + 4 * g + r) * KTS];
#pragma unroll
            for (int jj = 0; jj < NJ; ++jj) {
              float x = s0[I][jj][0] * w[0];
#pragma unroll
              for (int r = 1; r < 4; ++r) x = fmaf(s0[I][jj][r], w[r], x);
              part[jj][I] = x;
            }
          }
#pragma unroll
          for (int jj = 0; jj < NJ; ++jj) {
#pragma unroll
            for (int n = NI / 2; n >= 1; n /= 2)
#pragma unroll
              for (int I = 0; I < n; ++I) part[jj][I] += part[jj][I + n];
            float x = part[jj][0];
            x += __shfl_xor(x, 16, 64);
            x += __shfl_xor(x, 32, 64);
            o[0][jj][0] = x;  // position 0 in the lanes with g = 0, as from the MFMA
          }
        } else {
#pragma unroll
          for (int I = 0; I < NI; ++I)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
              const float a = c < T ? e_wt[(16 * I + 4 * g + r) * KTS + c] : 0.f;  // columns past TW unwritten
#pragma unroll
              for (int jj = 0; jj < NJ; ++jj)
                o[I % NC][jj] = __builtin_amdgcn_mfma_f32_16x16x4f32(a, s0[I][jj][r], o[I % NC][jj], 0, 0, 0);
            }
#pragma unroll
          for (int jj = 0; jj < NJ; ++jj)
#pragma unroll
            for (int r = 0; r < 4; ++r) o[0][jj][r] += o[1][jj][r];
        }
      }
      // ---- write back, rounded once
      int lane_st = lane_off;
      asm volatile("" : "+v"(lane_st));
#pragma unroll
      for (int I = 0; I < NI; ++I)
#pragma unroll
        for (int jj = 0; jj < NJ; ++jj)
#pragma unroll
          for (int r = 0; r < 4; ++r)
            st_state(rs_tile, lane_st + (r * D + 16 * jj) * SB, 16 * I * D * SB, s0[I][jj][r],
                     std::integral_constant<int, SDT>{});
      if constexpr (FUSED) {  // the outputs after the write-back, one test of their dtype
        auto put = [&](auto odt) {
#pragma unroll
          for (int jj = 0; jj < NJ; ++jj) {
            const int col = 16 * (NJ * wave + jj) + c;
#pragma unroll
            for (int r = 0; r < 4; ++r) {
              const int t = 4 * g + r;
              if (t < T)
                store_elem(p.out, (((int64_t)b * T + t) * p.Hv + h) * D + col,
                           p.scale * (o[0][jj][r] + e_acc[t * D + col]), decltype(odt)::value);
            }
          }
        };
        if (p.out_dt == GDN_BF16) put(std::integral_constant<int, GDN_BF16>{});
        else if (p.out_dt == GDN_F16) put(std::integral_constant<int, GDN_F16>{});
        else put(std::integral_constant<int, GDN_F32>{});
      }
    }
    if constexpr (CDT >= 0) {
      const __amdgpu_buffer_rsrc_t rs_copy = __builtin_amdgcn_make_buffer_rsrc(
          static_cast<uint16_t*>(P.read_pool) + unit * (int64_t)(D * D), 0, D * D * 2, 0x00020000);
      int coff = (4 * g * D + NJ * 16 * wave + c) * 2;
      asm volatile("" : "+v"(coff));
#pragma unroll
      for (int I = 0; I < NI; ++I)
#pragma unroll
        for (int jj = 0; jj < NJ; ++jj)
#pragma unroll
          for (int r = 0; r < 4; ++r)
            st_state(rs_copy, coff + (r * D + 16 * jj) * 2, 16 * I * D * 2, s0[I][jj][r], std::integral_constant<int, CDT>{});
    }
    __syncthreads();  // LDS staging is reused by the next unit
  }, std::integral_constant<bool, FUSED>{});
}

// ---------------------------------------------------------------- prep
// Dynamic LDS of the prep kernel: packed keys and values [L][D * EB / 4 + 1]
// words each (live entries, at most L: the committed ones then the window),
// packed window queries [T][...], then floats: beta and prefix sums of g [L]
// each, decay-weighted key products [L][L], key / query products [L][T],
// coefficients c and e^G c [T][L] each.
__host__ __device__ inline size_t replay_prep_words(int D, int EB, int L, int T) {
  const size_t Ls = (size_t)L, Ts = (size_t)T, row = (size_t)D * EB / 4 + 1;
  return 2 * Ls * row + Ts * row + 2 * Ls + Ls * Ls + 3 * Ls * Ts;
}
__host__ __device__ inline size_t replay_prep_lds_bytes(int D, int L, int T) {
  return replay_prep_words(D, 4, L, T) * sizeof(float);  // the f32-input size bounds both
}

// One workgroup of NWP waves per unit.  Loads are issued in two rounds: the
// window rows (which need only the row index) together with the slot, then
// the unit's ring pointers and, after them, only its live ring entries and
// their gates (many workgroups share a CU, so the extra dependent load is
// hidden, and the ring bytes read drop to the live entries).  Keys and
// values stay packed (input dtype) in LDS and are widened on use.  Phases (one barrier each): staging and gates; the Gram
// and key / query MFMA tiles, shared over the waves; the back substitution,
// one wave per window position; w and acc, one thread per element.
template <int D, int EB, int NWP>
__global__ void __launch_bounds__(NWP * 64) gdn_replay_prep_kernel(const ReplayArgs P, float* __restrict__ ws) {
  constexpr int NTH = NWP * 64;
  constexpr int VE = 16 / EB;             // elements per 16-byte load
  constexpr int CPR = D / VE;             // 16-byte loads per row
  constexpr int LDW = D * EB / 4 + 1;     // LDS words per packed row (+1: bank spread)
  constexpr int RB = NTH / CPR;           // rows per workgroup-wide load round
  static_assert(64 % CPR == 0, "a wave covers whole rows");
  constexpr int NR = 2;                   // load rounds held in registers per row kind
  using Row = PackedRow<EB>;
  extern __shared__ uint32_t s_words[];

  const DecodeArgs& p = P.d;
  const RingArgs& R = P.ring;
  const int T = P.T, L = R.L;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int b = blockIdx.x / p.Hv;
  const int h = blockIdx.x - b * p.Hv;
  const int hk = h / (p.Hv / p.Hk);
  uint32_t* e_k = s_words;                  // [L][LDW] live order: committed, then window
  uint32_t* e_v = e_k + L * LDW;            // [L][LDW]
  uint32_t* e_q = e_v + L * LDW;            // [T][LDW]
  float* e_b = reinterpret_cast<float*>(e_q + T * LDW);  // [L]
  float* e_G = e_b + L;                     // [L]
  float* s_F = e_G + L;                     // [L][L]
  float* s_kq = s_F + L * L;                // [L][T]
  float* s_c = s_kq + L * T;                // [T][L]
  float* s_ec = s_c + T * L;                // [T][L]

  const int lr = tid / CPR, lc = (tid - lr * CPR) * VE;  // this thread's row offset and column in a round
  const char* kin = static_cast<const char*>(p.k);
  const char* vin = static_cast<const char*>(p.v);
  const char* qin = static_cast<const char*>(p.q);

  // NR load rounds (RB rows each) through registers; `rowptr(r)` gives the
  // global address of row r, `dst(r)` its LDS row (or null to skip).
  auto load_batch = [&](int r0, int nrows, auto rowptr, u32x4 (&x)[NR]) {
#pragma unroll
    for (int u = 0; u < NR; ++u) {
      const int r = (r0 + u) * RB + lr;
      u32x4 z = {0u, 0u, 0u, 0u};
      if (r < nrows) z = *reinterpret_cast<const u32x4*>(rowptr(r) + lc * EB);
      x[u] = z;
    }
  };
  auto commit_batch = [&](int r0, int nrows, auto dst, const u32x4 (&x)[NR]) {
#pragma unroll
    for (int u = 0; u < NR; ++u) {
      const int r = (r0 + u) * RB + lr;
      uint32_t* d = (r < nrows) ? dst(r) : nullptr;
      if (d != nullptr) {
#pragma unroll
        for (int w = 0; w < 4; ++w) d[lc * EB / 4 + w] = x[u][w];
      }
    }
  };
  auto win_k = [&](int t) { return kin + (((int64_t)b * T + t) * p.Hk + hk) * D * EB; };
  auto win_v = [&](int t) { return vin + (((int64_t)b * T + t) * p.Hv + h) * D * EB; };
  auto win_q = [&](int t) { return qin + (((int64_t)b * T + t) * p.Hk + hk) * D * EB; };

  // ---- load round 1: the unit record (slot and the ring pointers after any fold,
  // written by the fold's check), the first window rows and the window gate inputs
  const int4 rc = reinterpret_cast<const int4*>(P.rec)[blockIdx.x];
  const int slot = rc.x;
  u32x4 wk[NR], wv[NR], wq[NR];
  load_batch(0, T, win_k, wk);
  load_batch(0, T, win_v, wv);
  load_batch(0, T, win_q, wq);
  float ga = 0.f, gb = 0.f;
  if (tid < T) {
    const int64_t gi = ((int64_t)b * T + tid) * p.Hv + h;
    ga = load_elem(p.a, gi, p.in_dt);
    gb = load_elem(p.b, gi, p.in_dt);
  }
  if (slot < 0) return;  // padded row (the stream kernel writes zeros)
  const int64_t unit = (int64_t)slot * p.Hv + h;

  // ---- load round 2: the unit's live entries (committed, in ring order from the
  // start pointer) and their gates
  const int64_t ring_e = unit * L;
  const int st = rc.y;                 // in [0, L)
  const int cnt = min(rc.z, L - T);    // the fold kernel left room for the window
  const int n_all = cnt + T;           // <= L
  const int64_t kring_e = ring_key_base(p, slot, h, L);
  const char* rk = static_cast<const char*>(R.k) + kring_e * D * EB;
  const char* rv = static_cast<const char*>(R.v) + ring_e * D * EB;
  auto live_src_k = [&](int i) { return rk + (int64_t)((st + i) % L) * D * EB; };
  auto live_src_v = [&](int i) { return rv + (int64_t)((st + i) % L) * D * EB; };
  u32x4 xk[NR], xv[NR];
  load_batch(0, cnt, live_src_k, xk);
  load_batch(0, cnt, live_src_v, xv);
  float rg = 0.f, rb = 0.f;
  if (tid < cnt) {
    const int64_t j = ring_e + (st + tid) % L;
    rg = R.g[j];
    rb = R.beta[j];
  }

  // ---- commit in live order: committed entries 0..cnt-1, then the window
  auto live_k = [&](int i) -> uint32_t* { return e_k + i * LDW; };
  auto live_v = [&](int i) -> uint32_t* { return e_v + i * LDW; };
  auto wdst_k = [&](int t) -> uint32_t* { return e_k + (cnt + t) * LDW; };
  auto wdst_v = [&](int t) -> uint32_t* { return e_v + (cnt + t) * LDW; };
  auto wdst_q = [&](int t) -> uint32_t* { return e_q + t * LDW; };
  commit_batch(0, T, wdst_k, wk);
  commit_batch(0, T, wdst_v, wv);
  commit_batch(0, T, wdst_q, wq);
  commit_batch(0, cnt, live_k, xk);
  commit_batch(0, cnt, live_v, xv);
  for (int r0 = NR; r0 * RB < T; r0 += NR) {  // longer windows
    load_batch(r0, T, win_k, wk);
    load_batch(r0, T, win_v, wv);
    load_batch(r0, T, win_q, wq);
    commit_batch(r0, T, wdst_k, wk);
    commit_batch(r0, T, wdst_v, wv);
    commit_batch(r0, T, wdst_q, wq);
  }
  for (int r0 = NR; r0 * RB < cnt; r0 += NR) {  // longer rings
    load_batch(r0, cnt, live_src_k, xk);
    load_batch(r0, cnt, live_src_v, xv);
    commit_batch(r0, cnt, live_k, xk);
    commit_batch(r0, cnt, live_v, xv);
  }
  // gates and their prefix sums in live order (wave 0): lane j takes live
  // entry j, a committed entry from ring position (st + j) % L or window
  // position j - cnt
  float wg = 0.f, wbeta = 0.f;
  if (tid < T) {
    wg = gate_g(ga, p.A_log[h], p.dt_bias[h]);
    wbeta = sigmoid_f(gb);
  }
  if (wave == 0) {
    const float g_r = rg, b_r = rb;  // lane j < cnt loaded live entry j
    const int from_win = (lane - cnt) & 63;
    const float g_w = __shfl(wg, from_win, 64), b_w = __shfl(wbeta, from_win, 64);
    const float g = lane < cnt ? g_r : (lane < n_all ? g_w : 0.f);
    const float be = lane < cnt ? b_r : (lane < n_all ? b_w : 0.f);
    float x = g;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
      const float y = __shfl_up(x, off, 64);
      if (lane >= off) x += y;
    }
    if (lane < L) {
      e_b[lane] = be;
      e_G[lane] = x;
    }
  }
  __syncthreads();

  // ---- append the window to the ring (raw input bytes) and move the pointers
  const int base = (st + cnt) % L;
  for (int x = tid; x < T * CPR; x += NTH) {
    const int t = x / CPR, c = (x - t * CPR) * VE;
    const int64_t j = ring_e + (base + t) % L, kj = kring_e + (base + t) % L;
    const int64_t ko = ((((int64_t)b * T + t) * p.Hk + hk) * D + c) * EB;
    const int64_t vo = ((((int64_t)b * T + t) * p.Hv + h) * D + c) * EB;
    if (appends_keys(p, h))
      *reinterpret_cast<u32x4*>(static_cast<char*>(R.k) + (kj * D + c) * EB) = *reinterpret_cast<const u32x4*>(kin + ko);
    *reinterpret_cast<u32x4*>(static_cast<char*>(R.v) + (j * D + c) * EB) =
        *reinterpret_cast<const u32x4*>(vin + vo);
  }
  if (tid < T) {
    const int64_t j = ring_e + (base + tid) % L;
    R.g[j] = wg;
    R.beta[j] = wbeta;
  }
  if (tid == 0 && h == 0) {  // the slot's pointers, once per slot
    R.start[slot] = st;
    R.count[slot] = n_all;
  }

  // ---- decay-weighted key products s_F[i][j] = e^{G_i - G_j} k_j . k_i (j < i)
  // and key / query products s_kq[j][t] = e^{G_{cnt+t} - G_j} k_j . q_t
  // (j <= cnt + t), 16 x 16 MFMA tiles shared over the waves; every exponent <= 0
  {
    const int nt = (n_all + 15) >> 4, qt = (T + 15) >> 4;
    const int n_gt = nt * (nt + 1) / 2;
    const int i4 = 4 * (lane >> 4), jc = lane & 15;
    for (int job = wave; job < n_gt + nt * qt; job += NWP) {
      int I, J;
      const bool gram = job < n_gt;
      if (gram) {
        I = 0;
        int rem = job;
        while (rem >= nt - I) {
          rem -= nt - I;
          ++I;
        }
        J = I + rem;
      } else {
        I = (job - n_gt) / qt;
        J = (job - n_gt) - I * qt;
      }
      const uint32_t* Y = gram ? e_k + 16 * J * LDW : e_q + 16 * J * LDW;
      const int ny = gram ? n_all - 16 * J : T - 16 * J;
      const f32x4 g = tile_xyt<D, EB>(e_k + 16 * I * LDW, n_all - 16 * I, Y, ny, LDW, p.in_dt, lane);
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int a = 16 * I + i4 + r, j = 16 * J + jc;
        if (gram) {
          if (a < j && j < n_all) s_F[j * L + a] = expf(e_G[j] - e_G[a]) * g[r];
        } else if (a < n_all && j < T) {
          s_kq[a * T + j] = a <= cnt + j ? expf(e_G[cnt + j] - e_G[a]) * g[r] : 0.f;
        }
      }
    }
  }
  __syncthreads();

  // ---- back substitution, one wave per window position: lane j holds the residual of live entry j
  for (int t = wave; t < T; t += NWP) {
    const int e_last = cnt + t;
    const int j = lane;
    const bool live = j <= e_last;
    float r = live ? s_kq[j * T + t] : 0.f;
    float cj = 0.f;
    for (int i = e_last; i >= 0; --i) {
      // c_i = beta_i * residual_i, then every earlier entry drops its term
      const float f = j < i ? s_F[i * L + j] : 0.f;
      const float ci =
          __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, e_b[i] * r), i));
      if (j == i) cj = ci;
      r = fmaf(-f, ci, r);
    }
    if (j < n_all) {
      s_c[t * L + j] = live ? cj : 0.f;
      s_ec[t * L + j] = live ? expf(e_G[j]) * cj : 0.f;
    }
  }
  __syncthreads();
  // ---- w_t = e^{G_n} q_t - sum_j e^{G_j} c_j k_j and acc_t = sum_j c_j v_j, to the workspace
  float* wsu = ws + ((int64_t)b * p.Hv + h) * T * 2 * D;
  for (int x = tid; x < T * D; x += NTH) {
    const int t = x / D, c = x - t * D;
    const int e_last = cnt + t;
    float w = expf(e_G[e_last]) * Row::get(e_q + t * LDW, c, p.in_dt);
    float acc = 0.f;
    for (int jj = 0; jj <= e_last; ++jj) {
      w = fmaf(-s_ec[t * L + jj], Row::get(e_k + jj * LDW, c, p.in_dt), w);
      acc = fmaf(s_c[t * L + jj], Row::get(e_v + jj * LDW, c, p.in_dt), acc);
    }
    wsu[(2 * t) * D + c] = w;
    wsu[(2 * t + 1) * D + c] = acc;
  }
}

// ---------------------------------------------------------------- prep, one wave per unit
// For rings of at most 16 entries, 16-bit inputs and D = 64 or 128: one wave
// per unit and no workgroup barrier.  For the key products lane l stands for
// live entry e = l % 16 (the committed entries in ring order, then the window)
// and holds that entry's key row in the operand layout of the 16x16x32 MFMA:
// with g = l / 16 and NS = D / 32, the 16-byte chunks NS g .. NS g + NS - 1,
// the reduction index permuted alike on both sides so that each lane reads
// one contiguous run.  K K^T is then one MFMA chain over the key registers and
// K Q^T a second over the window queries.  Every 16-lane row runs the back
// substitution alike.  For w and acc the wave switches to columns: lane l owns
// columns CPL l .. CPL l + CPL - 1 (CPL = D / 64) of every value row (loaded
// one row per instruction) and of every key row (read back from LDS), so both
// are plain sums over the entries with the coefficients in scalar registers.
// The window goes to the ring straight from the registers that loaded it.
//
// FUSED: the prep runs first in the step and decides each unit's fold itself
// (count + T > L).  It writes the unit's record for the fold and the stream
// (slot, ring pointers before the step, fold flag), forms w and acc over the
// live entries after any fold, and appends the window to the ring only for
// units that do not fold: a folding unit's window would overwrite the entries
// the fold still reads, so the stream appends it.  The ring pointers are not
// moved here (another value head's prep of the slot may still be reading them):
// the stream, the last kernel of the step, moves them.

// Dynamic LDS of the one-wave prep (bytes): window queries [T][D] and key rows
// [16][D] (16-bit), the strictly lower decay-weighted key products packed by
// rows (F[i][j] at i (i - 1) / 2 + j, 120 floats) and key / query products
// [16][T].  Under 5 KiB at D = 128, T = 1, so 32 waves fit a CU.
__host__ __device__ inline size_t replay_prep16_lds_bytes(int D, int T) {
  return (size_t)T * D * 2 + 16 * (size_t)D * 2 + 120 * sizeof(float) + 16 * (size_t)T * sizeof(float);
}

template <int D, int IDT, bool FUSED>
__global__ void __launch_bounds__(64, 8) gdn_replay_prep16_kernel(const ReplayArgs P, float* __restrict__ ws) {
  static_assert(D == 64 || D == 128, "two or four 16-byte chunks per lane");
  static_assert(IDT == GDN_BF16 || IDT == GDN_F16, "16-bit inputs");
  constexpr int NS = D / 32;   // MFMA chunks per lane and row
  constexpr int RB = 2 * D;    // bytes per row
  constexpr int CPL = D / 64;  // columns per lane in the column layout
  typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
  typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
  extern __shared__ uint32_t s_words[];

  const DecodeArgs& p = P.d;
  const RingArgs& R = P.ring;
  const int T = P.T, L = R.L;
  const int lane = threadIdx.x, e = lane & 15, g = lane >> 4;
  const int u = GDN_REPLAY_PREP_XCD ? xcd_unit(blockIdx.x, gridDim.x) : (int)blockIdx.x;
  const int b = u / p.Hv;
  const int h = u - b * p.Hv;
  const int hk = h / (p.Hv / p.Hk);
  const int coff = g * NS * 16;  // byte offset of this lane's MFMA run in a row
  const int ccol = CPL * lane;   // first column of this lane in the column layout
  uint16_t* s_q = reinterpret_cast<uint16_t*>(s_words);  // [T][D]
  uint16_t* s_k = s_q + T * D;                           // [16][D]
  float* s_F = reinterpret_cast<float*>(s_k + 16 * D);   // F[i][j], j < i, at i (i - 1) / 2 + j
  float* s_kq = s_F + 120;                               // [16][T]
  const u32x4 z4 = {0u, 0u, 0u, 0u};
  // this lane's CPL 16-bit columns of a row (zero-extended when CPL = 1)
  auto cols_at = [&](const void* row) -> uint32_t {
    if constexpr (CPL == 2) return *reinterpret_cast<const uint32_t*>(static_cast<const char*>(row) + 2 * ccol);
    else return *reinterpret_cast<const uint16_t*>(static_cast<const char*>(row) + 2 * ccol);
  };
  auto widen = [&](uint32_t x, float (&f)[CPL]) {
    f[0] = IDT == GDN_BF16 ? bf16_bits_to_f32(x & 0xffffu) : f16_bits_to_f32(x & 0xffffu);
    if constexpr (CPL == 2) f[1] = IDT == GDN_BF16 ? bf16_bits_to_f32(x >> 16) : f16_bits_to_f32(x >> 16);
  };

  // ---- load round 1: the unit record (slot and the ring pointers after any fold,
  // written by the fold's check; FUSED: the slot, then the pointers in a round of
  // their own) and the window queries (lane e: query e)
  int4 rc;
  if constexpr (FUSED) {
    rc.x = p.slot_map[b];
    if (rc.x < 0 || (int64_t)rc.x >= p.num_slots) rc.x = -1;
  } else {
    rc = reinterpret_cast<const int4*>(P.rec)[u];
  }
  const int slot = rc.x;
  const float A_log = p.A_log[h], dt_bias = p.dt_bias[h];
  u32x4 qx[NS];
  {
    const bool qv = e < T;
    const char* src = static_cast<const char*>(p.q) + (((int64_t)b * T + (qv ? e : 0)) * p.Hk + hk) * RB + coff;
#pragma unroll
    for (int s = 0; s < NS; ++s) {  // every lane loads (a valid row), so no branch splits the round
      const u32x4 x = *reinterpret_cast<const u32x4*>(src + 16 * s);
      qx[s] = qv ? x : z4;
    }
    // taken here, so the compiler issues the query loads beside the record load instead
    // of after the record's test (that had made them a dependent round of their own)
#pragma unroll
    for (int s = 0; s < NS; ++s) asm volatile("" : "+v"(qx[s]));
  }
  bool folds = false;  // FUSED: this unit folds in this step
  if constexpr (FUSED) {
    if (slot < 0) {  // padded row: a record that neither folds nor streams a tile
      if (lane == 0) reinterpret_cast<int4*>(P.rec)[u] = int4{-1, 0, 0, 0};
      return;
    }
    const RingPos rp = ring_pos(R, slot);
    folds = rp.cnt + T > L;
    if (lane == 0) reinterpret_cast<int4*>(P.rec)[u] = int4{slot, rp.st, rp.cnt, folds ? 1 : 0};
    rc.y = folds ? (rp.st + rp.cnt) % L : rp.st;  // the pointers after any fold, as the fold's check gives them
    rc.z = folds ? 0 : rp.cnt;
  }
  if (slot < 0) return;  // padded row (the stream kernel writes zeros)
  const int64_t unit = (int64_t)slot * p.Hv + h;
  const int st = rc.y;                 // in [0, L)
  const int cnt = min(rc.z, L - T);    // the fold left room for the window
  const int n_all = cnt + T;           // <= L <= 16

  // the queries wait in LDS (their registers are free during load round 2) for the
  // K Q^T operands and the e^{G_n} q term of w
  if (e < T) {
#pragma unroll
    for (int s = 0; s < NS; ++s) *reinterpret_cast<u32x4*>(s_q + e * D + 8 * (NS * g + s)) = qx[s];
  }
  asm volatile("" ::: "memory");

  // ---- load round 2: lane e loads key row e, a committed entry from ring position
  // (st + e) % L and a window one (position e - cnt) from the inputs; that ring
  // position is also where a window entry is appended.  Value rows go by
  // columns: row j is one load over the wave.
  const bool live = e < n_all, committed = e < cnt;
  const int tw = committed ? 0 : min(e - cnt, T - 1);
  // ring position of live entry j: st < L and j < n_all <= L, so one subtraction wraps it
  auto ring_at = [&](int j) { const int x = st + j; return x >= L ? x - L : x; };
  const int pe = live ? ring_at(e) : 0;
  const int64_t rj = unit * L + pe, krj = ring_key_base(p, slot, h, L) + pe;
  const char* ks = committed ? static_cast<const char*>(R.k) + krj * RB
                             : static_cast<const char*>(p.k) + (((int64_t)b * T + tw) * p.Hk + hk) * RB;
  u32x4 kx[NS];
#pragma unroll
  for (int s = 0; s < NS; ++s) {  // a lane past the live entries reads window row T - 1
    const u32x4 x = *reinterpret_cast<const u32x4*>(ks + coff + 16 * s);
    kx[s] = live ? x : z4;
  }
  // value rows through two buffer resources, the unit's ring entries and its
  // window rows in the inputs, with the row's byte offset as the scalar offset
  const __amdgpu_buffer_rsrc_t rs_vring = __builtin_amdgcn_make_buffer_rsrc(
      static_cast<char*>(R.v) + unit * L * RB, 0, L * RB, 0x00020000);
  const __amdgpu_buffer_rsrc_t rs_vwin = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<char*>(static_cast<const char*>(p.v)) + ((int64_t)b * T * p.Hv + h) * RB, 0,
      ((T - 1) * p.Hv + 1) * RB, 0x00020000);
  const int vstep = p.Hv * RB;
  auto vcols = [&](__amdgpu_buffer_rsrc_t rs, int soff) -> uint32_t {
    if constexpr (CPL == 2) return __builtin_amdgcn_raw_buffer_load_b32(rs, 2 * ccol, soff, 0);
    else return __builtin_amdgcn_raw_buffer_load_b16(rs, 2 * ccol, soff, 0);
  };
  uint32_t vr[16];
#pragma unroll
  for (int j = 0; j < 16; ++j) {
    uint32_t x = 0u;
    if (j < n_all) x = j < cnt ? vcols(rs_vring, ring_at(j) * RB) : vcols(rs_vwin, (j - cnt) * vstep);  // uniform
    vr[j] = x;
  }
  // both gate sources are read in every lane (in range for any lane) and selected
  float gl, bl;
  {
    float gr = R.g[rj], br = R.beta[rj];
    const int64_t gi = ((int64_t)b * T + tw) * p.Hv + h;
    // the input dtype as a constant: a run-time switch put a full wait between the two loads
    float ga = load_elem(p.a, gi, IDT), gb = load_elem(p.b, gi, IDT);
    // taken here, so that all four loads go out in this round (the compiler had sunk
    // some of them into the branches below, each a dependent round of its own)
    asm volatile("" : "+v"(gr), "+v"(br), "+v"(ga), "+v"(gb));
    gl = live ? (committed ? gr : gate_g(ga, A_log, dt_bias)) : 0.f;
    bl = live ? (committed ? br : sigmoid_f(gb)) : 0.f;
  }

  // ---- prefix sums G of g in live order (each 16-lane row alike)
  float G = gl;
#pragma unroll
  for (int off = 1; off < 16; off <<= 1) {
    const float y = __shfl_up(G, off, 16);
    if (e >= off) G += y;
  }

  // ---- key rows to LDS for the column layout; append the window to the ring
#pragma unroll
  for (int s = 0; s < NS; ++s) *reinterpret_cast<u32x4*>(s_k + e * D + 8 * (NS * g + s)) = kx[s];
  if (live && !committed && !folds) {  // a folding unit's window is appended by the stream
    if (appends_keys(p, h)) {
      char* kd = static_cast<char*>(R.k) + krj * RB + coff;
#pragma unroll
      for (int s = 0; s < NS; ++s) *reinterpret_cast<u32x4*>(kd + 16 * s) = kx[s];
    }
    if (g == 0) {
      R.g[rj] = gl;
      R.beta[rj] = bl;
    }
  }
#pragma unroll
  for (int j = 0; j < 16; ++j) {
    if (j >= cnt && j < n_all && !folds) {  // uniform
      if constexpr (CPL == 2) __builtin_amdgcn_raw_buffer_store_b32(vr[j], rs_vring, 2 * ccol, ring_at(j) * RB, 0);
      else __builtin_amdgcn_raw_buffer_store_b16((uint16_t)vr[j], rs_vring, 2 * ccol, ring_at(j) * RB, 0);
    }
  }
  if (!FUSED && lane == 0 && h == 0) {  // the slot's pointers, once per slot
    R.start[slot] = st;
    R.count[slot] = n_all;
  }

  // ---- K K^T and K Q^T; element r of lane (e, g) is row 4 g + r, column e
  f32x4 kk = {0.f, 0.f, 0.f, 0.f}, kq = kk;
#pragma unroll
  for (int s = 0; s < NS; ++s) qx[s] = e < T ? *reinterpret_cast<const u32x4*>(s_q + e * D + 8 * (NS * g + s)) : z4;
#pragma unroll
  for (int s = 0; s < NS; ++s) {
    if constexpr (IDT == GDN_BF16) {
      kk = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, kx[s]), __builtin_bit_cast(bf16x8, kx[s]),
                                                   kk, 0, 0, 0);
      kq = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, kx[s]), __builtin_bit_cast(bf16x8, qx[s]),
                                                   kq, 0, 0, 0);
    } else {
      kk = __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8, kx[s]), __builtin_bit_cast(f16x8, kx[s]),
                                                  kk, 0, 0, 0);
      kq = __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8, kx[s]), __builtin_bit_cast(f16x8, qx[s]),
                                                  kq, 0, 0, 0);
    }
  }
  // decay weights (every exponent <= 0): F[i][j] = e^{G_i - G_j} k_i . k_j for
  // j < i; kq[j][t] = e^{G_{cnt+t} - G_j} k_j . q_t for j <= cnt + t
  {
    const float Gt = __shfl(G, min(cnt + e, 15), 64);
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int i = 4 * g + r;
      const float Gi = __shfl(G, i, 64);
      if (e < i) s_F[i * (i - 1) / 2 + e] = exp_neg(Gi - G) * kk[r];
      if (e < T) s_kq[i * T + e] = i <= cnt + e ? exp_neg(Gt - Gi) * kq[r] : 0.f;
    }
  }
  // the LDS writes above are read by other lanes below: a wave-level barrier
  // (LDS requests of one wave complete in order; this keeps the compiler's)
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");

  float* wsu = ws + ((int64_t)b * p.Hv + h) * T * 2 * D;
  const float eG = exp_neg(G);
  for (int t = 0; t < T; ++t) {
    // LDS bases made opaque per position: the loop-invariant reads below stay
    // inside the loop instead of holding 32 registers across it
    int zoff = 0;
    asm volatile("" : "+v"(zoff));
    const float* s_Ft = s_F + zoff;
    const uint16_t* s_kt = s_k + zoff;
    // ---- back substitution, rows alike: lane e holds the residual of entry e;
    // c_i = beta_i r_i, then every earlier entry drops its term
    float r = s_kq[e * T + t], c = 0.f;
    {
      float fcol[16];
#pragma unroll
      for (int i = 0; i < 16; ++i) fcol[i] = e < i ? s_Ft[i * (i - 1) / 2 + e] : 0.f;
#pragma unroll
      for (int i = 15; i >= 0; --i) {
        const float ci = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, bl * r), i));
        c = e == i ? ci : c;
        r = fmaf(-fcol[i], ci, r);
      }
    }
    // ---- by columns: acc_t = sum_j c_j v_j and w_t = e^{G_n} q_t - sum_j e^{G_j} c_j k_j
    const float ec = eG * c;
    const float eGn = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, eG), cnt + t));
    float acc[CPL], w[CPL], x[CPL];
    widen(cols_at(s_q + t * D), x);
#pragma unroll
    for (int u = 0; u < CPL; ++u) {
      acc[u] = 0.f;
      w[u] = eGn * x[u];
    }
#pragma unroll
    for (int j = 0; j < 16; ++j) {
      const float cj = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, c), j));
      const float ej = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, ec), j));
      widen(vr[j], x);
#pragma unroll
      for (int u = 0; u < CPL; ++u) acc[u] = fmaf(cj, x[u], acc[u]);
      widen(cols_at(s_kt + j * D), x);
#pragma unroll
      for (int u = 0; u < CPL; ++u) w[u] = fmaf(-ej, x[u], w[u]);
    }
    if constexpr (CPL == 2) {
      *reinterpret_cast<float2*>(wsu + 2 * t * D + ccol) = make_float2(w[0], w[1]);
      *reinterpret_cast<float2*>(wsu + (2 * t + 1) * D + ccol) = make_float2(acc[0], acc[1]);
    } else {
      wsu[2 * t * D + ccol] = w[0];
      wsu[(2 * t + 1) * D + ccol] = acc[0];
    }
  }
}

// ---------------------------------------------------------------- stream
// Fused fold (16-bit inputs): the prep runs first and writes every unit's record
// {slot, start, count before the step, folds}, the fold then folds the flagged
// units and writes their windows' outputs, and the stream kernel streams only
// the tiles of the other units.  The window of a folded unit goes to the ring
// here, after the fold has read the committed entries it overwrites (the prep
// appends the windows of the other units), and the first value head of each
// slot writes the slot's new pointers.
template <int D>
__device__ void replay_fused_tail(const ReplayArgs& P, int b, int h, const int4 rc, int tid, int nth) {
  const DecodeArgs& p = P.d;
  const RingArgs& R = P.ring;
  const int T = P.T, L = R.L, slot = rc.x;
  const bool folded = rc.w != 0;
  const int st = folded ? (rc.y + rc.z) % L : rc.y;  // rc.y < L, rc.z <= L
  if (folded) {
    constexpr int CPR = D / 8;  // 16-byte chunks per 16-bit row
    const int64_t unit = (int64_t)slot * p.Hv + h, krow = ring_key_base(p, slot, h, L);
    const int hk = h / (p.Hv / p.Hk);
    const bool keys = appends_keys(p, h);
    for (int i = tid; i < T * CPR; i += nth) {
      const int t = i / CPR, c = 16 * (i - t * CPR);
      const int pos = st + t >= L ? st + t - L : st + t;  // st < L, t < T <= L
      const u32x4 v = *reinterpret_cast<const u32x4*>(static_cast<const char*>(p.v) +
                                                      (((int64_t)b * T + t) * p.Hv + h) * D * 2 + c);
      *reinterpret_cast<u32x4*>(static_cast<char*>(R.v) + (unit * L + pos) * D * 2 + c) = v;
      if (keys) {
        const u32x4 k = *reinterpret_cast<const u32x4*>(static_cast<const char*>(p.k) +
                                                        (((int64_t)b * T + t) * p.Hk + hk) * D * 2 + c);
        *reinterpret_cast<u32x4*>(static_cast<char*>(R.k) + (krow + pos) * D * 2 + c) = k;
      }
    }
    if (tid < T) {
      const int pos = st + tid >= L ? st + tid - L : st + tid;
      const int64_t gi = ((int64_t)b * T + tid) * p.Hv + h;
      R.g[unit * L + pos] = gate_g(load_elem(p.a, gi, p.in_dt), p.A_log[h], p.dt_bias[h]);
      R.beta[unit * L + pos] = sigmoid_f(load_elem(p.b, gi, p.in_dt));
    }
  }
  if (tid == 0 && h == 0) {  // the slot's pointers, once per slot
    R.start[slot] = st;
    R.count[slot] = folded ? T : rc.z + T;
  }
}

template <int SDT, int D, bool NT, int TB, bool FUSED>
__global__ void __launch_bounds__((ReplayGeom<SDT, D>::NW * 64))
gdn_replay_stream_kernel(const ReplayArgs P, const float* __restrict__ ws) {
  using G = ReplayGeom<SDT, D>;
  constexpr int VEC = G::VEC, LPR = G::LPR, RPW = G::RPW, NW = G::NW, PASSES = G::PASSES;
  constexpr int NTH = NW * 64;
  using IO = TileIO<SDT, VEC, NT>;
  using ST = typename StateElem<SDT>::T;
  extern __shared__ __align__(16) float s_w[];  // [T][D] (read 4 floats at a time)
  __shared__ float s_out[TB][NW][D];

  const DecodeArgs& p = P.d;
  const int T = P.T;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  // 16-bit checkpoints streamed past the Infinity Cache: XCD-aware unit order
  constexpr bool XO = GDN_REPLAY_XCD != 0 && SDT != GDN_F32 && NT;
  const int u = XO ? xcd_unit(blockIdx.x, gridDim.x) : (int)blockIdx.x;
  const int b = u / p.Hv;
  const int h = u - b * p.Hv;
  int slot;
  if constexpr (FUSED) {
    const int4 rc = reinterpret_cast<const int4*>(P.rec)[u];  // the prep's record
    slot = rc.x;
    if (slot >= 0) replay_fused_tail<D>(P, b, h, rc, tid, NTH);
    if (slot >= 0 && rc.w != 0) return;  // folded: the fold wrote the outputs
  } else {
    slot = p.slot_map[b];
  }
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
  const float* wsu = ws + ((int64_t)b * p.Hv + h) * T * 2 * D;
  // The first 4 NTH elements of w and this thread's 4 acc elements of the first
  // TB positions go out before the tile, every thread loading (indices clamped
  // into the unit's rows): loads complete in order, so their waits do not cover
  // the tile, and the acc load is no longer a dependent round after the
  // reduction.
  const int nt0 = T < TB ? T : TB;
  const int iw = min(4 * tid, T * D - 4), ia = min(4 * tid, nt0 * D - 4);
  const f32x4 w0 = *reinterpret_cast<const f32x4*>(wsu + 2 * (iw / D) * D + iw % D);
  const f32x4 a0 = *reinterpret_cast<const f32x4*>(wsu + (2 * (ia / D) + 1) * D + ia % D);
  typename IO::Raw raw[PASSES];
#pragma unroll
  for (int pp = 0; pp < PASSES; ++pp) raw[pp] = IO::load_raw(tile + (r0 + pp * NW * RPW) * D + c0);
  // unconditional (threads past T D / 4 rewrite the last group with the same values),
  // so the compiler cannot sink the w load below the tile's into a branch
  *reinterpret_cast<f32x4*>(s_w + iw) = w0;
  for (int i = 4 * (tid + NTH); i < T * D; i += 4 * NTH) {  // windows past 4 NTH elements
    const int t = i / D, c = i - t * D;
    *reinterpret_cast<f32x4*>(s_w + t * D + c) = *reinterpret_cast<const f32x4*>(wsu + 2 * t * D + c);
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
    const bool out_vec = (reinterpret_cast<uintptr_t>(p.out) & 15) == 0;
    for (int i = 4 * tid; i < nt * D; i += 4 * NTH) {  // 4 outputs per thread, one access each way
      const int tb = i / D, c = i - tb * D;
      const f32x4 acc = (t0 == 0 && i == ia) ? a0 : *reinterpret_cast<const f32x4*>(wsu + (2 * (t0 + tb) + 1) * D + c);
      float o[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        float x = acc[j];
#pragma unroll
        for (int w = 0; w < NW; ++w) x += s_out[tb][w][c + j];
        o[j] = p.scale * x;
      }
      store_vec<4>(p.out, (((int64_t)b * T + t0 + tb) * p.Hv + h) * D + c, o, p.out_dt, out_vec);
    }
    __syncthreads();
  }
}

// Persistent stream for fp32 128 x 128 checkpoints and windows of up to
// kStreamPersistTMax positions (the decode layer's standard step and its
// verify windows).  One workgroup of 16 waves per compute unit
// walks the units u = blockIdx.x + i G with the next unit's tile and w / acc
// rows in flight while the current S0^T w is reduced (the decode kernel's
// persistent layout and two-level column sums; the tile is only read).  Unit
// slots are staged in LDS first; every load is unconditional (padded rows read
// through a zero-size buffer), so the compiler's waits leave the next unit's
// loads outstanding.
constexpr int kStreamPersistNW = 16;
constexpr int kStreamPersistMaxIter = 512;
constexpr int kStreamPersistTMax = 5;  // window positions per unit (LDS: 80 KiB of partials at 5)

// FUSED: units come from the prep's records.  The workgroup's streamed units
// (mapped or padded) are listed from the front of the staging arrays and its
// folded units from the back; a folded unit only appends its window (a wave per
// unit, before the stream), so the stream walks the first list alone.
template <bool NTL, int TMAX, bool FUSED>
__global__ void __launch_bounds__(kStreamPersistNW * 64, 4)
gdn_replay_stream_persist_kernel(const ReplayArgs P, const float* __restrict__ ws) {
  constexpr int D = 128, NW = kStreamPersistNW, VEC = 4, LPR = 32, RPW = 2, PASSES = D / (RPW * NW);
  static_assert(PASSES == 4, "four rows per lane");
  static_assert(TMAX * D <= 4 * NW * 64, "four w / acc elements per thread");
  typedef unsigned int Raw __attribute__((ext_vector_type(4)));
  __shared__ __attribute__((aligned(16))) float s_red[2][TMAX][NW][D];  // [parity][position][wave][column]
  __shared__ __attribute__((aligned(16))) float s_w[2][TMAX][D];        // [parity][position][row]: w
  __shared__ int s_slot[kStreamPersistMaxIter];
  __shared__ int s_unit[FUSED ? kStreamPersistMaxIter : 1];  // FUSED: the units of both lists
  __shared__ int s_n[2];                                     // FUSED: streamed and folded units

  const DecodeArgs& p = P.d;
  const int T = P.T;  // 1 <= T <= TMAX (launcher)
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int c0 = (lane % LPR) * VEC, r0 = wave * RPW + lane / LPR;
  const int units = p.B * p.Hv, G = gridDim.x;
  const int t0 = blockIdx.x;
  if (t0 >= units) return;
  const int n_iter = (units - t0 + G - 1) / G;  // <= kStreamPersistMaxIter (launcher)
  if constexpr (FUSED) {
    if (tid < 2) s_n[tid] = 0;
    __syncthreads();
    for (int i = tid; i < n_iter; i += NW * 64) {
      const int u = t0 + i * G;
      const int4 rc = reinterpret_cast<const int4*>(P.rec)[u];
      if (rc.x >= 0 && rc.w != 0) {
        const int k = n_iter - 1 - atomicAdd(&s_n[1], 1);
        s_unit[k] = u;
      } else {
        const int k = atomicAdd(&s_n[0], 1);
        s_unit[k] = u;
        s_slot[k] = rc.x;
        if (rc.x >= 0 && u % p.Hv == 0) {  // the slot's pointers, once per slot
          P.ring.start[rc.x] = rc.y;
          P.ring.count[rc.x] = rc.z + T;
        }
      }
    }
  } else {
    for (int i = tid; i < n_iter; i += NW * 64) s_slot[i] = p.slot_map[(t0 + i * G) / p.Hv];
  }

  auto valid = [&](int slot) { return slot >= 0 && (int64_t)slot < p.num_slots; };
  // thread tid < T D / 4 carries elements 4 tid.. of the unit's w vectors (w_t by
  // position), one access; thread tid < T D sums column sc of position st and
  // writes that output, with its acc element in a register
  const bool wthr = tid < T * D / 4;
  const int wi = wthr ? 4 * tid : 0, wt = wi / D, wc = wi - wt * D;
  const bool sthr = tid < T * D;
  const int si = sthr ? tid : 0, st = si / D, sc = si - st * D;
  struct In {
    Raw raw[PASSES];
    f32x4 w;
    float acc;
  };
  auto fetch = [&](int u, int slot, In& x) {
    const float* wsu = ws + (int64_t)u * T * 2 * D;  // per position: w, then acc
    x.w = *reinterpret_cast<const f32x4*>(wsu + 2 * wt * D + wc);  // before the tile: waiting for these leaves the tile in flight
    x.acc = wsu[(2 * st + 1) * D + sc];
    const int h = u % p.Hv;
    const bool ok = valid(slot);
    const float* tile = static_cast<const float*>(p.pool) + (ok ? ((int64_t)slot * p.Hv + h) * (int64_t)(D * D) : 0);
    const __amdgpu_buffer_rsrc_t rs =
        __builtin_amdgcn_make_buffer_rsrc(const_cast<float*>(tile), 0, ok ? D * D * 4 : 0, 0x00020000);
#pragma unroll
    for (int pp = 0; pp < PASSES; ++pp)
      x.raw[pp] = __builtin_bit_cast(
          Raw, __builtin_amdgcn_raw_buffer_load_b128(rs, (r0 * D + c0) * 4, pp * NW * RPW * D * 4, NTL ? 2 : 0));
  };

  // One barrier per unit: the partial column sums of unit i (buffer i mod 2) are
  // written before its barrier and summed after it; the next write to that buffer
  // is unit i + 2's, after the barrier of unit i + 1, which every thread reaches
  // only when its sums of unit i are done.  w of unit i + 1 is written before the
  // barrier of unit i and read before the barrier of unit i + 1, so two buffers
  // serve it too.  acc never passes through LDS.
  In cur, nxt;
  __syncthreads();  // s_slot, s_unit, s_n
  int n_run = n_iter;  // units streamed
  if constexpr (FUSED) {
    n_run = s_n[0];
    // the folded units' windows (and their slots' pointers), a unit per wave
    for (int k = wave; k < s_n[1]; k += NW) {
      const int u = __builtin_amdgcn_readfirstlane(s_unit[n_iter - 1 - k]), h = u % p.Hv;
      replay_fused_tail<D>(P, u / p.Hv, h, reinterpret_cast<const int4*>(P.rec)[u], lane, 64);
    }
    if (n_run == 0) return;  // uniform
  }
  auto unit_at = [&](int i) {
    if constexpr (FUSED) return s_unit[i];
    else return t0 + i * G;
  };
  fetch(unit_at(0), s_slot[0], cur);
  if (wthr) *reinterpret_cast<f32x4*>(&s_w[0][wt][wc]) = cur.w;
  __syncthreads();
  for (int it = 0, par = 0; it < n_run; ++it, par ^= 1) {
    const int t = unit_at(it);
    const bool more = it + 1 < n_run;
    // past the last unit the loads repeat this unit's, with no tile
    fetch(more ? unit_at(it + 1) : t, more ? s_slot[it + 1] : -1, nxt);
    const int b = t / p.Hv, h = t - b * p.Hv;
    auto out_row = [&](int tt) { return (((int64_t)b * T + tt) * p.Hv + h) * D; };
    const int sl = s_slot[it];
    const bool live = valid(sl);  // uniform over the workgroup
    if (live) {
#pragma unroll
      for (int tt = 0; tt < TMAX; ++tt) {
        if (tt < T) {
          float part[VEC];
#pragma unroll
          for (int e = 0; e < VEC; ++e) part[e] = 0.f;
#pragma unroll
          for (int pp = 0; pp < PASSES; ++pp) {
            const float wr = s_w[par][tt][r0 + pp * NW * RPW];
#pragma unroll
            for (int e = 0; e < VEC; ++e) part[e] = fmaf(__uint_as_float(cur.raw[pp][e]), wr, part[e]);
          }
#pragma unroll
          for (int e = 0; e < VEC; ++e) part[e] = xor_sum_from<LPR>(part[e]);
          if (lane < LPR)
            *reinterpret_cast<f32x4*>(&s_red[par][tt][wave][c0]) = f32x4{part[0], part[1], part[2], part[3]};
        }
      }
    }
    if (wthr) *reinterpret_cast<f32x4*>(&s_w[par ^ 1][wt][wc]) = nxt.w;  // the next unit's w
    __syncthreads();
    if (sthr) {  // position st, column sc (padded rows: zeros)
      float a = 0.f;
#pragma unroll
      for (int w = 0; w < NW; ++w) a += s_red[par][st][w][sc];
      store_elem(p.out, out_row(st) + sc, live ? p.scale * (cur.acc + a) : 0.f, p.out_dt);
    }
    cur = nxt;
  }
}

// ---------------------------------------------------------------- rollback
__global__ void gdn_replay_rollback_kernel(const ReplayArgs P) {
  const int b = blockIdx.x * blockDim.x + threadIdx.x;
  const DecodeArgs& p = P.d;
  if (b >= p.B) return;
  const int slot = p.slot_map[b];
  if (slot < 0 || (int64_t)slot >= p.num_slots) return;
  int r = P.num_rejected[b];
  r = r < 0 ? 0 : r;
  int32_t* cnt = P.ring.count + slot;
  const int c = *cnt - r;
  *cnt = c < 0 ? 0 : c;
}

// After a flush's fold: every mapped slot's ring is empty, its start moved past
// the folded entries (one thread per row).
__global__ void gdn_replay_advance_kernel(const ReplayArgs P) {
  const int b = blockIdx.x * blockDim.x + threadIdx.x;
  const DecodeArgs& p = P.d;
  if (b >= p.B) return;
  const int slot = p.slot_map[b];
  if (slot < 0 || (int64_t)slot >= p.num_slots) return;
  const RingPos rp = ring_pos(P.ring, slot);
  P.ring.start[slot] = (rp.st + rp.cnt) % P.ring.L;
  P.ring.count[slot] = 0;
}

// ---------------------------------------------------------------- launchers
template <int SDT, int D, int EB, int CDT, bool FUSED = false>
static hipError_t launch_fold(const ReplayArgs& a, hipStream_t s) {
  constexpr int kFusedTW = 4;  // windows of up to 4 positions use the smaller prefetch
  using G = FoldGeom<SDT, D>;
  constexpr bool NT = (SDT == GDN_F32) && (GDN_REPLAY_NT_F32 != 0);
  void (*kern)(const ReplayArgs);
  int threads;
  size_t lds = replay_fold_lds_bytes(D, a.ring.L);
  if constexpr (FUSED) {  // the caller checked L <= 16
    static_assert((D == 64 || D == 128) && CDT < 0 && EB == 2, "fused fold: 16-bit inputs, MFMA fold");
    kern = a.T <= kFusedTW ? &gdn_replay_fold_mfma_kernel<SDT, D, NT, EB, CDT, kFusedTW>
                           : &gdn_replay_fold_mfma_kernel<SDT, D, NT, EB, CDT, 16>;
    threads = 256;
    lds = replay_fold_mfma_lds_bytes(D, a.T <= kFusedTW ? kFusedTW : 16);
  } else if constexpr ((D == 64 || D == 128) && CDT < 0) {  // the dual-precision fold measured faster on the VALU
    if (a.ring.L <= 16) {
      kern = &gdn_replay_fold_mfma_kernel<SDT, D, NT, EB, CDT>;
      threads = 256;
      lds = replay_fold_mfma_lds_bytes(D);
    } else {
      kern = &gdn_replay_fold_kernel<SDT, D, NT, EB, CDT>;
      threads = kFoldColThreads;
    }
  } else if constexpr (D >= 32) {
    kern = &gdn_replay_fold_kernel<SDT, D, NT, EB, CDT>;
    threads = kFoldColThreads;
  } else {
    kern = &gdn_replay_fold_rows_kernel<SDT, D, NT, EB, CDT>;
    threads = G::NW * 64;
  }
  int per_cu = 0, cus = 0;
  hipError_t e = resident_blocks(reinterpret_cast<const void*>(kern), threads, lds, &per_cu);
  if (e == hipSuccess) e = device_cus(&cus);
  if (e != hipSuccess) return e;
  const int64_t units = (int64_t)a.d.B * a.d.Hv;
  const int64_t fill = (int64_t)(per_cu > 0 ? per_cu : 1) * cus;
  const unsigned grid = (unsigned)(units < fill ? units : fill);
  hipLaunchKernelGGL(kern, dim3(grid), dim3(threads), lds, s, a);
  return hipGetLastError();
}

template <int SDT, int D, int EB>
static hipError_t launch_fold_any(const ReplayArgs& a, hipStream_t s) {
  if constexpr (SDT == GDN_F32) {
    if (a.read_pool != nullptr)
      return a.read_dt == GDN_BF16 ? launch_fold<SDT, D, EB, GDN_BF16>(a, s) : launch_fold<SDT, D, EB, GDN_F16>(a, s);
  }
  return launch_fold<SDT, D, EB, -1>(a, s);
}

template <int SDT, int D, bool NT, int TB, bool FUSED>
static void launch_stream(const ReplayArgs& a, unsigned grid, size_t lds, float* ws, hipStream_t s) {
  using G = ReplayGeom<SDT, D>;
  hipLaunchKernelGGL((gdn_replay_stream_kernel<SDT, D, NT, TB, FUSED>), dim3(grid), dim3(G::NW * 64), lds, s, a, ws);
}

// Outputs read the checkpoint itself, or its 16-bit read copy (dual precision).
template <int D, bool FUSED>
static hipError_t launch_stream_any(const ReplayArgs& a, int read_dt, float* ws, hipStream_t s) {
  const unsigned grid = (unsigned)((int64_t)a.d.B * a.d.Hv);
  const size_t lds = (size_t)a.T * D * sizeof(float);
  const bool one = a.T <= 1;
  const bool nt16 = stream_tile_reads((long long)grid * D * D * 2);  // 16-bit checkpoints read once per call
  if constexpr (D == 128) {
    if (read_dt == GDN_F32 && a.T >= 1 && a.T <= kStreamPersistTMax && GDN_REPLAY_STREAM_PERSIST != 0) {
      constexpr bool NTL = GDN_REPLAY_NT_F32 != 0;
      void (*kern)(const ReplayArgs, const float*) = a.T == 1
                                                         ? &gdn_replay_stream_persist_kernel<NTL, 1, FUSED>
                                                         : &gdn_replay_stream_persist_kernel<NTL, kStreamPersistTMax, FUSED>;
      int per_cu = 0, cus = 0;
      hipError_t e = resident_blocks(reinterpret_cast<const void*>(kern), kStreamPersistNW * 64, 0, &per_cu);
      // one workgroup per CU even where two fit (T = 1: 164 against 168 us per call)
      per_cu = per_cu > 1 ? 1 : per_cu;
      if (e == hipSuccess) e = device_cus(&cus);
      if (e != hipSuccess) return e;
      const int64_t fill = (int64_t)(per_cu > 0 ? per_cu : 1) * cus;
      const unsigned pgrid = (unsigned)((int64_t)grid < fill ? (int64_t)grid : fill);
      if ((int64_t)grid > 8 * (int64_t)pgrid && (int64_t)grid <= (int64_t)pgrid * kStreamPersistMaxIter) {
        hipLaunchKernelGGL(kern, dim3(pgrid), dim3(kStreamPersistNW * 64), 0, s, a, static_cast<const float*>(ws));
        return hipGetLastError();
      }
    }
  }
  switch (read_dt) {
    case GDN_F32:
      one ? launch_stream<GDN_F32, D, GDN_REPLAY_NT_F32 != 0, 1, FUSED>(a, grid, lds, ws, s)
          : launch_stream<GDN_F32, D, GDN_REPLAY_NT_F32 != 0, kStreamTB, FUSED>(a, grid, lds, ws, s);
      break;
    case GDN_BF16:
      if (nt16)
        one ? launch_stream<GDN_BF16, D, true, 1, FUSED>(a, grid, lds, ws, s)
            : launch_stream<GDN_BF16, D, true, kStreamTB, FUSED>(a, grid, lds, ws, s);
      else
        one ? launch_stream<GDN_BF16, D, false, 1, FUSED>(a, grid, lds, ws, s)
            : launch_stream<GDN_BF16, D, false, kStreamTB, FUSED>(a, grid, lds, ws, s);
      break;
    case GDN_F16:
      if (nt16)
        one ? launch_stream<GDN_F16, D, true, 1, FUSED>(a, grid, lds, ws, s)
            : launch_stream<GDN_F16, D, true, kStreamTB, FUSED>(a, grid, lds, ws, s);
      else
        one ? launch_stream<GDN_F16, D, false, 1, FUSED>(a, grid, lds, ws, s)
            : launch_stream<GDN_F16, D, false, kStreamTB, FUSED>(a, grid, lds, ws, s);
      break;
    default:
      return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

template <int SDT, int D>
static hipError_t launch_replay_t(const ReplayArgs& a0, float* ws, hipStream_t s) {
  const bool f32_in = a0.d.in_dt == GDN_F32;
  ReplayArgs a = a0;
  a.rec = nullptr;
  if (a.T > 0)  // the preps read the unit records the fold's check writes
    a.rec = reinterpret_cast<int32_t*>(reinterpret_cast<char*>(ws) + replay_vectors_bytes(a.d.B, a.d.Hv, a.T, D));
  const unsigned grid = (unsigned)((int64_t)a.d.B * a.d.Hv);
  // fused fold: prep, fold, stream (16-bit 128 x 128 tiles stay apart: the fold's
  // outputs pushed those kernels past their registers)
  if constexpr (D == 64 || (D == 128 && SDT == GDN_F32)) {
    if (a.T > 0 && !f32_in && a.ring.L <= 16 && a.read_pool == nullptr) {
      const size_t lds = replay_prep16_lds_bytes(D, a.T);
      if (a.d.in_dt == GDN_BF16)
        hipLaunchKernelGGL((gdn_replay_prep16_kernel<D, GDN_BF16, true>), dim3(grid), dim3(64), lds, s, a, ws);
      else
        hipLaunchKernelGGL((gdn_replay_prep16_kernel<D, GDN_F16, true>), dim3(grid), dim3(64), lds, s, a, ws);
      hipError_t e = hipGetLastError();
      if (e == hipSuccess) e = launch_fold<SDT, D, 2, -1, true>(a, s);
      if (e != hipSuccess) return e;
      return launch_stream_any<D, true>(a, SDT, ws, s);
    }
  }
  hipError_t e = f32_in ? launch_fold_any<SDT, D, 4>(a, s) : launch_fold_any<SDT, D, 2>(a, s);
  if (e != hipSuccess) return e;
  if (a.T == 0) {  // flush: the slots' pointers move once every head has folded
    hipLaunchKernelGGL(gdn_replay_advance_kernel, dim3((unsigned)((a.d.B + 255) / 256)), dim3(256), 0, s, a);
    return hipGetLastError();
  }
  constexpr int NWP = GDN_REPLAY_PREP_WAVES;
  if constexpr (D == 64 || D == 128) {
    if (!f32_in && a.ring.L <= 16) {
      const size_t lds = replay_prep16_lds_bytes(D, a.T);
      if (a.d.in_dt == GDN_BF16)
        hipLaunchKernelGGL((gdn_replay_prep16_kernel<D, GDN_BF16, false>), dim3(grid), dim3(64), lds, s, a, ws);
      else
        hipLaunchKernelGGL((gdn_replay_prep16_kernel<D, GDN_F16, false>), dim3(grid), dim3(64), lds, s, a, ws);
      goto prep_done;
    }
  }
  if (f32_in)
    hipLaunchKernelGGL((gdn_replay_prep_kernel<D, 4, NWP>), dim3(grid), dim3(NWP * 64),
                       replay_prep_words(D, 4, a.ring.L, a.T) * sizeof(float), s, a, ws);
  else
    hipLaunchKernelGGL((gdn_replay_prep_kernel<D, 2, NWP>), dim3(grid), dim3(NWP * 64),
                       replay_prep_words(D, 2, a.ring.L, a.T) * sizeof(float), s, a, ws);
prep_done:
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  if (a.read_pool == nullptr) return launch_stream_any<D, false>(a, SDT, ws, s);
  ReplayArgs r = a;
  r.d.pool = a.read_pool;
  return launch_stream_any<D, false>(r, a.read_dt, ws, s);
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
  const unsigned grid = (unsigned)((a.d.B + 255) / 256);
  hipLaunchKernelGGL(gdn_replay_rollback_kernel, dim3(grid), dim3(256), 0, s, a);
  return hipGetLastError();
}

size_t replay_lds_total(int D, int L, int T) {
  const size_t prep = T > 0 ? replay_prep_lds_bytes(D, L, T) : 0;
  const size_t fold = replay_fold_lds_bytes(D, L) + 2 * 8 * (size_t)D * sizeof(float);
  return prep > fold ? prep : fold;
}

}  // namespace gdn
