// Internal launch interface between the C ABI (gdn_api.cpp) and the kernels.
// Arguments here are already validated by the ABI layer.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "gdn.h"

namespace gdn {

struct DecodeArgs {
  const void* q;
  const void* k;
  const void* v;
  const void* a;
  const void* b;
  const float* A_log;
  const float* dt_bias;
  void* pool;
  const int32_t* slot_map;
  void* out;
  int64_t num_slots;
  int32_t B, Hk, Hv;
  int32_t in_dt, out_dt;
  float scale;
};

struct RingArgs {
  void* k;
  void* v;
  float* g;
  float* beta;
  int32_t* start;
  int32_t* count;
  int32_t L;
};

struct ReplayArgs {
  DecodeArgs d;  // q, k, v, a, b laid out [B, T, H, d]; pool is the checkpoint pool
  RingArgs ring;
  int32_t T;     // 1..L; 0 selects the flush-only kernel
  const int32_t* num_rejected;
  void* read_pool;  // dual-precision mode: the 16-bit read copy of the fp32 checkpoint (else null)
  int32_t read_dt;
  int32_t* rec;     // [B * Hv][4] unit records (slot or -1, start and count after any fold), written by
                    // the fold's check for the one-wave prep; null when that prep is not used
};

struct SpecArgs {
  DecodeArgs d;  // q, k, v, a, b laid out [B, T, H, d]; slot_map holds the source slots
  const int32_t* dst_slots;  // [B, T]
  int32_t T;
};

struct CopyArgs {
  const gdn_state_ref* refs;  // [P], device
  const int32_t* src;         // [n], device
  const int32_t* dst;         // [n], device
  int32_t P, n;
};
constexpr int kCopyThreads = 256;
constexpr uint64_t kCopyChunk = 64 * 1024;  // bytes of a slot per workgroup

struct M2Args {
  const void* x;      // [B, T, H, P] (decode: T = 1)
  const void* Bm;     // [B, T, G, N]
  const void* Cm;     // [B, T, G, N]
  const void* dt;     // [B, T, H]
  const float* A_log;
  const float* dt_bias;
  const float* Dskip;
  void* pool;         // [num_slots, H, P, N]
  const int32_t* slot_map;
  void* y;            // [B, T, H, P]
  int64_t num_slots;
  int32_t B, H, G, in_dt, out_dt;
  int32_t T, L;       // replay window and ring length
  void* rx;           // ring x [num_slots, H, L, P]
  void* rB;           // ring B [num_slots, G, L, N]
  float* rg;          // ring g [num_slots, H, L]
  float* rdtp;        // ring dt' [num_slots, H, L]
  int32_t* start;     // [num_slots]
  int32_t* count;     // [num_slots]
  const int32_t* num_rejected;
};

struct PrefillArgs {
  const void* q;
  const void* k;
  const void* v;
  const void* a;
  const void* b;
  const float* A_log;
  const float* dt_bias;
  void* pool;
  const int32_t* slot_map;
  const int32_t* cu_seqlens;
  void* out;
  int64_t num_slots;
  int64_t total_tokens;
  int32_t N, Hk, Hv;
  int32_t in_dt, out_dt;
  float scale;
};

// Each returns hipSuccess or the launch error.
hipError_t launch_decode(const DecodeArgs& a, int state_dt, int D, hipStream_t s);
// state_dt: dtype of the checkpoint pool a.d.pool; with a.read_pool set the
// checkpoint is the fp32 master and outputs read the read_dt copy.
hipError_t launch_replay(const ReplayArgs& a, int state_dt, int D, float* ws, hipStream_t s);
hipError_t launch_replay_flush(const ReplayArgs& a, int state_dt, int D, hipStream_t s);
hipError_t launch_replay_rollback(const ReplayArgs& a, hipStream_t s);
hipError_t launch_prefill(const PrefillArgs& a, int state_dt, int D, int chunk, float* ws, hipStream_t s);
hipError_t launch_spec(const SpecArgs& a, int state_dt, int D, hipStream_t s);
hipError_t launch_copy_blocks(const CopyArgs& a, uint64_t max_slot_bytes, hipStream_t s);
hipError_t launch_m2_decode(const M2Args& a, int state_dt, int P, int N, hipStream_t s);
// fold, step (T > 0) and pointer advance; T == 0 is the flush
hipError_t launch_m2_replay(const M2Args& a, int state_dt, int P, int N, hipStream_t s);
hipError_t launch_m2_rollback(const M2Args& a, hipStream_t s);
size_t m2_lds_bytes(int P, int N, int L, int T, int heads_per_group);

// Dynamic LDS of the speculative-decode kernel; launches need <= kSpecMaxLds.
size_t spec_lds_bytes(int D, int T);
constexpr size_t kSpecMaxLds = 49152;

// Compute units of the current device (cached per device).
hipError_t device_cus(int* cus);
// Workgroups of `kernel` resident on one compute unit at this block size and
// dynamic LDS (cached per device, kernel, block and LDS size).
hipError_t resident_blocks(const void* kernel, int block, size_t lds, int* per_cu);

// Largest LDS footprint of the replay kernels for this shape; launches need <= 64 KiB.
size_t replay_lds_total(int D, int L, int T);
constexpr size_t kMaxLds = 65536;

// Workspace of gdn_replay_decode: w_t and acc_t (dv floats each) per
// (sequence, value head, window position).
size_t replay_workspace_bytes(int64_t B, int Hv, int T, int D);

// Fixed device scratch that gdn_replay_decode_noalloc uses in place of a caller
// workspace: one array per GPU the library runs on, kept until the process
// ends.  kReplayScratchBytes holds the workspace of 512 rows x 32 value heads
// x 5-token windows at head dim 128 (81.25 MiB).  replay_scratch() returns its
// device address on the current device, looked up once per device.
constexpr size_t kReplayScratchBytes = (size_t)96 << 20;
hipError_t replay_scratch(void** ptr);

// Workspace of the chunked prefill for chunks of C tokens: per (chunk slot,
// value head) the inverse T, the causal decay-weighted Q K^T, gamma and beta
// of one chunk.
size_t prefill_workspace_bytes(int N, int64_t total, int Hv, int C);
bool prefill_chunk_slots_fit(int N, int64_t total, int Hk, int Hv, int C);

}  // namespace gdn
