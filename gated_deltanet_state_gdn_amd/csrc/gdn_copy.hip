// State-block copy for prefix caching: for every (source slot, destination
// slot) job and every state tensor named by a device table, copy the source
// slot's bytes over the destination slot's (vLLM PR #48109 page, the XPU
// state-pointer fix: its implementation section describes the state-copy
// kernel behind --mamba-cache-mode align, fed by a table of state base
// addresses; its risk section notes that those addresses must keep all 64
// bits, so this table holds them as unsigned 64-bit values and the kernel
// only adds offsets to them).
//
// Grid: x = chunk of the slot (kCopyChunk bytes), y = state tensor, z = job.
// A chunk is moved with 16-byte vector accesses when the addresses and the
// length allow it, else 4-byte or single-byte ones.
#include "gdn_device.h"
#include "gdn_launch.h"

namespace gdn {

template <typename V>
__device__ __forceinline__ void copy_span(const char* __restrict__ s, char* __restrict__ d, uint64_t n) {
  const V* sv = reinterpret_cast<const V*>(s);
  V* dv = reinterpret_cast<V*>(d);
  const uint64_t cnt = n / sizeof(V);
  constexpr int U = 4;  // loads in flight per thread
  uint64_t i = threadIdx.x;
  for (; i + (U - 1) * kCopyThreads < cnt; i += U * kCopyThreads) {
    V x[U];
#pragma unroll
    for (int u = 0; u < U; ++u) x[u] = __builtin_nontemporal_load(sv + i + u * kCopyThreads);
#pragma unroll
    for (int u = 0; u < U; ++u) __builtin_nontemporal_store(x[u], dv + i + u * kCopyThreads);
  }
  for (; i < cnt; i += kCopyThreads) dv[i] = sv[i];
}

__global__ void __launch_bounds__(kCopyThreads) gdn_copy_blocks_kernel(const CopyArgs a) {
  const gdn_state_ref r = a.refs[blockIdx.y];
  const int job = blockIdx.z;
  const int s = a.src[job], d = a.dst[job];
  if (s < 0 || d < 0 || (uint64_t)s >= r.num_slots || (uint64_t)d >= r.num_slots) return;
  const uint64_t off = (uint64_t)blockIdx.x * kCopyChunk;
  if (off >= r.slot_bytes) return;
  const uint64_t n = r.slot_bytes - off < kCopyChunk ? r.slot_bytes - off : kCopyChunk;
  // unsigned 64-bit address arithmetic: no bit of the base is lost
  const char* sp = reinterpret_cast<const char*>(r.base + (uint64_t)s * r.slot_bytes + off);
  char* dp = reinterpret_cast<char*>(r.base + (uint64_t)d * r.slot_bytes + off);
  const uint64_t mis = reinterpret_cast<uint64_t>(sp) | reinterpret_cast<uint64_t>(dp) | n;
  if ((mis & 15) == 0)
    copy_span<u32x4>(sp, dp, n);
  else if ((mis & 3) == 0)
    copy_span<uint32_t>(sp, dp, n);
  else
    copy_span<unsigned char>(sp, dp, n);
}

hipError_t launch_copy_blocks(const CopyArgs& a, uint64_t max_slot_bytes, hipStream_t s) {
  if (a.n == 0 || a.P == 0) return hipSuccess;
  const uint64_t chunks = (max_slot_bytes + kCopyChunk - 1) / kCopyChunk;
  hipLaunchKernelGGL(gdn_copy_blocks_kernel, dim3((unsigned)chunks, (unsigned)a.P, (unsigned)a.n), dim3(kCopyThreads),
                     0, s, a);
  return hipGetLastError();
}

}  // namespace gdn
