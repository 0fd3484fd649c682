// C ABI of the GDN state-update library: argument validation and dispatch.
//
// Every entry point validates synchronously on the host and only then
// enqueues kernels on the caller's stream.  Nothing is allocated and no state
// is kept between calls except the calling thread's last-error text.
#include <hip/hip_runtime.h>

#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <map>
#include <mutex>
#include <tuple>

#include "gdn.h"
#include "gdn_launch.h"

namespace {

thread_local char g_last_error[256] = "";

gdn_status fail(gdn_status st, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_last_error, sizeof(g_last_error), fmt, ap);
  va_end(ap);
  return st;
}

gdn_status ok() {
  g_last_error[0] = '\0';
  return GDN_OK;
}

bool valid_dtype(int dt) { return dt == GDN_F32 || dt == GDN_BF16 || dt == GDN_F16; }
size_t dtype_bytes(int dt) { return dt == GDN_F32 ? 4 : 2; }
bool aligned(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

#define GDN_REQUIRE(cond, st, ...) \
  do {                             \
    if (!(cond)) return fail(st, __VA_ARGS__); \
  } while (0)

#define GDN_TRY(expr)                   \
  do {                                  \
    gdn_status st_ = (expr);            \
    if (st_ != GDN_OK) return st_;      \
  } while (0)

gdn_status check_dims(const gdn_dims* d) {
  GDN_REQUIRE(d != nullptr, GDN_EINVAL, "dims is NULL");
  GDN_REQUIRE(d->num_k_heads >= 1 && d->num_v_heads >= 1, GDN_EINVAL, "head counts must be >= 1 (Hk=%d Hv=%d)",
              d->num_k_heads, d->num_v_heads);
  GDN_REQUIRE(d->num_v_heads % d->num_k_heads == 0, GDN_EINVAL, "Hv=%d is not a multiple of Hk=%d",
              d->num_v_heads, d->num_k_heads);
  GDN_REQUIRE(d->dk >= 1 && d->dv >= 1, GDN_EINVAL, "head dims must be >= 1 (dk=%d dv=%d)", d->dk, d->dv);
  GDN_REQUIRE(d->dk == d->dv && (d->dk == 16 || d->dk == 32 || d->dk == 64 || d->dk == 128), GDN_EUNSUPPORTED,
              "head dims dk=%d dv=%d: compiled for dk == dv in {16, 32, 64, 128}", d->dk, d->dv);
  return GDN_OK;
}

float eff_scale(const gdn_dims* d) { return d->scale > 0.f ? d->scale : 1.0f / sqrtf((float)d->dk); }

gdn_status check_pool(const gdn_pool* p, const char* what) {
  GDN_REQUIRE(p != nullptr, GDN_EINVAL, "%s pool is NULL", what);
  GDN_REQUIRE(p->base != nullptr, GDN_EINVAL, "%s pool base is NULL", what);
  GDN_REQUIRE(valid_dtype(p->dtype), GDN_EINVAL, "%s pool dtype %d is not a gdn_dtype", what, (int)p->dtype);
  GDN_REQUIRE(aligned(p->base, 16), GDN_EINVAL, "%s pool base is not 16-byte aligned", what);
  GDN_REQUIRE(p->num_slots >= 1 && p->num_slots <= INT32_MAX, GDN_EINVAL, "%s pool num_slots=%lld out of range",
              what, (long long)p->num_slots);
  return GDN_OK;
}

gdn_status check_gates(const gdn_gates* g, int in_dt) {
  GDN_REQUIRE(g != nullptr, GDN_EINVAL, "gates is NULL");
  GDN_REQUIRE(g->a && g->b && g->A_log && g->dt_bias, GDN_EINVAL, "a gate pointer is NULL");
  const size_t eb = dtype_bytes(in_dt);
  GDN_REQUIRE(aligned(g->a, eb) && aligned(g->b, eb) && aligned(g->A_log, 4) && aligned(g->dt_bias, 4),
              GDN_EINVAL, "a gate pointer is misaligned for its dtype");
  return GDN_OK;
}

gdn_status check_dtypes(int in_dt, int out_dt) {
  GDN_REQUIRE(valid_dtype(in_dt), GDN_EINVAL, "in_dtype %d is not a gdn_dtype", in_dt);
  GDN_REQUIRE(valid_dtype(out_dt), GDN_EINVAL, "out_dtype %d is not a gdn_dtype", out_dt);
  return GDN_OK;
}

gdn_status check_io(const void* q, const void* k, const void* v, int in_dt, const void* out, int out_dt) {
  GDN_TRY(check_dtypes(in_dt, out_dt));
  GDN_REQUIRE(q && k && v, GDN_EINVAL, "q, k or v is NULL");
  GDN_REQUIRE(out != nullptr, GDN_EINVAL, "out is NULL");
  GDN_REQUIRE(aligned(q, 16) && aligned(k, 16) && aligned(v, 16), GDN_EINVAL, "q, k or v is not 16-byte aligned");
  GDN_REQUIRE(aligned(out, dtype_bytes(out_dt)), GDN_EINVAL, "out misaligned for out_dtype");
  return GDN_OK;
}

gdn_status check_ring(const gdn_ring* r, int in_dt) {
  GDN_REQUIRE(r != nullptr, GDN_EINVAL, "ring is NULL");
  GDN_REQUIRE(r->k && r->v && r->g && r->beta && r->start && r->count, GDN_EINVAL, "a ring pointer is NULL");
  GDN_REQUIRE(r->num_slots >= 1 && r->num_slots <= INT32_MAX, GDN_EINVAL, "ring num_slots=%lld out of range",
              (long long)r->num_slots);
  GDN_REQUIRE(r->L >= 1, GDN_EINVAL, "ring length L=%d must be >= 1", r->L);
  GDN_REQUIRE(r->L <= 64, GDN_EUNSUPPORTED, "ring length L=%d: at most 64 is supported", r->L);
  GDN_REQUIRE(valid_dtype(r->dtype), GDN_EINVAL, "ring dtype %d is not a gdn_dtype", (int)r->dtype);
  if (in_dt >= 0)
    GDN_REQUIRE((int)r->dtype == in_dt, GDN_EINVAL, "ring dtype %d differs from in_dtype %d", (int)r->dtype, in_dt);
  GDN_REQUIRE(aligned(r->k, 16) && aligned(r->v, 16) && aligned(r->g, 4) && aligned(r->beta, 4) &&
                  aligned(r->start, 4) && aligned(r->count, 4),
              GDN_EINVAL, "a ring pointer is misaligned");
  return GDN_OK;
}

gdn_status launched(hipError_t e) {
  if (e != hipSuccess) return fail(GDN_ELAUNCH, "kernel launch failed: %s", hipGetErrorString(e));
  return ok();
}

gdn::RingArgs ring_args(const gdn_ring* r) {
  return gdn::RingArgs{r->k, r->v, r->g, r->beta, r->start, r->count, r->L};
}

}  // namespace

namespace gdn {

hipError_t device_cus(int* cus) {
  static std::mutex mu;
  static std::map<int, int> cache;
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  std::lock_guard<std::mutex> lock(mu);
  auto it = cache.find(dev);
  if (it == cache.end()) {
    int n = 0;
    e = hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev);
    if (e != hipSuccess) return e;
    it = cache.emplace(dev, n > 0 ? n : 1).first;
  }
  *cus = it->second;
  return hipSuccess;
}

hipError_t resident_blocks(const void* kernel, int block, size_t lds, int* per_cu) {
  static std::mutex mu;
  static std::map<std::tuple<int, const void*, int, size_t>, int> cache;
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  const auto key = std::make_tuple(dev, kernel, block, lds);
  std::lock_guard<std::mutex> lock(mu);
  auto it = cache.find(key);
  if (it == cache.end()) {
    int n = 0;
    e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, kernel, block, lds);
    if (e != hipSuccess) return e;
    it = cache.emplace(key, n > 0 ? n : 1).first;
  }
  *per_cu = it->second;
  return hipSuccess;
}

}  // namespace gdn

extern "C" {

const char* gdn_status_string(gdn_status s) {
  switch (s) {
    case GDN_OK: return "GDN_OK: success";
    case GDN_EINVAL: return "GDN_EINVAL: invalid argument";
    case GDN_EUNSUPPORTED: return "GDN_EUNSUPPORTED: request outside the compiled configurations";
    case GDN_ELAUNCH: return "GDN_ELAUNCH: kernel launch failed";
    default: return "unknown gdn_status";
  }
}

const char* gdn_last_error(void) { return g_last_error; }

gdn_status gdn_decode_step(const gdn_dims* dims, int32_t B, const void* q, const void* k, const void* v,
                           gdn_dtype in_dtype, const gdn_gates* gates, const gdn_pool* state,
                           const int32_t* slot_map, void* out, gdn_dtype out_dtype, void* stream) {
  GDN_TRY(check_dims(dims));
  GDN_REQUIRE(B >= 0, GDN_EINVAL, "B=%d must be >= 0", B);
  GDN_REQUIRE((int64_t)B * dims->num_v_heads <= INT32_MAX, GDN_EINVAL, "B * Hv exceeds the grid limit");
  GDN_TRY(check_dtypes(in_dtype, out_dtype));
  if (B == 0) return ok();  // nothing is read or written
  GDN_TRY(check_io(q, k, v, in_dtype, out, out_dtype));
  GDN_TRY(check_gates(gates, in_dtype));
  GDN_TRY(check_pool(state, "state"));
  GDN_REQUIRE(slot_map != nullptr && aligned(slot_map, 4), GDN_EINVAL, "slot_map is NULL or misaligned");
  gdn::DecodeArgs a{q, k, v, gates->a, gates->b, gates->A_log, gates->dt_bias, state->base, slot_map, out,
                    state->num_slots, B, dims->num_k_heads, dims->num_v_heads, (int32_t)in_dtype,
                    (int32_t)out_dtype, eff_scale(dims)};
  return launched(gdn::launch_decode(a, state->dtype, dims->dk, static_cast<hipStream_t>(stream)));
}

gdn_status gdn_spec_decode(const gdn_dims* dims, int32_t B, int32_t T, const void* q, const void* k, const void* v,
                           gdn_dtype in_dtype, const gdn_gates* gates, const gdn_pool* state,
                           const int32_t* src_slots, const int32_t* dst_slots, void* out, gdn_dtype out_dtype,
                           void* stream) {
  GDN_TRY(check_dims(dims));
  GDN_REQUIRE(B >= 0, GDN_EINVAL, "B=%d must be >= 0", B);
  GDN_REQUIRE(T >= 1, GDN_EINVAL, "window T=%d must be >= 1", T);
  GDN_REQUIRE((int64_t)B * dims->num_v_heads <= INT32_MAX, GDN_EINVAL, "B * Hv exceeds the grid limit");
  GDN_REQUIRE((int64_t)B * T * dims->num_v_heads * dims->dv <= INT64_MAX / 8, GDN_EINVAL, "B * T too large");
  GDN_TRY(check_dtypes(in_dtype, out_dtype));
  GDN_REQUIRE(gdn::spec_lds_bytes(dims->dk, T) <= gdn::kSpecMaxLds, GDN_EUNSUPPORTED,
              "window T=%d at dk=%d exceeds the 48 KiB LDS staging budget", T, dims->dk);
  if (B == 0) return ok();  // nothing is read or written
  GDN_TRY(check_io(q, k, v, in_dtype, out, out_dtype));
  GDN_TRY(check_gates(gates, in_dtype));
  GDN_TRY(check_pool(state, "state"));
  GDN_REQUIRE(src_slots != nullptr && aligned(src_slots, 4), GDN_EINVAL, "src_slots is NULL or misaligned");
  GDN_REQUIRE(dst_slots != nullptr && aligned(dst_slots, 4), GDN_EINVAL, "dst_slots is NULL or misaligned");
  gdn::SpecArgs a{};
  a.d = gdn::DecodeArgs{q, k, v, gates->a, gates->b, gates->A_log, gates->dt_bias, state->base, src_slots, out,
                        state->num_slots, B, dims->num_k_heads, dims->num_v_heads, (int32_t)in_dtype,
                        (int32_t)out_dtype, eff_scale(dims)};
  a.dst_slots = dst_slots;
  a.T = T;
  return launched(gdn::launch_spec(a, state->dtype, dims->dk, static_cast<hipStream_t>(stream)));
}

gdn_status gdn_copy_state_blocks(const gdn_state_ref* refs, int32_t P, uint64_t max_slot_bytes,
                                 const int32_t* src_slots, const int32_t* dst_slots, int32_t n, void* stream) {
  GDN_REQUIRE(P >= 0 && P <= 65535, GDN_EINVAL, "P=%d out of [0, 65535]", P);
  GDN_REQUIRE(n >= 0 && n <= 65535, GDN_EINVAL, "n=%d out of [0, 65535]", n);
  if (P == 0 || n == 0) return ok();  // nothing is read or written
  GDN_REQUIRE(refs != nullptr && aligned(refs, 8), GDN_EINVAL, "refs is NULL or not 8-byte aligned");
  GDN_REQUIRE(src_slots != nullptr && aligned(src_slots, 4), GDN_EINVAL, "src_slots is NULL or misaligned");
  GDN_REQUIRE(dst_slots != nullptr && aligned(dst_slots, 4), GDN_EINVAL, "dst_slots is NULL or misaligned");
  GDN_REQUIRE(max_slot_bytes >= 1 && (max_slot_bytes + gdn::kCopyChunk - 1) / gdn::kCopyChunk <= INT32_MAX,
              GDN_EINVAL, "max_slot_bytes=%llu out of [1, 2^31 chunks]", (unsigned long long)max_slot_bytes);
  gdn::CopyArgs a{refs, src_slots, dst_slots, P, n};
  return launched(gdn::launch_copy_blocks(a, max_slot_bytes, static_cast<hipStream_t>(stream)));
}

size_t gdn_chunk_prefill_workspace_bytes(const gdn_dims* dims, int32_t N, int64_t total_tokens, int32_t chunk) {
  if (dims == nullptr || N <= 0 || total_tokens <= 0 || dims->num_v_heads < 1) return 0;
  if (chunk != 16 && chunk != 32 && chunk != 64) return 0;
  return gdn::prefill_workspace_bytes(N, total_tokens, dims->num_v_heads, chunk);
}

gdn_status gdn_chunk_prefill(const gdn_dims* dims, int32_t N, const int32_t* cu_seqlens, int64_t total_tokens,
                             int32_t chunk, const void* q, const void* k, const void* v, gdn_dtype in_dtype,
                             const gdn_gates* gates, const gdn_pool* state, const int32_t* slot_map, void* out,
                             gdn_dtype out_dtype, void* workspace, size_t workspace_bytes, void* stream) {
  GDN_TRY(check_dims(dims));
  GDN_REQUIRE(N >= 0, GDN_EINVAL, "N=%d must be >= 0", N);
  GDN_REQUIRE(total_tokens >= 0 && total_tokens <= INT32_MAX, GDN_EINVAL, "total_tokens=%lld out of [0, 2^31)",
              (long long)total_tokens);
  GDN_REQUIRE(chunk == 16 || chunk == 32 || chunk == 64, GDN_EUNSUPPORTED, "chunk=%d: 16, 32 and 64 are compiled",
              chunk);
  GDN_REQUIRE((int64_t)N * dims->num_v_heads <= INT32_MAX / 4, GDN_EINVAL, "N * Hv exceeds the grid limit");
  GDN_TRY(check_dtypes(in_dtype, out_dtype));
  if (N == 0 || total_tokens == 0) return ok();  // nothing is read or written
  GDN_TRY(check_io(q, k, v, in_dtype, out, out_dtype));
  GDN_TRY(check_gates(gates, in_dtype));
  GDN_TRY(check_pool(state, "state"));
  GDN_REQUIRE(cu_seqlens != nullptr && aligned(cu_seqlens, 4), GDN_EINVAL, "cu_seqlens is NULL or misaligned");
  GDN_REQUIRE(slot_map != nullptr && aligned(slot_map, 4), GDN_EINVAL, "slot_map is NULL or misaligned");
  const size_t need = gdn_chunk_prefill_workspace_bytes(dims, N, total_tokens, chunk);
  GDN_REQUIRE(workspace_bytes >= need, GDN_EINVAL, "workspace of %zu bytes is below the %zu required",
              workspace_bytes, need);
  GDN_REQUIRE(need == 0 || (workspace != nullptr && aligned(workspace, 256)), GDN_EINVAL,
              "workspace is NULL or not 256-byte aligned");
  GDN_REQUIRE(gdn::prefill_chunk_slots_fit(N, total_tokens, dims->num_k_heads, dims->num_v_heads, chunk), GDN_EINVAL,
              "N + total_tokens / chunk chunk slots exceed the grid limit");
  gdn::PrefillArgs a{q, k, v, gates->a, gates->b, gates->A_log, gates->dt_bias, state->base, slot_map, cu_seqlens,
                     out, state->num_slots, total_tokens, N, dims->num_k_heads, dims->num_v_heads,
                     (int32_t)in_dtype, (int32_t)out_dtype, eff_scale(dims)};
  return launched(gdn::launch_prefill(a, state->dtype, dims->dk, chunk, static_cast<float*>(workspace),
                                      static_cast<hipStream_t>(stream)));
}

size_t gdn_replay_workspace_bytes(const gdn_dims* dims, int32_t B, int32_t T) {
  if (dims == nullptr || B <= 0 || T <= 0 || dims->num_v_heads < 1 || dims->dv < 1) return 0;
  return gdn::replay_workspace_bytes(B, dims->num_v_heads, T, dims->dv);
}

namespace {

// A dual-precision checkpoint: an fp32 master plus a 16-bit read copy of the same slots.
gdn_status check_dual(const gdn_pool* master, const gdn_pool* copy) {
  GDN_REQUIRE(master->dtype == GDN_F32, GDN_EINVAL, "the dual-precision master checkpoint must be f32");
  GDN_TRY(check_pool(copy, "read copy"));
  GDN_REQUIRE(copy->dtype == GDN_BF16 || copy->dtype == GDN_F16, GDN_EINVAL, "the read copy must be bf16 or f16");
  GDN_REQUIRE(copy->num_slots == master->num_slots, GDN_EINVAL, "read copy holds %lld slots, the master %lld",
              (long long)copy->num_slots, (long long)master->num_slots);
  GDN_REQUIRE(copy->base != master->base, GDN_EINVAL, "the read copy aliases the master");
  return ok();
}

gdn_status replay_decode_impl(const gdn_dims* dims, int32_t B, int32_t T, const void* q, const void* k,
                              const void* v, gdn_dtype in_dtype, const gdn_gates* gates, const gdn_pool* ckpt,
                              const gdn_pool* read_copy, const int32_t* slot_map, const gdn_ring* ring, void* out,
                              gdn_dtype out_dtype, void* workspace, size_t workspace_bytes, void* stream) {
  GDN_TRY(check_dims(dims));
  GDN_REQUIRE(B >= 0, GDN_EINVAL, "B=%d must be >= 0", B);
  GDN_REQUIRE((int64_t)B * dims->num_v_heads <= INT32_MAX, GDN_EINVAL, "B * Hv exceeds the grid limit");
  GDN_TRY(check_dtypes(in_dtype, out_dtype));
  GDN_REQUIRE(ring != nullptr, GDN_EINVAL, "ring is NULL");
  GDN_REQUIRE(T >= 1 && T <= ring->L, GDN_EINVAL, "window T=%d must satisfy 1 <= T <= L=%d", T, ring->L);
  if (B == 0) return ok();  // nothing is read or written
  GDN_TRY(check_io(q, k, v, in_dtype, out, out_dtype));
  GDN_TRY(check_gates(gates, in_dtype));
  GDN_TRY(check_pool(ckpt, "checkpoint"));
  if (read_copy != nullptr) GDN_TRY(check_dual(ckpt, read_copy));
  GDN_TRY(check_ring(ring, in_dtype));
  GDN_REQUIRE(ring->num_slots == ckpt->num_slots, GDN_EINVAL, "ring holds %lld slots, the checkpoint pool %lld",
              (long long)ring->num_slots, (long long)ckpt->num_slots);
  GDN_REQUIRE(gdn::replay_lds_total(dims->dk, ring->L, T) <= gdn::kMaxLds, GDN_EUNSUPPORTED,
              "ring length L=%d with window T=%d at dk=%d exceeds the 64 KiB LDS staging budget", ring->L, T,
              dims->dk);
  const size_t need = gdn_replay_workspace_bytes(dims, B, T);
  GDN_REQUIRE(workspace_bytes >= need, GDN_EINVAL, "workspace of %zu bytes is below the %zu required",
              workspace_bytes, need);
  GDN_REQUIRE(workspace != nullptr && aligned(workspace, 256), GDN_EINVAL,
              "workspace is NULL or not 256-byte aligned");
  GDN_REQUIRE(slot_map != nullptr && aligned(slot_map, 4), GDN_EINVAL, "slot_map is NULL or misaligned");
  gdn::ReplayArgs a{};
  a.d = gdn::DecodeArgs{q, k, v, gates->a, gates->b, gates->A_log, gates->dt_bias, ckpt->base, slot_map, out,
                        ckpt->num_slots, B, dims->num_k_heads, dims->num_v_heads, (int32_t)in_dtype,
                        (int32_t)out_dtype, eff_scale(dims)};
  a.ring = ring_args(ring);
  a.T = T;
  if (read_copy != nullptr) {
    a.read_pool = read_copy->base;
    a.read_dt = (int32_t)read_copy->dtype;
  }
  return launched(gdn::launch_replay(a, ckpt->dtype, dims->dk, static_cast<float*>(workspace),
                                     static_cast<hipStream_t>(stream)));
}

gdn_status replay_flush_impl(const gdn_dims* dims, int32_t B, const gdn_pool* ckpt, const gdn_pool* read_copy,
                             const int32_t* slot_map, const gdn_ring* ring, void* stream) {
  GDN_TRY(check_dims(dims));
  GDN_REQUIRE(B >= 0, GDN_EINVAL, "B=%d must be >= 0", B);
  GDN_REQUIRE((int64_t)B * dims->num_v_heads <= INT32_MAX, GDN_EINVAL, "B * Hv exceeds the grid limit");
  if (B == 0) return ok();  // nothing is read or written
  GDN_TRY(check_pool(ckpt, "checkpoint"));
  if (read_copy != nullptr) GDN_TRY(check_dual(ckpt, read_copy));
  GDN_TRY(check_ring(ring, -1));
  GDN_REQUIRE(ring->num_slots == ckpt->num_slots, GDN_EINVAL, "ring holds %lld slots, the checkpoint pool %lld",
              (long long)ring->num_slots, (long long)ckpt->num_slots);
  GDN_REQUIRE(gdn::replay_lds_total(dims->dk, ring->L, 0) <= gdn::kMaxLds, GDN_EUNSUPPORTED,
              "ring length L=%d at dk=%d exceeds the 64 KiB LDS staging budget", ring->L, dims->dk);
  GDN_REQUIRE(slot_map != nullptr && aligned(slot_map, 4), GDN_EINVAL, "slot_map is NULL or misaligned");
  gdn::ReplayArgs a{};
  a.d.pool = ckpt->base;
  a.d.slot_map = slot_map;
  a.d.num_slots = ckpt->num_slots;
  a.d.B = B;
  a.d.Hk = dims->num_k_heads;
  a.d.Hv = dims->num_v_heads;
  a.d.in_dt = (int32_t)ring->dtype;
  a.d.scale = eff_scale(dims);
  a.ring = ring_args(ring);
  a.T = 0;
  if (read_copy != nullptr) {
    a.read_pool = read_copy->base;
    a.read_dt = (int32_t)read_copy->dtype;
  }
  return launched(gdn::launch_replay_flush(a, ckpt->dtype, dims->dk, static_cast<hipStream_t>(stream)));
}

}  // namespace

gdn_status gdn_replay_decode(const gdn_dims* dims, int32_t B, int32_t T, const void* q, const void* k,
                             const void* v, gdn_dtype in_dtype, const gdn_gates* gates, const gdn_pool* ckpt,
                             const int32_t* slot_map, const gdn_ring* ring, void* out, gdn_dtype out_dtype,
                             void* workspace, size_t workspace_bytes, void* stream) {
  return replay_decode_impl(dims, B, T, q, k, v, in_dtype, gates, ckpt, nullptr, slot_map, ring, out, out_dtype,
                            workspace, workspace_bytes, stream);
}

gdn_status gdn_replay_decode_noalloc(const gdn_dims* dims, int32_t B, int32_t T, const void* q, const void* k,
                                     const void* v, gdn_dtype in_dtype, const gdn_gates* gates, const gdn_pool* ckpt,
                                     const int32_t* slot_map, const gdn_ring* ring, void* out, gdn_dtype out_dtype,
                                     void* stream) {
  GDN_TRY(check_dims(dims));
  GDN_REQUIRE(B >= 0, GDN_EINVAL, "B=%d must be >= 0", B);
  GDN_REQUIRE(T >= 1, GDN_EINVAL, "window T=%d must be >= 1", T);
  if (B == 0) return replay_decode_impl(dims, B, T, q, k, v, in_dtype, gates, ckpt, nullptr, slot_map, ring, out,
                                        out_dtype, nullptr, 0, stream);
  const size_t need = gdn_replay_workspace_bytes(dims, B, T);
  GDN_REQUIRE(need <= gdn::kReplayScratchBytes, GDN_EUNSUPPORTED,
              "B=%d x Hv=%d x T=%d at dv=%d needs %zu bytes of workspace; the fixed scratch holds %zu "
              "(use gdn_replay_decode with a caller workspace)",
              B, dims->num_v_heads, T, dims->dv, need, gdn::kReplayScratchBytes);
  void* ws = nullptr;
  const hipError_t e = gdn::replay_scratch(&ws);
  if (e != hipSuccess) return fail(GDN_ELAUNCH, "device scratch lookup failed: %s", hipGetErrorString(e));
  return replay_decode_impl(dims, B, T, q, k, v, in_dtype, gates, ckpt, nullptr, slot_map, ring, out, out_dtype, ws,
                            gdn::kReplayScratchBytes, stream);
}

gdn_status gdn_replay_decode_dual(const gdn_dims* dims, int32_t B, int32_t T, const void* q, const void* k,
                                  const void* v, gdn_dtype in_dtype, const gdn_gates* gates,
                                  const gdn_pool* master, const gdn_pool* read_copy, const int32_t* slot_map,
                                  const gdn_ring* ring, void* out, gdn_dtype out_dtype, void* workspace,
                                  size_t workspace_bytes, void* stream) {
  if (B > 0) GDN_REQUIRE(read_copy != nullptr, GDN_EINVAL, "read copy is NULL");
  return replay_decode_impl(dims, B, T, q, k, v, in_dtype, gates, master, read_copy, slot_map, ring, out,
                            out_dtype, workspace, workspace_bytes, stream);
}

gdn_status gdn_replay_flush(const gdn_dims* dims, int32_t B, const gdn_pool* ckpt, const int32_t* slot_map,
                            const gdn_ring* ring, void* stream) {
  return replay_flush_impl(dims, B, ckpt, nullptr, slot_map, ring, stream);
}

gdn_status gdn_replay_flush_dual(const gdn_dims* dims, int32_t B, const gdn_pool* master,
                                 const gdn_pool* read_copy, const int32_t* slot_map, const gdn_ring* ring,
                                 void* stream) {
  if (B > 0) GDN_REQUIRE(read_copy != nullptr, GDN_EINVAL, "read copy is NULL");
  return replay_flush_impl(dims, B, master, read_copy, slot_map, ring, stream);
}

gdn_status gdn_replay_rollback(const gdn_dims* dims, int32_t B, const int32_t* slot_map, const int32_t* num_rejected,
                               const gdn_ring* ring, void* stream) {
  GDN_TRY(check_dims(dims));
  GDN_REQUIRE(B >= 0, GDN_EINVAL, "B=%d must be >= 0", B);
  GDN_REQUIRE((int64_t)B * dims->num_v_heads <= INT32_MAX, GDN_EINVAL, "B * Hv exceeds the grid limit");
  if (B == 0) return ok();  // nothing is read or written
  GDN_TRY(check_ring(ring, -1));
  GDN_REQUIRE(slot_map != nullptr && aligned(slot_map, 4), GDN_EINVAL, "slot_map is NULL or misaligned");
  GDN_REQUIRE(num_rejected != nullptr && aligned(num_rejected, 4), GDN_EINVAL, "num_rejected is NULL or misaligned");
  gdn::ReplayArgs a{};
  a.d.slot_map = slot_map;
  a.d.B = B;
  a.d.Hk = dims->num_k_heads;
  a.d.Hv = dims->num_v_heads;
  a.d.num_slots = ring->num_slots;
  a.ring = ring_args(ring);
  a.num_rejected = num_rejected;
  return launched(gdn::launch_replay_rollback(a, static_cast<hipStream_t>(stream)));
}

}  // extern "C"

// ------------------------------------------------------------------ Mamba2
namespace {

gdn_status check_m2_dims(const gdn_m2_dims* d) {
  GDN_REQUIRE(d != nullptr, GDN_EINVAL, "dims is NULL");
  GDN_REQUIRE(d->num_heads >= 1 && d->num_groups >= 1, GDN_EINVAL, "head and group counts must be >= 1");
  GDN_REQUIRE(d->num_heads % d->num_groups == 0, GDN_EINVAL, "H=%d is not a multiple of G=%d", d->num_heads,
              d->num_groups);
  const auto ok_dim = [](int x) { return x == 16 || x == 64 || x == 128; };
  GDN_REQUIRE(d->headdim >= 1 && d->dstate >= 1, GDN_EINVAL, "headdim and dstate must be >= 1");
  GDN_REQUIRE(ok_dim(d->headdim) && ok_dim(d->dstate), GDN_EUNSUPPORTED,
              "headdim=%d dstate=%d: compiled for {16, 64, 128} each", d->headdim, d->dstate);
  return GDN_OK;
}

gdn_status check_m2_io(const void* x, const void* Bm, const void* Cm, const gdn_m2_params* pr, int in_dt,
                       const void* y, int out_dt) {
  GDN_REQUIRE(x && Bm && Cm, GDN_EINVAL, "x, Bm or Cm is NULL");
  GDN_REQUIRE(y != nullptr, GDN_EINVAL, "y is NULL");
  const size_t eb = dtype_bytes(in_dt);
  GDN_REQUIRE(aligned(x, eb) && aligned(Bm, eb) && aligned(Cm, eb), GDN_EINVAL, "x, Bm or Cm misaligned");
  GDN_REQUIRE(aligned(y, dtype_bytes(out_dt)), GDN_EINVAL, "y misaligned for out_dtype");
  GDN_REQUIRE(pr != nullptr, GDN_EINVAL, "params is NULL");
  GDN_REQUIRE(pr->dt && pr->A_log && pr->dt_bias && pr->D, GDN_EINVAL, "a parameter pointer is NULL");
  GDN_REQUIRE(aligned(pr->dt, eb) && aligned(pr->A_log, 4) && aligned(pr->dt_bias, 4) && aligned(pr->D, 4),
              GDN_EINVAL, "a parameter pointer is misaligned");
  return GDN_OK;
}

gdn_status check_m2_ring(const gdn_m2_ring* r, int in_dt, int64_t num_slots) {
  GDN_REQUIRE(r != nullptr, GDN_EINVAL, "ring is NULL");
  GDN_REQUIRE(r->x && r->Bm && r->g && r->dtp && r->start && r->count, GDN_EINVAL, "a ring pointer is NULL");
  GDN_REQUIRE(r->num_slots == num_slots, GDN_EINVAL, "ring holds %lld slots, the checkpoint pool %lld",
              (long long)r->num_slots, (long long)num_slots);
  GDN_REQUIRE(r->L >= 1, GDN_EINVAL, "ring length L=%d must be >= 1", r->L);
  GDN_REQUIRE(r->L <= 64, GDN_EUNSUPPORTED, "ring length L=%d: at most 64 is supported", r->L);
  GDN_REQUIRE(valid_dtype(r->dtype), GDN_EINVAL, "ring dtype %d is not a gdn_dtype", (int)r->dtype);
  if (in_dt >= 0)
    GDN_REQUIRE((int)r->dtype == in_dt, GDN_EINVAL, "ring dtype %d differs from in_dtype %d", (int)r->dtype, in_dt);
  const size_t eb = dtype_bytes(r->dtype);
  GDN_REQUIRE(aligned(r->x, 16) && aligned(r->Bm, eb) && aligned(r->g, 4) && aligned(r->dtp, 4) &&
                  aligned(r->start, 4) && aligned(r->count, 4),
              GDN_EINVAL, "a ring pointer is misaligned");
  return GDN_OK;
}

gdn::M2Args m2_args(const gdn_m2_dims* d, int32_t B, int32_t T, const void* x, const void* Bm, const void* Cm,
                    int in_dt, const gdn_m2_params* pr, const gdn_pool* pool, const int32_t* slot_map, void* y,
                    int out_dt) {
  gdn::M2Args a{};
  a.x = x;
  a.Bm = Bm;
  a.Cm = Cm;
  if (pr != nullptr) {
    a.dt = pr->dt;
    a.A_log = pr->A_log;
    a.dt_bias = pr->dt_bias;
    a.Dskip = pr->D;
  }
  a.pool = pool->base;
  a.slot_map = slot_map;
  a.y = y;
  a.num_slots = pool->num_slots;
  a.B = B;
  a.H = d->num_heads;
  a.G = d->num_groups;
  a.in_dt = in_dt;
  a.out_dt = out_dt;
  a.T = T;
  return a;
}

void m2_ring_args(gdn::M2Args& a, const gdn_m2_ring* r) {
  a.L = r->L;
  a.rx = r->x;
  a.rB = r->Bm;
  a.rg = r->g;
  a.rdtp = r->dtp;
  a.start = r->start;
  a.count = r->count;
}

}  // namespace

gdn_status gdn_mamba2_decode_step(const gdn_m2_dims* dims, int32_t B, const void* x, const void* Bm,
                                  const void* Cm, gdn_dtype in_dtype, const gdn_m2_params* params,
                                  const gdn_pool* state, const int32_t* slot_map, void* y, gdn_dtype out_dtype,
                                  void* stream) {
  GDN_TRY(check_m2_dims(dims));
  GDN_REQUIRE(B >= 0, GDN_EINVAL, "B=%d must be >= 0", B);
  GDN_REQUIRE((int64_t)B * dims->num_heads <= INT32_MAX, GDN_EINVAL, "B * H exceeds the grid limit");
  GDN_TRY(check_dtypes(in_dtype, out_dtype));
  if (B == 0) return ok();  // nothing is read or written
  GDN_TRY(check_m2_io(x, Bm, Cm, params, in_dtype, y, out_dtype));
  GDN_TRY(check_pool(state, "state"));
  GDN_REQUIRE(slot_map != nullptr && aligned(slot_map, 4), GDN_EINVAL, "slot_map is NULL or misaligned");
  gdn::M2Args a = m2_args(dims, B, 1, x, Bm, Cm, in_dtype, params, state, slot_map, y, out_dtype);
  return launched(gdn::launch_m2_decode(a, state->dtype, dims->headdim, dims->dstate, static_cast<hipStream_t>(stream)));
}

gdn_status gdn_mamba2_replay_decode(const gdn_m2_dims* dims, int32_t B, int32_t T, const void* x, const void* Bm,
                                    const void* Cm, gdn_dtype in_dtype, const gdn_m2_params* params,
                                    const gdn_pool* ckpt, const int32_t* slot_map, const gdn_m2_ring* ring, void* y,
                                    gdn_dtype out_dtype, void* stream) {
  GDN_TRY(check_m2_dims(dims));
  GDN_REQUIRE(B >= 0, GDN_EINVAL, "B=%d must be >= 0", B);
  GDN_REQUIRE((int64_t)B * dims->num_heads <= INT32_MAX, GDN_EINVAL, "B * H exceeds the grid limit");
  GDN_TRY(check_dtypes(in_dtype, out_dtype));
  GDN_REQUIRE(aligned(x, 16), GDN_EINVAL, "x must be 16-byte aligned (it is read four elements at a time)");
  GDN_REQUIRE(ring != nullptr, GDN_EINVAL, "ring is NULL");
  GDN_REQUIRE(T >= 1 && T <= ring->L, GDN_EINVAL, "window T=%d must satisfy 1 <= T <= L=%d", T, ring->L);
  if (B == 0) return ok();  // nothing is read or written
  GDN_TRY(check_m2_io(x, Bm, Cm, params, in_dtype, y, out_dtype));
  GDN_TRY(check_pool(ckpt, "checkpoint"));
  GDN_TRY(check_m2_ring(ring, in_dtype, ckpt->num_slots));
  GDN_REQUIRE(gdn::m2_lds_bytes(dims->headdim, dims->dstate, ring->L, T, dims->num_heads / dims->num_groups) <=
                  gdn::kMaxLds,
              GDN_EUNSUPPORTED, "ring length L=%d with window T=%d and %d heads per group exceeds the 64 KiB staging "
              "budget", ring->L, T, dims->num_heads / dims->num_groups);
  GDN_REQUIRE(slot_map != nullptr && aligned(slot_map, 4), GDN_EINVAL, "slot_map is NULL or misaligned");
  gdn::M2Args a = m2_args(dims, B, T, x, Bm, Cm, in_dtype, params, ckpt, slot_map, y, out_dtype);
  m2_ring_args(a, ring);
  return launched(gdn::launch_m2_replay(a, ckpt->dtype, dims->headdim, dims->dstate, static_cast<hipStream_t>(stream)));
}

gdn_status gdn_mamba2_replay_flush(const gdn_m2_dims* dims, int32_t B, const gdn_pool* ckpt, const int32_t* slot_map,
                                   const gdn_m2_ring* ring, void* stream) {
  GDN_TRY(check_m2_dims(dims));
  GDN_REQUIRE(B >= 0, GDN_EINVAL, "B=%d must be >= 0", B);
  GDN_REQUIRE((int64_t)B * dims->num_heads <= INT32_MAX, GDN_EINVAL, "B * H exceeds the grid limit");
  if (B == 0) return ok();
  GDN_TRY(check_pool(ckpt, "checkpoint"));
  GDN_TRY(check_m2_ring(ring, -1, ckpt->num_slots));
  GDN_REQUIRE(gdn::m2_lds_bytes(dims->headdim, dims->dstate, ring->L, 0, 1) <= gdn::kMaxLds, GDN_EUNSUPPORTED,
              "ring length L=%d exceeds the 64 KiB staging budget", ring->L);
  GDN_REQUIRE(slot_map != nullptr && aligned(slot_map, 4), GDN_EINVAL, "slot_map is NULL or misaligned");
  gdn::M2Args a = m2_args(dims, B, 0, nullptr, nullptr, nullptr, (int)ring->dtype, nullptr, ckpt, slot_map, nullptr,
                          GDN_F32);
  m2_ring_args(a, ring);
  return launched(gdn::launch_m2_replay(a, ckpt->dtype, dims->headdim, dims->dstate, static_cast<hipStream_t>(stream)));
}

gdn_status gdn_mamba2_replay_rollback(const gdn_m2_dims* dims, int32_t B, const int32_t* slot_map,
                                      const int32_t* num_rejected, const gdn_m2_ring* ring, void* stream) {
  GDN_TRY(check_m2_dims(dims));
  GDN_REQUIRE(B >= 0, GDN_EINVAL, "B=%d must be >= 0", B);
  if (B == 0) return ok();
  GDN_REQUIRE(ring != nullptr, GDN_EINVAL, "ring is NULL");
  GDN_TRY(check_m2_ring(ring, -1, ring->num_slots));
  GDN_REQUIRE(slot_map != nullptr && aligned(slot_map, 4), GDN_EINVAL, "slot_map is NULL or misaligned");
  GDN_REQUIRE(num_rejected != nullptr && aligned(num_rejected, 4), GDN_EINVAL, "num_rejected is NULL or misaligned");
  gdn::M2Args a{};
  a.slot_map = slot_map;
  a.num_slots = ring->num_slots;
  a.B = B;
  a.num_rejected = num_rejected;
  m2_ring_args(a, ring);
  return launched(gdn::launch_m2_rollback(a, static_cast<hipStream_t>(stream)));
}
