// C ABI entry points: host-side validation, workspace layout and launches.
// Every check that can be made on the host is made before anything is
// enqueued; device-side conditions are recorded in the workspace flag word.
#include "skv_internal.h"

#include <hip/hip_ext.h>

#include <stdarg.h>
#include <stdio.h>
#include <string.h>
#include <stdint.h>

#include <mutex>
#include <vector>

namespace skv {

// ---- diagnostic kernel timer (not thread-safe, not for graph capture) ----
namespace {
struct KernelTimer {
  int kind = 0;                 // 0: off, else the kind of kernel timed
  std::vector<hipEvent_t> ev;   // begin/end pairs
  size_t used = 0;              // events recorded since enable
  int64_t dropped = 0;
};
KernelTimer g_timer;
constexpr size_t kTimerPairs = 4096;
}  // namespace

bool timer_next(int kind, hipEvent_t* start, hipEvent_t* stop) {
  if (g_timer.kind != kind) return false;
  if (g_timer.used + 2 > g_timer.ev.size()) {
    ++g_timer.dropped;
    return false;
  }
  *start = g_timer.ev[g_timer.used];
  *stop = g_timer.ev[g_timer.used + 1];
  g_timer.used += 2;
  return true;
}

static thread_local char g_err[512] = "";

skv_status set_error(skv_status s, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof(g_err), fmt, ap);
  va_end(ap);
  return s;
}

static skv_status ok() {
  g_err[0] = '\0';
  return SKV_OK;
}

skv_status validate_desc(const skv_layer_desc* d) {
  if (!d) return set_error(SKV_ERR_INVALID, "descriptor is NULL");
  if (d->struct_size < sizeof(skv_layer_desc))
    return set_error(SKV_ERR_INVALID, "struct_size %u < %zu", d->struct_size, sizeof(skv_layer_desc));
  if (d->batch < 1) return set_error(SKV_ERR_INVALID, "batch %d < 1", d->batch);
  if (d->max_ctx < 1) return set_error(SKV_ERR_INVALID, "max_ctx %d < 1", d->max_ctx);
  if (d->n_kv_heads < 1 || d->n_q_heads < d->n_kv_heads || d->n_q_heads % d->n_kv_heads)
    return set_error(SKV_ERR_INVALID, "n_q_heads %d must be a positive multiple of n_kv_heads %d",
                     d->n_q_heads, d->n_kv_heads);
  if (d->n_q_heads / d->n_kv_heads > 16)
    return set_error(SKV_ERR_UNSUPPORTED, "query heads per KV head %d > 16", d->n_q_heads / d->n_kv_heads);
  if (d->head_dim != 128 && d->head_dim != 256)
    return set_error(SKV_ERR_UNSUPPORTED, "head_dim %d not in {128, 256}", d->head_dim);
  if (d->topk < 1 || d->topk > kMaxTopk)
    return set_error(SKV_ERR_UNSUPPORTED, "topk %d outside [1, %d]", d->topk, kMaxTopk);
  if (d->n_sink < 0 || d->n_tail < 0) return set_error(SKV_ERR_INVALID, "negative n_sink / n_tail");
  if (d->index_mode == SKV_INDEX_SKETCH_INT4) {
    if (d->block != 1) return set_error(SKV_ERR_INVALID, "token mode needs block == 1 (got %d)", d->block);
    if (d->rank < 16 || d->rank > 256 || d->rank % 16)
      return set_error(SKV_ERR_UNSUPPORTED, "rank %d not a multiple of 16 in [16, 256]", d->rank);
    const int tb = d->n_kv_heads * d->rank / 2;
    if (tb != 32 && tb != 64 && tb != 128 && tb != 256)
      return set_error(SKV_ERR_UNSUPPORTED, "sketch bytes per token %d not in {32,64,128,256}", tb);
    if (d->q_dtype != SKV_Q_F16) return set_error(SKV_ERR_UNSUPPORTED, "token mode needs fp16 queries");
    if (d->kv_dtype == SKV_KV_I8_ROWSCALE) {
      if (d->head_dim != 256) return set_error(SKV_ERR_UNSUPPORTED, "int8 K/V needs head_dim 256");
    } else if (d->kv_dtype != SKV_KV_F16) {
      return set_error(SKV_ERR_UNSUPPORTED, "token mode K/V must be int8+scale or fp16");
    }
    if ((int64_t)d->n_sink + d->topk + d->n_tail > (int64_t)1 << 20)
      return set_error(SKV_ERR_UNSUPPORTED, "n_sink + topk + n_tail too large");
  } else if (d->index_mode == SKV_INDEX_POOLED_BF16) {
    if (d->block != 4) return set_error(SKV_ERR_INVALID, "block mode needs block == 4 (got %d)", d->block);
    if (d->n_sink != 0 || d->n_tail != 0)
      return set_error(SKV_ERR_UNSUPPORTED, "block mode has no sinks / tail");
    if (d->index_dim != 64 && d->index_dim != 128 && d->index_dim != 256)
      return set_error(SKV_ERR_UNSUPPORTED, "index_dim %d not in {64,128,256}", d->index_dim);
    if (d->kv_dtype != SKV_KV_BF16 || d->q_dtype != SKV_Q_BF16)
      return set_error(SKV_ERR_UNSUPPORTED, "block mode needs bf16 K/V and queries");
  } else {
    return set_error(SKV_ERR_INVALID, "index_mode %d unknown", d->index_mode);
  }
  {
    const int64_t cand = max_candidates(*d);
    const int seg = d->index_mode == SKV_INDEX_SKETCH_INT4 ? kSegTok : kSegBlk;
    if ((cand + seg - 1) / seg > kMaxSeg)
      return set_error(SKV_ERR_UNSUPPORTED, "more than %d candidates per sequence", kMaxSeg * seg);
  }
  if (select_capacity(*d) > kMaxAttChunks * att_rows_per_wg(*d))
    return set_error(SKV_ERR_UNSUPPORTED, "select capacity %d > %d", select_capacity(*d),
                     kMaxAttChunks * att_rows_per_wg(*d));
  return ok();
}

static skv_status check_ws(const skv_layer_desc* d, void* ws, size_t ws_bytes, WsLayout* L) {
  *L = ws_layout(*d);
  if (!ws) return set_error(SKV_ERR_WORKSPACE, "workspace is NULL");
  if (ws_bytes < L->total)
    return set_error(SKV_ERR_WORKSPACE, "workspace %zu bytes < required %zu", ws_bytes, L->total);
  if (((uintptr_t)ws) % 256) return set_error(SKV_ERR_WORKSPACE, "workspace not 256-byte aligned");
  return SKV_OK;
}

static skv_status launched(hipError_t e, const char* what) {
  if (e != hipSuccess) return set_error(SKV_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
  return ok();
}

static skv_status check_kv(const skv_layer_desc* d, const skv_kv_view* kv) {
  if (!kv || !kv->k || !kv->v) return set_error(SKV_ERR_INVALID, "kv view / k / v is NULL");
  if (kv->rows < 1) return set_error(SKV_ERR_INVALID, "kv rows %lld < 1", (long long)kv->rows);
  if (d->kv_dtype == SKV_KV_I8_ROWSCALE && (!kv->k_scale || !kv->v_scale))
    return set_error(SKV_ERR_INVALID, "int8 K/V need k_scale and v_scale");
  if ((((uintptr_t)kv->k) | ((uintptr_t)kv->v)) % 16)
    return set_error(SKV_ERR_INVALID, "k / v must be 16-byte aligned");
  return SKV_OK;
}

// ---- scratch of the allocation-free step ---------------------------------
// A file-scope device array stands in for the caller's workspace; every device
// the library runs on holds its own copy (zero at load) until the process
// ends.  Host code never passes `scratch` itself to a kernel (its host-side
// name is a stand-in, not a device address): the address is looked up once per
// device with hipGetSymbolAddress and kept below.
constexpr size_t kScratchBytes = (size_t)SKV_NOALLOC_SCRATCH_BYTES;
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
static void* g_scratch_addr[kMaxDevices];
static std::mutex g_scratch_mu;

// device address of `scratch` on the current device
static skv_status scratch_address(void** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return set_error(SKV_ERR_HIP, "step_noalloc: %s", hipGetErrorString(e));
  if (dev < 0 || dev >= kMaxDevices)
    return set_error(SKV_ERR_UNSUPPORTED, "step_noalloc: device %d beyond %d", dev, kMaxDevices);
  std::lock_guard<std::mutex> guard(g_scratch_mu);
  if (!g_scratch_addr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !p)
      return set_error(SKV_ERR_HIP, "step_noalloc: scratch address: %s", hipGetErrorString(e));
    g_scratch_addr[dev] = p;
  }
  *out = g_scratch_addr[dev];
  return SKV_OK;
}

// hands the call's flag word to the caller (if asked) and clears it, so the
// next call on this device starts from zero
__global__ void flags_handoff_kernel(uint32_t* __restrict__ f, uint32_t* __restrict__ out) {
  const uint32_t v = *f;
  if (out) *out = v;
  *f = 0u;
}

// ---- plain streaming read (measurement aid) -------------------------------
// Every 16-byte word of the buffer is loaded once (8 per thread in flight);
// each workgroup stores the xor of what it read, so no load is dropped.
constexpr int kReadThreads = 256;
constexpr int kReadUnroll = 8;
__global__ __launch_bounds__(kReadThreads) void read_bytes_kernel(const uint4* __restrict__ src,
                                                                  size_t n16, uint32_t* __restrict__ sink) {
  uint32_t acc = 0;
  const size_t stride = (size_t)gridDim.x * kReadThreads;
  size_t i = (size_t)blockIdx.x * kReadThreads + threadIdx.x;
  for (; i + (kReadUnroll - 1) * stride < n16; i += kReadUnroll * stride) {
    uint4 w[kReadUnroll];
#pragma unroll
    for (int u = 0; u < kReadUnroll; ++u) w[u] = src[i + u * stride];
#pragma unroll
    for (int u = 0; u < kReadUnroll; ++u) acc ^= w[u].x ^ w[u].y ^ w[u].z ^ w[u].w;
  }
  for (; i < n16; i += stride) {
    const uint4 w = src[i];
    acc ^= w.x ^ w.y ^ w.z ^ w.w;
  }
  for (int o = 32; o > 0; o >>= 1) acc ^= (uint32_t)__shfl_xor((int)acc, o);
  __shared__ uint32_t s_acc[kReadThreads / 64];
  if ((threadIdx.x & 63) == 0) s_acc[threadIdx.x >> 6] = acc;
  __syncthreads();
  if (threadIdx.x == 0) sink[blockIdx.x] = s_acc[0] ^ s_acc[1] ^ s_acc[2] ^ s_acc[3];
}

}  // namespace skv

using namespace skv;

extern "C" {

int sparsekv_abi_version(void) { return SPARSEKV_ABI_VERSION; }

const char* sparsekv_status_str(skv_status s) {
  switch (s) {
    case SKV_OK: return "ok";
    case SKV_ERR_INVALID: return "invalid argument";
    case SKV_ERR_UNSUPPORTED: return "unsupported configuration";
    case SKV_ERR_WORKSPACE: return "workspace missing or too small";
    case SKV_ERR_OOM: return "out of memory";
    case SKV_ERR_HIP: return "HIP runtime error";
    case SKV_ERR_HOST_MEMORY: return "host memory not pinned / mapped";
    case SKV_ERR_STATE: return "device flags raised";
    default: return "unknown status";
  }
}

const char* sparsekv_last_error(void) { return g_err; }

skv_status sparsekv_validate(const skv_layer_desc* d) { return validate_desc(d); }

skv_status sparsekv_select_capacity(const skv_layer_desc* d, int32_t* cap) {
  skv_status s = validate_desc(d);
  if (s != SKV_OK) return s;
  if (!cap) return set_error(SKV_ERR_INVALID, "cap is NULL");
  *cap = select_capacity(*d);
  return SKV_OK;
}

skv_status sparsekv_workspace_size(const skv_layer_desc* d, size_t* bytes) {
  skv_status s = validate_desc(d);
  if (s != SKV_OK) return s;
  if (!bytes) return set_error(SKV_ERR_INVALID, "bytes is NULL");
  *bytes = ws_layout(*d).total;
  return SKV_OK;
}

// the layer with n_query query tokens per sequence seen as batch*n_query
// virtual sequences (token mode)
static skv_status multi_desc(const skv_layer_desc* d, int32_t n_query, skv_layer_desc* dv) {
  skv_status s = validate_desc(d);
  if (s != SKV_OK) return s;
  if (d->index_mode != SKV_INDEX_SKETCH_INT4)
    return set_error(SKV_ERR_UNSUPPORTED, "multi-query step: token mode only");
  if (n_query < 1 || n_query > kMaxQueries)
    return set_error(SKV_ERR_UNSUPPORTED, "n_query %d outside [1, %d]", n_query, kMaxQueries);
  const int tb = d->n_kv_heads * d->rank / 2;
  if (tb != 64 && tb != 128 && tb != 256)
    return set_error(SKV_ERR_UNSUPPORTED, "multi-query step: sketch bytes per token %d not in {64,128,256}", tb);
  if ((int64_t)d->batch * n_query > (1 << 20))
    return set_error(SKV_ERR_UNSUPPORTED, "batch * n_query too large");
  *dv = *d;
  dv->batch = d->batch * n_query;
  return validate_desc(dv);
}

skv_status sparsekv_workspace_size_multi(const skv_layer_desc* d, int32_t n_query, size_t* bytes) {
  skv_layer_desc dv;
  skv_status s = multi_desc(d, n_query, &dv);
  if (s != SKV_OK) return s;
  if (!bytes) return set_error(SKV_ERR_INVALID, "bytes is NULL");
  *bytes = ws_layout(dv).total;
  return SKV_OK;
}

skv_status sparsekv_step_multi(const skv_layer_desc* d, int32_t n_query, const int32_t* ctx_len,
                               const void* q, const float* basis, int8_t* qs, float* qs_scale,
                               const void* index_keys, const uint16_t* index_scale,
                               const skv_kv_view* kv, int32_t* idx, int32_t* n_sel, float sm_scale,
                               float* out, void* ws, size_t ws_bytes, void* stream) {
  skv_layer_desc dv;
  skv_status s = multi_desc(d, n_query, &dv);
  if (s != SKV_OK) return s;
  WsLayout L;
  if ((s = check_ws(&dv, ws, ws_bytes, &L)) != SKV_OK) return s;
  if ((s = check_kv(d, kv)) != SKV_OK) return s;
  if (!ctx_len || !q || !basis || !qs || !qs_scale || !index_keys || !index_scale || !idx || !n_sel || !out)
    return set_error(SKV_ERR_INVALID, "step_multi: NULL pointer");
  if ((((uintptr_t)index_keys) | ((uintptr_t)qs)) % 16)
    return set_error(SKV_ERR_INVALID, "step_multi: index_keys and qs must be 16-byte aligned");
  hipStream_t st = (hipStream_t)stream;
  hipError_t e = launch_qsketch_proj(dv, q, basis, ws, L, st);
  if (e == hipSuccess)
    e = launch_sample_collect_multi(dv, n_query, ctx_len, qs, qs_scale, index_keys, index_scale, ws, L, st);
  if (e == hipSuccess)
    e = launch_final_multi(dv, n_query, ctx_len, qs, index_keys, index_scale, idx, n_sel, ws, L, st);
  if (e == hipSuccess) e = launch_attend(dv, q, *kv, idx, n_sel, sm_scale, out, ws, L, st, n_query);
  return launched(e, "step_multi");
}

skv_status sparsekv_attend_multi(const skv_layer_desc* d, int32_t n_query, const void* q,
                                 const skv_kv_view* kv, const int32_t* idx, const int32_t* n_sel,
                                 float sm_scale, float* out, void* ws, size_t ws_bytes,
                                 void* stream) {
  skv_layer_desc dv;
  skv_status s = multi_desc(d, n_query, &dv);
  if (s != SKV_OK) return s;
  WsLayout L;
  if ((s = check_ws(&dv, ws, ws_bytes, &L)) != SKV_OK) return s;
  if ((s = check_kv(d, kv)) != SKV_OK) return s;
  if (!q || !idx || !n_sel || !out) return set_error(SKV_ERR_INVALID, "attend_multi: NULL pointer");
  if (((uintptr_t)q) % 16) return set_error(SKV_ERR_INVALID, "attend_multi: q not 16-byte aligned");
  return launched(launch_attend(dv, q, *kv, idx, n_sel, sm_scale, out, ws, L, (hipStream_t)stream,
                                n_query),
                  "attend_multi");
}

static skv_status prefill_desc(const skv_layer_desc* d, int32_t n_query) {
  skv_status s = validate_desc(d);
  if (s != SKV_OK) return s;
  if (d->kv_dtype != SKV_KV_F16 && d->kv_dtype != SKV_KV_BF16)
    return set_error(SKV_ERR_UNSUPPORTED, "prefill: K/V rows must be fp16 or bf16");
  if ((d->kv_dtype == SKV_KV_BF16) != (d->q_dtype == SKV_Q_BF16))
    return set_error(SKV_ERR_UNSUPPORTED, "prefill: queries must have the K/V element type");
  if (n_query < 1) return set_error(SKV_ERR_INVALID, "prefill: n_query %d < 1", n_query);
  return SKV_OK;
}

skv_status sparsekv_prefill_workspace_size(const skv_layer_desc* d, int32_t n_query, size_t* bytes) {
  skv_status s = prefill_desc(d, n_query);
  if (s != SKV_OK) return s;
  if (!bytes) return set_error(SKV_ERR_INVALID, "bytes is NULL");
  *bytes = prefill_workspace_bytes(*d, n_query);
  return ok();
}

skv_status sparsekv_prefill_attend(const skv_layer_desc* d, int32_t n_query, const void* q,
                                   const int32_t* idx, const int32_t* n_sel, int32_t cap,
                                   const void* host_k, const void* host_v, int64_t n_tokens,
                                   void* chunk_buf, size_t chunk_bytes, float sm_scale, float* out,
                                   void* ws, size_t ws_bytes, void* stream) {
  skv_status s = prefill_desc(d, n_query);
  if (s != SKV_OK) return s;
  if (!q || !idx || !n_sel || !host_k || !host_v || !chunk_buf || !out || !ws)
    return set_error(SKV_ERR_INVALID, "prefill: NULL pointer");
  if (cap < 1) return set_error(SKV_ERR_INVALID, "prefill: cap %d < 1", cap);
  if (n_tokens < 1 || n_tokens > INT32_MAX)
    return set_error(SKV_ERR_INVALID, "prefill: n_tokens %lld outside [1, 2^31)", (long long)n_tokens);
  if (prefill_chunk_tokens(*d, chunk_bytes) < 1)
    return set_error(SKV_ERR_INVALID, "prefill: chunk buffer of %zu bytes holds no token", chunk_bytes);
  if (((uintptr_t)chunk_buf) % 16) return set_error(SKV_ERR_INVALID, "prefill: chunk buffer not 16-byte aligned");
  if (ws_bytes < prefill_workspace_bytes(*d, n_query))
    return set_error(SKV_ERR_WORKSPACE, "workspace %zu bytes < required %zu", ws_bytes,
                     prefill_workspace_bytes(*d, n_query));
  if (((uintptr_t)ws) % 256) return set_error(SKV_ERR_WORKSPACE, "workspace not 256-byte aligned");
  return launched(launch_prefill(*d, n_query, q, idx, n_sel, cap, host_k, host_v, n_tokens, chunk_buf,
                                 chunk_bytes, sm_scale, out, ws, (hipStream_t)stream),
                  "prefill");
}

skv_status sparsekv_qsketch(const skv_layer_desc* d, const void* q, const float* basis, int8_t* qs,
                            float* qs_scale, void* ws, size_t ws_bytes, void* stream) {
  skv_status s = validate_desc(d);
  if (s != SKV_OK) return s;
  if (d->index_mode != SKV_INDEX_SKETCH_INT4)
    return set_error(SKV_ERR_INVALID, "qsketch is a token-mode stage");
  WsLayout L;
  if ((s = check_ws(d, ws, ws_bytes, &L)) != SKV_OK) return s;
  if (!q || !basis || !qs || !qs_scale) return set_error(SKV_ERR_INVALID, "qsketch: NULL pointer");
  return launched(launch_qsketch(*d, q, basis, qs, qs_scale, ws, L, (hipStream_t)stream), "qsketch");
}

skv_status sparsekv_score(const skv_layer_desc* d, const int32_t* ctx_len, const void* index_query,
                          const void* index_keys, const uint16_t* index_scale, double* keys,
                          void* ws, size_t ws_bytes, void* stream) {
  skv_status s = validate_desc(d);
  if (s != SKV_OK) return s;
  WsLayout L;
  if ((s = check_ws(d, ws, ws_bytes, &L)) != SKV_OK) return s;
  if (!ctx_len || !index_query || !index_keys || !keys)
    return set_error(SKV_ERR_INVALID, "score: NULL pointer");
  if (d->index_mode == SKV_INDEX_SKETCH_INT4 && !index_scale)
    return set_error(SKV_ERR_INVALID, "score: token mode needs index_scale");
  if (((uintptr_t)index_keys) % 16) return set_error(SKV_ERR_INVALID, "score: index_keys not 16-byte aligned");
  return launched(launch_score(*d, ctx_len, index_query, index_keys, index_scale, keys,
                               ws_ptr<uint32_t>(ws, L.flags), (hipStream_t)stream),
                  "score");
}

skv_status sparsekv_topk(const skv_layer_desc* d, const int32_t* ctx_len, const double* keys,
                         int32_t* idx, int32_t* n_sel, void* ws, size_t ws_bytes, void* stream) {
  skv_status s = validate_desc(d);
  if (s != SKV_OK) return s;
  WsLayout L;
  if ((s = check_ws(d, ws, ws_bytes, &L)) != SKV_OK) return s;
  if (!ctx_len || !keys || !idx || !n_sel) return set_error(SKV_ERR_INVALID, "topk: NULL pointer");
  return launched(launch_topk(*d, ctx_len, keys, idx, n_sel, ws, L, (hipStream_t)stream), "topk");
}

skv_status sparsekv_score_topk(const skv_layer_desc* d, const int32_t* ctx_len,
                               const void* index_query, const void* index_keys,
                               const uint16_t* index_scale, int32_t* idx, int32_t* n_sel,
                               void* ws, size_t ws_bytes, void* stream) {
  skv_status s = validate_desc(d);
  if (s != SKV_OK) return s;
  WsLayout L;
  if ((s = check_ws(d, ws, ws_bytes, &L)) != SKV_OK) return s;
  if (!ctx_len || !index_query || !index_keys || !idx || !n_sel)
    return set_error(SKV_ERR_INVALID, "score_topk: NULL pointer");
  if (d->index_mode == SKV_INDEX_SKETCH_INT4 && !index_scale)
    return set_error(SKV_ERR_INVALID, "score_topk: token mode needs index_scale");
  if (((uintptr_t)index_keys) % 16) return set_error(SKV_ERR_INVALID, "score_topk: index_keys not 16-byte aligned");
  return launched(launch_score_select(*d, ctx_len, index_query, nullptr, nullptr, nullptr, nullptr, index_keys,
                                      index_scale, idx, n_sel, ws, L, (hipStream_t)stream),
                  "score_topk");
}

skv_status sparsekv_attend(const skv_layer_desc* d, const void* q, const skv_kv_view* kv,
                           const int32_t* idx, const int32_t* n_sel, float sm_scale, float* out,
                           void* ws, size_t ws_bytes, void* stream) {
  skv_status s = validate_desc(d);
  if (s != SKV_OK) return s;
  WsLayout L;
  if ((s = check_ws(d, ws, ws_bytes, &L)) != SKV_OK) return s;
  if ((s = check_kv(d, kv)) != SKV_OK) return s;
  if (!q || !idx || !n_sel || !out) return set_error(SKV_ERR_INVALID, "attend: NULL pointer");
  if (((uintptr_t)q) % 16) return set_error(SKV_ERR_INVALID, "attend: q not 16-byte aligned");
  return launched(launch_attend(*d, q, *kv, idx, n_sel, sm_scale, out, ws, L, (hipStream_t)stream),
                  "attend");
}

static skv_status check_step_args(const skv_layer_desc* d, const int32_t* ctx_len, const void* q,
                                  const float* basis, const int8_t* qs, const float* qs_scale,
                                  const void* index_query, const void* index_keys,
                                  const uint16_t* index_scale, const skv_kv_view* kv,
                                  const int32_t* idx, const int32_t* n_sel, const float* out) {
  skv_status s = check_kv(d, kv);
  if (s != SKV_OK) return s;
  if (!ctx_len || !q || !index_keys || !idx || !n_sel || !out)
    return set_error(SKV_ERR_INVALID, "step: NULL pointer");
  if (((uintptr_t)index_keys) % 16) return set_error(SKV_ERR_INVALID, "step: index_keys not 16-byte aligned");
  const bool tok = d->index_mode == SKV_INDEX_SKETCH_INT4;
  if (tok && (!basis || !qs || !qs_scale || !index_scale))
    return set_error(SKV_ERR_INVALID, "step: token mode needs basis, qs, qs_scale and index_scale");
  if (!tok && !index_query) return set_error(SKV_ERR_INVALID, "step: block mode needs index_query");
  return SKV_OK;
}

static hipError_t launch_step(const skv_layer_desc* d, const int32_t* ctx_len, const void* q,
                              const float* basis, int8_t* qs, float* qs_scale,
                              const void* index_query, const void* index_keys,
                              const uint16_t* index_scale, const skv_kv_view* kv, int32_t* idx,
                              int32_t* n_sel, float sm_scale, float* out, void* ws,
                              const WsLayout& L, hipStream_t st) {
  const bool tok = d->index_mode == SKV_INDEX_SKETCH_INT4;
  // token mode: the projection here, its quantization in the front kernel
  hipError_t e = tok ? launch_qsketch_proj(*d, q, basis, ws, L, st) : hipSuccess;
  if (e == hipSuccess)
    e = launch_score_select(*d, ctx_len, tok ? nullptr : index_query, q, basis, tok ? qs : nullptr,
                            tok ? qs_scale : nullptr, index_keys, index_scale, idx, n_sel, ws, L, st);
  if (e == hipSuccess) e = launch_attend(*d, q, *kv, idx, n_sel, sm_scale, out, ws, L, st);
  return e;
}

skv_status sparsekv_step(const skv_layer_desc* d, const int32_t* ctx_len, const void* q,
                         const float* basis, int8_t* qs, float* qs_scale, const void* index_query,
                         const void* index_keys, const uint16_t* index_scale,
                         const skv_kv_view* kv, int32_t* idx, int32_t* n_sel, float sm_scale,
                         float* out, void* ws, size_t ws_bytes, void* stream) {
  skv_status s = validate_desc(d);
  if (s != SKV_OK) return s;
  WsLayout L;
  if ((s = check_ws(d, ws, ws_bytes, &L)) != SKV_OK) return s;
  if ((s = check_step_args(d, ctx_len, q, basis, qs, qs_scale, index_query, index_keys, index_scale,
                           kv, idx, n_sel, out)) != SKV_OK)
    return s;
  return launched(launch_step(d, ctx_len, q, basis, qs, qs_scale, index_query, index_keys,
                              index_scale, kv, idx, n_sel, sm_scale, out, ws, L, (hipStream_t)stream),
                  "step");
}

skv_status sparsekv_step_noalloc(const skv_layer_desc* d, const int32_t* ctx_len, const void* q,
                                 const float* basis, int8_t* qs, float* qs_scale,
                                 const void* index_query, const void* index_keys,
                                 const uint16_t* index_scale, const skv_kv_view* kv, int32_t* idx,
                                 int32_t* n_sel, float sm_scale, float* out, uint32_t* flags,
                                 void* stream) {
  skv_status s = validate_desc(d);
  if (s != SKV_OK) return s;
  const WsLayout L = ws_layout(*d);
  if (L.total > kScratchBytes)
    return set_error(SKV_ERR_WORKSPACE, "step_noalloc: the layer needs %zu bytes of scratch, more than %zu",
                     L.total, kScratchBytes);
  if ((s = check_step_args(d, ctx_len, q, basis, qs, qs_scale, index_query, index_keys, index_scale,
                           kv, idx, n_sel, out)) != SKV_OK)
    return s;
  void* ws = nullptr;   // the device address of `scratch`, never the array's host-side name
  if ((s = scratch_address(&ws)) != SKV_OK) return s;
  const hipStream_t st = (hipStream_t)stream;
  hipError_t e = launch_step(d, ctx_len, q, basis, qs, qs_scale, index_query, index_keys,
                             index_scale, kv, idx, n_sel, sm_scale, out, ws, L, st);
  if (e != hipSuccess) return launched(e, "step_noalloc");
  hipLaunchKernelGGL(flags_handoff_kernel, dim3(1), dim3(1), 0, st, ws_ptr<uint32_t>(ws, L.flags), flags);
  return launched(hipGetLastError(), "step_noalloc");
}

skv_status sparsekv_append(const skv_layer_desc* d, int32_t* ctx_len, const void* k_new,
                           const void* v_new, const float* basis, const skv_kv_view* kv,
                           void* index_keys, uint16_t* index_scale, void* ws, size_t ws_bytes,
                           void* stream) {
  skv_status s = validate_desc(d);
  if (s != SKV_OK) return s;
  if (d->index_mode != SKV_INDEX_SKETCH_INT4)
    return set_error(SKV_ERR_UNSUPPORTED, "append: token mode only");
  WsLayout L;
  if ((s = check_ws(d, ws, ws_bytes, &L)) != SKV_OK) return s;
  if ((s = check_kv(d, kv)) != SKV_OK) return s;
  if (!ctx_len || !k_new || !v_new || !basis || !index_keys || !index_scale)
    return set_error(SKV_ERR_INVALID, "append: NULL pointer");
  if (kv->rows < d->max_ctx)
    return set_error(SKV_ERR_INVALID, "append: kv rows %lld < max_ctx %d", (long long)kv->rows, d->max_ctx);
  return launched(launch_append(*d, ctx_len, k_new, v_new, basis, *kv, index_keys, index_scale, ws, L,
                                (hipStream_t)stream),
                  "append");
}

skv_status sparsekv_append_block(const skv_layer_desc* d, int32_t* ctx_len, const void* k_new,
                                 const void* v_new, const void* index_raw, void* index_stage,
                                 const skv_kv_view* kv, void* index_keys, void* ws,
                                 size_t ws_bytes, void* stream) {
  skv_status s = validate_desc(d);
  if (s != SKV_OK) return s;
  if (d->index_mode != SKV_INDEX_POOLED_BF16)
    return set_error(SKV_ERR_UNSUPPORTED, "append_block: block mode only");
  WsLayout L;
  if ((s = check_ws(d, ws, ws_bytes, &L)) != SKV_OK) return s;
  if ((s = check_kv(d, kv)) != SKV_OK) return s;
  if (!ctx_len || !k_new || !v_new || !index_raw || !index_stage || !index_keys)
    return set_error(SKV_ERR_INVALID, "append_block: NULL pointer");
  if (kv->rows < d->max_ctx)
    return set_error(SKV_ERR_INVALID, "append_block: kv rows %lld < max_ctx %d", (long long)kv->rows,
                     d->max_ctx);
  return launched(launch_append_block(*d, ctx_len, k_new, v_new, index_raw, index_stage, *kv,
                                      index_keys, ws, L, (hipStream_t)stream),
                  "append_block");
}

skv_status sparsekv_read_bytes(const void* src, size_t bytes, uint32_t* sink, int32_t n_wg,
                               void* stream) {
  if (!src || !sink) return set_error(SKV_ERR_INVALID, "read_bytes: NULL pointer");
  if (((uintptr_t)src) % 16 || bytes % 16) return set_error(SKV_ERR_INVALID, "read_bytes: needs 16-byte alignment and size");
  if (n_wg < 1 || n_wg > SKV_READ_MAX_WG) return set_error(SKV_ERR_INVALID, "read_bytes: n_wg %d outside [1, %d]", n_wg, SKV_READ_MAX_WG);
  if (bytes == 0) return SKV_OK;
  hipEvent_t ev0 = nullptr, ev1 = nullptr;
  const hipStream_t st = (hipStream_t)stream;
  if (timer_next(kTimerStream, &ev0, &ev1))
    hipExtLaunchKernelGGL(read_bytes_kernel, dim3(n_wg), dim3(kReadThreads), 0, st, ev0, ev1, 0,
                          (const uint4*)src, bytes / 16, sink);
  else
    hipLaunchKernelGGL(read_bytes_kernel, dim3(n_wg), dim3(kReadThreads), 0, st, (const uint4*)src, bytes / 16, sink);
  return launched(hipGetLastError(), "read_bytes");
}

skv_status sparsekv_timer_enable(int enable) {
  if (enable && g_timer.ev.empty()) {
    g_timer.ev.resize(2 * kTimerPairs);
    for (auto& e : g_timer.ev)
      if (hipEventCreate(&e) != hipSuccess) {
        g_timer.ev.clear();
        return set_error(SKV_ERR_HIP, "timer: event creation failed");
      }
  }
  g_timer.kind = enable == 0 ? 0 : (enable == SKV_TIMER_ATTEND ? SKV_TIMER_ATTEND : SKV_TIMER_STREAM);
  g_timer.used = 0;
  g_timer.dropped = 0;
  return ok();
}

skv_status sparsekv_set_contraction_path(int32_t path) {
  if (path != SKV_PATH_MFMA && path != SKV_PATH_VALU)
    return set_error(SKV_ERR_INVALID, "contraction path: %d is neither SKV_PATH_MFMA nor SKV_PATH_VALU", (int)path);
  g_contract_path = path;
  return ok();
}

skv_status sparsekv_timer_read(double* total_ms, int64_t* launches) {
  if (!total_ms || !launches) return set_error(SKV_ERR_INVALID, "timer: NULL pointer");
  double t = 0.0;
  for (size_t i = 0; i + 1 < g_timer.used; i += 2) {
    float ms = 0.0f;
    if (hipEventSynchronize(g_timer.ev[i + 1]) != hipSuccess ||
        hipEventElapsedTime(&ms, g_timer.ev[i], g_timer.ev[i + 1]) != hipSuccess)
      return set_error(SKV_ERR_HIP, "timer: %s", hipGetErrorString(hipGetLastError()));
    t += ms;
  }
  *total_ms = t;
  *launches = (int64_t)(g_timer.used / 2);
  return ok();
}

skv_status sparsekv_check(void* ws, size_t ws_bytes, void* stream, uint32_t* flags) {
  if (!ws || ws_bytes < 4) return set_error(SKV_ERR_WORKSPACE, "check: workspace missing");
  uint32_t f = 0, zero = 0;
  hipStream_t st = (hipStream_t)stream;
  if (hipStreamSynchronize(st) != hipSuccess ||
      hipMemcpy(&f, ws, 4, hipMemcpyDeviceToHost) != hipSuccess ||
      hipMemcpy(ws, &zero, 4, hipMemcpyHostToDevice) != hipSuccess)
    return set_error(SKV_ERR_HIP, "check: %s", hipGetErrorString(hipGetLastError()));
  if (flags) *flags = f;
  if (f & ~(uint32_t)SKV_FLAG_TOPK_SLOW)
    return set_error(SKV_ERR_STATE, "device flags 0x%x", f);
  return ok();
}

}  // extern "C"
