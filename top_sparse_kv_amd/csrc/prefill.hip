// Sparse prefill attention over K/V rows kept in host memory.
//
// Page "3.14M Context on 3x 3090: The Power of an Architecture That Puts KV
// Cache in Host RAM", sections "What Needs to Stay in VRAM" (K and V live in
// host RAM) and "The Downside to Keep in Mind": during prefill every token of
// a chunk picks its own tokens, so together they touch almost the whole
// history; fetching picks token by token would move the history once per
// token.  The loops are swapped: the history is cut into fixed-size chunks,
// each copied once from host memory into a small device working buffer, every
// query takes its picked rows inside that chunk, and the partial softmax
// results are merged chunk after chunk.  The bytes crossing the host link
// are the history once, whatever the buffer size.
//
// Per call: reset of the running state, then per chunk one DMA copy of its K
// rows and one of its V rows into one half of the buffer and one kernel, then
// the normalisation.  Copies run on a copy stream of the library's own and
// kernels on the caller's stream, ordered by events: the copy of chunk i + 1
// overlaps the kernel of chunk i, and a half is refilled only after the
// kernel that read it (chunk i - 2) has finished.
//
// prefill_chunk_kernel: one wave per (query, KV head).  The query's rows in
// [c0, c1) are found by a 64-way search of its ascending list (two rounds for
// lists up to 4096); then batches of 8 rows: every lane holds D/64 dims of K
// and V of each row and of the G query heads, the dots are summed over the
// wave (xor butterfly), and the running (max, sum, accumulator) of each query
// head is updated in base 2 and kept in the workspace between chunks.
#include "keys_common.h"

#include <algorithm>
#include <mutex>

namespace skv {
namespace {

constexpr int kPfRows = 8;                  // rows per batch
constexpr float kLog2eP = 1.4426950408889634f;
enum { PF_F16 = 0, PF_BF16 = 1 };

template <int T>
__device__ __forceinline__ float elem_to_float(uint16_t v) {
  if constexpr (T == PF_BF16) return bf16_bits_to_float(v);
  else return half_bits_to_float(v);
}

// sum over the 64 lanes, in every lane: DPP butterfly within each row of 16,
// then the four row sums
__device__ __forceinline__ float wave_sum_f(float x) {
  x += __uint_as_float(dpp_u32<0xB1>(__float_as_uint(x)));    // quad xor 1
  x += __uint_as_float(dpp_u32<0x4E>(__float_as_uint(x)));    // quad xor 2
  x += __uint_as_float(dpp_u32<0x141>(__float_as_uint(x)));   // half-row mirror
  x += __uint_as_float(dpp_u32<0x140>(__float_as_uint(x)));   // row mirror
  return (__int_as_float(__builtin_amdgcn_readlane(__float_as_int(x), 0)) +
          __int_as_float(__builtin_amdgcn_readlane(__float_as_int(x), 16))) +
         (__int_as_float(__builtin_amdgcn_readlane(__float_as_int(x), 32)) +
          __int_as_float(__builtin_amdgcn_readlane(__float_as_int(x), 48)));
}

// first index in list[0, n) whose value is >= x (list ascending); the whole
// wave takes part, each round narrows the range 64-fold
__device__ __forceinline__ int wave_lower_bound(const int32_t* list, int n, int x, int lane) {
  int a = 0, b = n;   // the answer lies in [a, b]
  while (b > a) {
    const int s = (b - a + 63) / 64;
    const int e = a + lane * s;
    const bool lt = e < b && list[e] < x;
    const int c = __popcll(__ballot(lt));   // lanes 0 .. c-1 sampled values below x
    if (c == 0) {
      b = a;
    } else {
      const int last = a + (c - 1) * s;     // below x
      a = last + 1;
      b = min(b, last + s);                 // the next sample (if any) is >= x
    }
  }
  return a;
}

__global__ void prefill_reset_kernel(float* __restrict__ ml, float* __restrict__ acc, int64_t n_heads,
                                     int D) {
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n_heads * D; i += stride) {
    acc[i] = 0.0f;
    if (i < n_heads) {
      ml[2 * i] = -__builtin_inff();
      ml[2 * i + 1] = 0.0f;
    }
  }
}

template <int ET, int D, int GM>   // GM: query heads per KV head, at most (8 or 16)
__global__ __launch_bounds__(64) void prefill_chunk_kernel(
    const uint16_t* __restrict__ q, const int32_t* __restrict__ idx, const int32_t* __restrict__ n_sel,
    int cap, const uint16_t* __restrict__ kbuf, const uint16_t* __restrict__ vbuf, int c0, int c1,
    int last, float scale_log2, int Hq, int Hkv, float* __restrict__ ml, float* __restrict__ acc,
    uint32_t* __restrict__ flags) {
  constexpr int DL = D / 64;   // dims per lane
  const int p = blockIdx.x, h = blockIdx.y, lane = threadIdx.x;
  const int G = Hq / Hkv;
  int n = n_sel[p];
  if (n < 0 || n > cap) {
    if (lane == 0 && c0 == 0) raise_flag(flags, SKV_FLAG_INDEX_RANGE);
    n = n < 0 ? 0 : cap;
  }
  const int32_t* list = idx + (size_t)p * cap;
  const int lo = wave_lower_bound(list, n, c0, lane);
  const int hi = wave_lower_bound(list, n, c1, lane);
  // positions below 0 (seen by the first chunk) or at / past the end (seen by
  // the last) belong to no chunk
  if (lane == 0 && h == 0 && ((c0 == 0 && lo > 0) || (last && hi < n)))
    raise_flag(flags, SKV_FLAG_INDEX_RANGE);
  if (hi <= lo) return;   // no picked row in this chunk (wave-uniform)

  const size_t head0 = (size_t)p * Hq + (size_t)h * G;   // first query head of this KV head
  float qv[GM][DL], m[GM], l[GM], o[GM][DL];
#pragma unroll
  for (int g = 0; g < GM; ++g) {
    if (g < G) {
#pragma unroll
      for (int e = 0; e < DL; ++e) {
        qv[g][e] = elem_to_float<ET>(q[(head0 + g) * D + lane * DL + e]) * scale_log2;
        o[g][e] = acc[(head0 + g) * D + lane * DL + e];
      }
      m[g] = ml[2 * (head0 + g)];
      l[g] = ml[2 * (head0 + g) + 1];
    }
  }
  const int rows = c1 - c0;
  for (int r0 = lo; r0 < hi; r0 += kPfRows) {
    float kf[kPfRows][DL], vf[kPfRows][DL];
    bool ok[kPfRows];
#pragma unroll
    for (int u = 0; u < kPfRows; ++u) {
      const int t = list[min(r0 + u, hi - 1)] - c0;   // row inside the buffer
      ok[u] = r0 + u < hi && t >= 0 && t < rows;      // an unsorted list can point outside
      const size_t off = ((size_t)(ok[u] ? t : 0) * Hkv + h) * D + lane * DL;
#pragma unroll
      for (int e = 0; e < DL; ++e) {
        kf[u][e] = elem_to_float<ET>(kbuf[off + e]);
        vf[u][e] = elem_to_float<ET>(vbuf[off + e]);
      }
    }
    if (lane == 0) {
#pragma unroll
      for (int u = 0; u < kPfRows; ++u)
        if (r0 + u < hi && !ok[u]) raise_flag(flags, SKV_FLAG_INDEX_RANGE);
    }
#pragma unroll
    for (int g = 0; g < GM; ++g) {
      if (g >= G) continue;
      float s[kPfRows], mb = -__builtin_inff();
#pragma unroll
      for (int u = 0; u < kPfRows; ++u) {
        float part = 0.0f;
#pragma unroll
        for (int e = 0; e < DL; ++e) part += qv[g][e] * kf[u][e];
        s[u] = wave_sum_f(part);
        mb = ok[u] ? fmaxf(mb, s[u]) : mb;
      }
      if (mb == -__builtin_inff()) continue;   // no valid row in the batch
      const float mn = fmaxf(m[g], mb);
      const float alpha = exp2f(m[g] - mn);     // 0 while the running max is -inf
      float lsum = 0.0f, ov[DL];
#pragma unroll
      for (int e = 0; e < DL; ++e) ov[e] = 0.0f;
#pragma unroll
      for (int u = 0; u < kPfRows; ++u) {
        const float w = ok[u] ? exp2f(s[u] - mn) : 0.0f;
        lsum += w;
#pragma unroll
        for (int e = 0; e < DL; ++e) ov[e] += w * vf[u][e];
      }
      l[g] = l[g] * alpha + lsum;
#pragma unroll
      for (int e = 0; e < DL; ++e) o[g][e] = o[g][e] * alpha + ov[e];
      m[g] = mn;
    }
  }
#pragma unroll
  for (int g = 0; g < GM; ++g) {
    if (g < G) {
#pragma unroll
      for (int e = 0; e < DL; ++e) acc[(head0 + g) * D + lane * DL + e] = o[g][e];
      if (lane == 0) {
        ml[2 * (head0 + g)] = m[g];
        ml[2 * (head0 + g) + 1] = l[g];
      }
    }
  }
}

__global__ void prefill_finish_kernel(const float* __restrict__ ml, const float* __restrict__ acc,
                                      float* __restrict__ out, int64_t n_heads, int D) {
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n_heads * D; i += stride) {
    const float l = ml[2 * (i / D) + 1];
    out[i] = l > 0.0f ? acc[i] / l : 0.0f;
  }
}

}  // namespace

size_t prefill_workspace_bytes(const skv_layer_desc& d, int n_query) {
  const size_t nh = (size_t)n_query * d.n_q_heads;
  return 256 + align_up(nh * 2 * 4, 256) + align_up(nh * (size_t)d.head_dim * 4, 256);
}

// tokens per chunk: the buffer holds two chunks (K and V rows of each)
size_t prefill_chunk_tokens(const skv_layer_desc& d, size_t chunk_bytes) {
  return chunk_bytes / (2 * 2 * (size_t)d.n_kv_heads * d.head_dim * 2);
}

namespace {
// per device: the copy stream and the events that order it against the
// caller's stream (created on first use, kept until the process ends)
struct PrefillStreams {
  hipStream_t copy = nullptr;
  hipEvent_t start = nullptr, copied[2] = {nullptr, nullptr}, done[2] = {nullptr, nullptr};
};
constexpr int kMaxDevices = 64;
PrefillStreams g_pf[kMaxDevices];
std::mutex g_pf_mu;

hipError_t prefill_streams(PrefillStreams** out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  PrefillStreams& r = g_pf[dev];
  if (!r.copy) {
    e = hipStreamCreateWithFlags(&r.copy, hipStreamNonBlocking);
    hipEvent_t* evs[5] = {&r.start, &r.copied[0], &r.copied[1], &r.done[0], &r.done[1]};
    for (int i = 0; i < 5 && e == hipSuccess; ++i) e = hipEventCreateWithFlags(evs[i], hipEventDisableTiming);
    if (e != hipSuccess) return e;
  }
  *out = &r;
  return hipSuccess;
}
}  // namespace

hipError_t launch_prefill(const skv_layer_desc& d, int n_query, const void* q, const int32_t* idx,
                          const int32_t* n_sel, int cap, const void* host_k, const void* host_v,
                          int64_t n_tokens, void* chunk_buf, size_t chunk_bytes, float sm_scale,
                          float* out, void* ws, hipStream_t st) {
  const int D = d.head_dim, Hkv = d.n_kv_heads, Hq = d.n_q_heads;
  const int64_t nh = (int64_t)n_query * Hq;
  uint32_t* flags = reinterpret_cast<uint32_t*>(ws);
  float* ml = reinterpret_cast<float*>(reinterpret_cast<char*>(ws) + 256);
  float* acc = reinterpret_cast<float*>(reinterpret_cast<char*>(ws) + 256 + align_up((size_t)nh * 8, 256));
  const int64_t C = (int64_t)prefill_chunk_tokens(d, chunk_bytes);
  const size_t row_bytes = (size_t)Hkv * D * 2;   // one token's K (or V) rows
  uint16_t* kbuf = reinterpret_cast<uint16_t*>(chunk_buf);   // [2 halves][K rows, V rows] of C tokens
  const int fill_blocks = (int)std::min<int64_t>((nh * D + 255) / 256, 4096);
  std::lock_guard<std::mutex> lock(g_pf_mu);   // the copy stream and events are shared per device
  PrefillStreams* ps = nullptr;
  hipError_t e = prefill_streams(&ps);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(prefill_reset_kernel, dim3(fill_blocks), dim3(256), 0, st, ml, acc, nh, D);
  e = hipGetLastError();
  // copies start after the work already on the caller's stream (which may
  // still read this buffer)
  if (e == hipSuccess) e = hipEventRecord(ps->start, st);
  if (e == hipSuccess) e = hipStreamWaitEvent(ps->copy, ps->start, 0);
  const bool bf = d.kv_dtype == SKV_KV_BF16;
  const float sl = sm_scale * kLog2eP;
  int64_t i = 0;
  for (int64_t c0 = 0; c0 < n_tokens && e == hipSuccess; c0 += C, ++i) {
    const int64_t c1 = std::min<int64_t>(n_tokens, c0 + C);
    const size_t bytes = (size_t)(c1 - c0) * row_bytes;
    const int half = (int)(i & 1);
    uint16_t* kh = kbuf + (size_t)half * 2 * C * (row_bytes / 2);
    uint16_t* vh = kh + (size_t)C * (row_bytes / 2);
    // refill this half once the kernel of chunk i - 2 has read it
    if (i >= 2) e = hipStreamWaitEvent(ps->copy, ps->done[half], 0);
    if (e == hipSuccess)
      e = hipMemcpyAsync(kh, reinterpret_cast<const char*>(host_k) + (size_t)c0 * row_bytes, bytes,
                         hipMemcpyHostToDevice, ps->copy);
    if (e == hipSuccess)
      e = hipMemcpyAsync(vh, reinterpret_cast<const char*>(host_v) + (size_t)c0 * row_bytes, bytes,
                         hipMemcpyHostToDevice, ps->copy);
    if (e == hipSuccess) e = hipEventRecord(ps->copied[half], ps->copy);
    if (e == hipSuccess) e = hipStreamWaitEvent(st, ps->copied[half], 0);
    if (e != hipSuccess) break;
    const dim3 grid(n_query, Hkv);
#define SKV_PF(ET, DD, GG)                                                                         \
  hipLaunchKernelGGL((prefill_chunk_kernel<ET, DD, GG>), grid, dim3(64), 0, st, (const uint16_t*)q,  \
                     idx, n_sel, cap, kh, vh, (int)c0, (int)c1, (int)(c1 == n_tokens), sl, Hq, Hkv, ml, acc, flags)
#define SKV_PF_G(ET, DD)                                                                           \
  do {                                                                                             \
    if (Hq / Hkv <= 8) SKV_PF(ET, DD, 8);                                                          \
    else SKV_PF(ET, DD, 16);                                                                       \
  } while (0)
    if (bf && D == 256) SKV_PF_G(PF_BF16, 256);
    else if (bf) SKV_PF_G(PF_BF16, 128);
    else if (D == 256) SKV_PF_G(PF_F16, 256);
    else SKV_PF_G(PF_F16, 128);
#undef SKV_PF_G
#undef SKV_PF
    e = hipGetLastError();
    if (e == hipSuccess) e = hipEventRecord(ps->done[half], st);
  }
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(prefill_finish_kernel, dim3(fill_blocks), dim3(256), 0, st, ml, acc, out, nh, D);
  return hipGetLastError();
}

}  // namespace skv
