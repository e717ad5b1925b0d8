// Stage A3: deterministic top-k per sequence, joined with sinks and tail.
//
// Page "8 agents x 250K context on two 3090s: sparse KV decode with a rank-64
// key sketch and a host-RAM tier", section "The mechanism": a deterministic
// radix select keeps the top 2048 tokens, one pick per layer shared by all
// KV heads, plus 64 sink tokens and the last 1024; short contexts run dense.
// Page "3.14M Context on 3x 3090: The Power of an Architecture That Puts KV
// Cache in Host RAM", section "Why": block mode reads the whole history until
// the context exceeds 4*block_topk+3 tokens, then exactly the budget.
//
// Order: larger key first, equal keys by lower position.  Keys are exact, so
// (key, position) is a unique composite and the kept set is unique; the
// kernels below find it without depending on workgroup scheduling.
//
// Plan per sequence (all on the caller's stream, no host decision):
//   init     zero the coarse histogram and the select state;
//   hist     many workgroups histogram a 13-bit order-preserving digit of the
//            key (fp32-rounded, so one bucket spans 1/16 of an octave); the
//            last workgroup to finish finds the bucket beta holding the k-th
//            largest key and the count n_c of keys in buckets >= beta;
//   collect  keys in buckets >= beta (all of the top k, plus the rest of
//            bucket beta -- typically a few thousand) go to a short list;
//   final    one workgroup per sequence: exact MSB-first radix select over the
//            96-bit composite (ordered key, ~position) of the list in LDS,
//            bitonic sort of the kept positions, output with sinks and tail.
// When n_c exceeds the list capacity (degenerate data, e.g. all keys equal)
// the final kernel runs the same exact radix select directly over every key
// of the sequence in global memory and compacts in position order (slow path,
// flagged as SKV_FLAG_TOPK_SLOW).
#include "skv_internal.h"

namespace skv {
namespace {

constexpr int kSelThreads = 256;
constexpr int kFinalThreads = 1024;

struct Range {
  int T, lo, n;   // candidates are keys[lo .. lo+n)
  bool dense;
  size_t stride;  // keys row stride
};

__device__ __forceinline__ Range cand_range(int mode, int T, int S, int k, int L, int max_ctx) {
  Range r;
  r.T = T;
  if (mode == SKV_INDEX_SKETCH_INT4) {
    r.stride = (size_t)max_ctx;
    r.dense = T <= S + k + L;
    r.lo = S;
    r.n = r.dense ? 0 : T - S - L;
  } else {
    r.stride = (size_t)(max_ctx / 4);
    const int nb = T / 4;
    r.dense = nb <= k;
    r.lo = 0;
    r.n = r.dense ? 0 : nb;
  }
  return r;
}

__device__ __forceinline__ double canon(double x) { return x + 0.0; }

__global__ void topk_init_kernel(uint32_t* __restrict__ hist, TopkState* __restrict__ state) {
  const int b = blockIdx.x;
  uint32_t* h = hist + (size_t)b * kHistBins;
  for (int i = threadIdx.x; i < kHistBins; i += blockDim.x) h[i] = 0u;
  if (threadIdx.x < sizeof(TopkState) / 4) reinterpret_cast<uint32_t*>(state + b)[threadIdx.x] = 0u;
}

__global__ __launch_bounds__(kSelThreads) void topk_hist_kernel(
    const double* __restrict__ keys, const int32_t* __restrict__ ctx_len,
    uint32_t* __restrict__ hist, TopkState* __restrict__ state, int mode, int max_ctx, int S,
    int k, int L) {
  __shared__ uint32_t h[kHistBins];
  __shared__ int s_last;
  const int b = blockIdx.y;
  int T = ctx_len[b];
  T = T < 0 ? 0 : (T > max_ctx ? max_ctx : T);
  const Range r = cand_range(mode, T, S, k, L, max_ctx);
  if (r.dense) return;
  const int n_chunks = (r.n + kHistChunk - 1) / kHistChunk;
  const int c = blockIdx.x;
  if (c >= n_chunks) return;
  for (int i = threadIdx.x; i < kHistBins; i += blockDim.x) h[i] = 0u;
  __syncthreads();
  const double* kb = keys + (size_t)b * r.stride + r.lo;
  const int i1 = min(r.n, (c + 1) * kHistChunk);
  for (int i = c * kHistChunk + threadIdx.x; i < i1; i += blockDim.x)
    atomicAdd(&h[key_digit(canon(kb[i]))], 1u);
  __syncthreads();
  uint32_t* gh = hist + (size_t)b * kHistBins;
  for (int i = threadIdx.x; i < kHistBins; i += blockDim.x)
    if (h[i]) atomicAdd(&gh[i], h[i]);
  __threadfence();
  __syncthreads();
  if (threadIdx.x == 0) s_last = (atomicAdd(&state[b].done, 1u) == (uint32_t)(n_chunks - 1));
  __syncthreads();
  if (!s_last) return;
  __threadfence();

  // last workgroup: bucket beta of the k-th largest key.  Thread t owns the 32
  // bins [kHistBins - 32(t+1), kHistBins - 32t); counts are summed from the top.
  constexpr int PER = kHistBins / kSelThreads;
  const int top = kHistBins - PER * threadIdx.x;
  uint32_t cnt[PER];
  uint32_t mine = 0;
#pragma unroll
  for (int j = 0; j < PER; ++j) {
    cnt[j] = __hip_atomic_load(&gh[top - 1 - j], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    mine += cnt[j];
  }
  // exclusive prefix over threads (descending bins) through LDS
  uint32_t* pre = h;  // reuse
  pre[threadIdx.x] = mine;
  __syncthreads();
  if (threadIdx.x == 0) {
    uint32_t run = 0;
    for (int t = 0; t < kSelThreads; ++t) {
      const uint32_t v = pre[t];
      pre[t] = run;
      run += v;
    }
  }
  __syncthreads();
  uint32_t cum = pre[threadIdx.x];
  const uint32_t need = (uint32_t)k;
  if (cum < need && cum + mine >= need) {
#pragma unroll
    for (int j = 0; j < PER; ++j) {
      const uint32_t nxt = cum + cnt[j];
      if (cum < need && nxt >= need) {
        state[b].beta = (uint32_t)(top - 1 - j);
        state[b].n_c = nxt;
        state[b].mode = nxt <= (uint32_t)kListCap ? kModeFast : kModeSlow;
      }
      cum = nxt;
    }
  }
}

__global__ __launch_bounds__(kSelThreads) void topk_collect_kernel(
    const double* __restrict__ keys, const int32_t* __restrict__ ctx_len,
    TopkState* __restrict__ state, uint64_t* __restrict__ lkey, uint32_t* __restrict__ lpos,
    int mode, int max_ctx, int S, int k, int L) {
  const int b = blockIdx.y;
  int T = ctx_len[b];
  T = T < 0 ? 0 : (T > max_ctx ? max_ctx : T);
  const Range r = cand_range(mode, T, S, k, L, max_ctx);
  if (r.dense) return;
  if (state[b].mode != kModeFast) return;
  const uint32_t beta = state[b].beta;
  const int c = blockIdx.x;
  const int i0 = c * kHistChunk;
  if (i0 >= r.n) return;
  const int i1 = min(r.n, i0 + kHistChunk);
  const double* kb = keys + (size_t)b * r.stride + r.lo;
  uint64_t* lk = lkey + (size_t)b * kListCap;
  uint32_t* lp = lpos + (size_t)b * kListCap;
  const int lane = threadIdx.x & 63;
  const uint64_t lt_mask = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
  for (int base = i0 + (threadIdx.x & ~63); base < i1; base += blockDim.x) {
    const int i = base + lane;
    double x = 0.0;
    bool sel = false;
    if (i < i1) {
      x = canon(kb[i]);
      sel = key_digit(x) >= beta;
    }
    const uint64_t m = __ballot(sel);
    if (m == 0) continue;
    uint32_t slot = 0;
    if (lane == 0) slot = atomicAdd(&state[b].list_count, (uint32_t)__popcll(m));
    slot = __shfl(slot, 0);
    if (sel) {
      const uint32_t at = slot + (uint32_t)__popcll(m & lt_mask);
      if (at < (uint32_t)kListCap) {
        lk[at] = ordered_u64(x);
        lp[at] = (uint32_t)(r.lo + i);
      }
    }
  }
}

// ---- exact radix select over unique 96-bit composites ----------------------
// composite = (hi: order-preserving key, lo: ~position); larger composite =
// larger key, or equal key and lower position.

__device__ __forceinline__ uint32_t comp_digit(uint64_t hi, uint32_t lo, int dg) {
  return dg >= 4 ? (uint32_t)(hi >> (8 * (dg - 4))) & 0xFFu : (lo >> (8 * dg)) & 0xFFu;
}

struct SelectShared {
  uint32_t hist[256];
  uint32_t wsum[kFinalThreads / 64];
  uint64_t pre_hi, mask_hi;
  uint32_t pre_lo, mask_lo;
  int need;
  int count;
};

// Finds the composite of the k-th largest element (0 < k <= n).  get(i) -> (hi, lo).
template <class Get>
__device__ void radix_select(Get get, int n, int k, SelectShared& sh, uint64_t& thr_hi,
                             uint32_t& thr_lo) {
  if (threadIdx.x == 0) {
    sh.pre_hi = 0;
    sh.mask_hi = 0;
    sh.pre_lo = 0;
    sh.mask_lo = 0;
    sh.need = k;
  }
  __syncthreads();
  for (int dg = 11; dg >= 0; --dg) {
    for (int i = threadIdx.x; i < 256; i += blockDim.x) sh.hist[i] = 0u;
    __syncthreads();
    const uint64_t ph = sh.pre_hi, mh = sh.mask_hi;
    const uint32_t pl = sh.pre_lo, ml = sh.mask_lo;
    for (int i = threadIdx.x; i < n; i += blockDim.x) {
      uint64_t hi;
      uint32_t lo;
      get(i, hi, lo);
      if ((hi & mh) == ph && (lo & ml) == pl) atomicAdd(&sh.hist[comp_digit(hi, lo, dg)], 1u);
    }
    __syncthreads();
    if (threadIdx.x < 64) {
      // lane l owns digits [252-4l, 255-4l], summed from the top
      const int lane = threadIdx.x;
      uint32_t c4[4];
      uint32_t s = 0;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        c4[j] = sh.hist[255 - 4 * lane - j];
        s += c4[j];
      }
      uint32_t incl = s;
#pragma unroll
      for (int off = 1; off < 64; off <<= 1) {
        const uint32_t v = __shfl_up(incl, off);
        if (lane >= off) incl += v;
      }
      const uint32_t excl = incl - s;
      const uint32_t need = (uint32_t)sh.need;
      if (excl < need && incl >= need) {
        uint32_t cum = excl;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const uint32_t nxt = cum + c4[j];
          if (cum < need && nxt >= need) {
            const uint32_t dval = (uint32_t)(255 - 4 * lane - j);
            if (dg >= 4) {
              sh.pre_hi |= (uint64_t)dval << (8 * (dg - 4));
              sh.mask_hi |= 0xFFull << (8 * (dg - 4));
            } else {
              sh.pre_lo |= dval << (8 * dg);
              sh.mask_lo |= 0xFFu << (8 * dg);
            }
            sh.need = (int)(need - cum);
          }
          cum = nxt;
        }
      }
    }
    __syncthreads();
  }
  thr_hi = sh.pre_hi;
  thr_lo = sh.pre_lo;
}

__device__ __forceinline__ bool comp_ge(uint64_t hi, uint32_t lo, uint64_t th, uint32_t tl) {
  return hi > th || (hi == th && lo >= tl);
}

__global__ __launch_bounds__(kFinalThreads) void topk_final_kernel(
    const double* __restrict__ keys, const int32_t* __restrict__ ctx_len,
    TopkState* __restrict__ state, const uint64_t* __restrict__ lkey,
    const uint32_t* __restrict__ lpos, int32_t* __restrict__ idx, int32_t* __restrict__ n_sel,
    uint32_t* __restrict__ flags, int mode, int max_ctx, int S, int k, int L, int cap) {
  __shared__ uint64_t s_key[kListCap];
  __shared__ uint32_t s_pos[kListCap];
  __shared__ uint32_t s_sel[kMaxTopk];
  __shared__ SelectShared sh;
  const int b = blockIdx.x;
  int T = ctx_len[b];
  T = T < 0 ? 0 : (T > max_ctx ? max_ctx : T);
  const Range r = cand_range(mode, T, S, k, L, max_ctx);
  int32_t* out = idx + (size_t)b * cap;
  if (r.dense) {
    for (int i = threadIdx.x; i < T; i += blockDim.x) out[i] = i;
    if (threadIdx.x == 0) n_sel[b] = T;
    return;
  }
  const int st_mode = (int)state[b].mode;
  uint64_t th;
  uint32_t tl;
  if (st_mode == kModeFast) {
    const int n = (int)min(state[b].list_count, (uint32_t)kListCap);
    for (int i = threadIdx.x; i < n; i += blockDim.x) {
      s_key[i] = lkey[(size_t)b * kListCap + i];
      s_pos[i] = lpos[(size_t)b * kListCap + i];
    }
    __syncthreads();
    radix_select([&](int i, uint64_t& hi, uint32_t& lo) { hi = s_key[i]; lo = ~s_pos[i]; }, n, k,
                 sh, th, tl);
    if (threadIdx.x == 0) sh.count = 0;
    __syncthreads();
    for (int i = threadIdx.x; i < n; i += blockDim.x)
      if (comp_ge(s_key[i], ~s_pos[i], th, tl)) {
        const int at = atomicAdd(&sh.count, 1);
        if (at < kMaxTopk) s_sel[at] = s_pos[i];
      }
    __syncthreads();
    // bitonic sort of the k kept positions (padded to a power of two)
    int P = 1;
    while (P < k) P <<= 1;
    for (int i = k + threadIdx.x; i < P; i += blockDim.x) s_sel[i] = 0xFFFFFFFFu;
    __syncthreads();
    for (int size = 2; size <= P; size <<= 1) {
      for (int stride = size >> 1; stride > 0; stride >>= 1) {
        for (int t = threadIdx.x; t < P / 2; t += blockDim.x) {
          const int pos = 2 * stride * (t / stride) + (t % stride);
          const int par = pos + stride;
          const bool asc = (pos & size) == 0;
          const uint32_t a = s_sel[pos], c = s_sel[par];
          if ((a > c) == asc) {
            s_sel[pos] = c;
            s_sel[par] = a;
          }
        }
        __syncthreads();
      }
    }
  } else {
    // slow exact path over every candidate key in global memory
    if (threadIdx.x == 0) raise_flag(flags, SKV_FLAG_TOPK_SLOW);
    const double* kb = keys + (size_t)b * r.stride + r.lo;
    const int lo0 = r.lo;
    radix_select(
        [&](int i, uint64_t& hi, uint32_t& lo) {
          hi = ordered_u64(canon(kb[i]));
          lo = ~(uint32_t)(lo0 + i);
        },
        r.n, k, sh, th, tl);
    // ordered compaction: positions come out ascending
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const uint64_t lt_mask = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
    if (threadIdx.x == 0) sh.count = 0;
    __syncthreads();
    for (int base = 0; base < r.n; base += blockDim.x) {
      const int i = base + threadIdx.x;
      bool sel = false;
      if (i < r.n) sel = comp_ge(ordered_u64(canon(kb[i])), ~(uint32_t)(lo0 + i), th, tl);
      const uint64_t m = __ballot(sel);
      if (lane == 0) sh.wsum[wave] = (uint32_t)__popcll(m);
      __syncthreads();
      uint32_t off = (uint32_t)sh.count;
      for (int w = 0; w < wave; ++w) off += sh.wsum[w];
      const uint32_t at = off + (uint32_t)__popcll(m & lt_mask);
      if (sel && at < (uint32_t)kMaxTopk) s_sel[at] = (uint32_t)(lo0 + i);
      __syncthreads();
      if (threadIdx.x == 0) {
        uint32_t tot = 0;
        for (int w = 0; w < (int)(blockDim.x >> 6); ++w) tot += sh.wsum[w];
        sh.count += (int)tot;
      }
      __syncthreads();
    }
  }
  __syncthreads();
  // output: ascending unique positions
  if (mode == SKV_INDEX_SKETCH_INT4) {
    for (int i = threadIdx.x; i < S; i += blockDim.x) out[i] = i;
    for (int i = threadIdx.x; i < k; i += blockDim.x) out[S + i] = (int32_t)s_sel[i];
    for (int i = threadIdx.x; i < L; i += blockDim.x) out[S + k + i] = T - L + i;
    if (threadIdx.x == 0) n_sel[b] = S + k + L;
  } else {
    for (int i = threadIdx.x; i < 4 * k; i += blockDim.x) out[i] = 4 * (int32_t)s_sel[i >> 2] + (i & 3);
    const int nb = T / 4;
    for (int i = threadIdx.x; i < T - 4 * nb; i += blockDim.x) out[4 * k + i] = 4 * nb + i;
    if (threadIdx.x == 0) n_sel[b] = 4 * k + (T - 4 * nb);
  }
}

}  // namespace

hipError_t launch_topk(const skv_layer_desc& d, const int32_t* ctx_len, const double* keys,
                       int32_t* idx, int32_t* n_sel, void* ws, const WsLayout& Lw,
                       hipStream_t st) {
  uint32_t* flags = ws_ptr<uint32_t>(ws, Lw.flags);
  uint32_t* hist = ws_ptr<uint32_t>(ws, Lw.hist);
  TopkState* state = ws_ptr<TopkState>(ws, Lw.state);
  uint64_t* lkey = ws_ptr<uint64_t>(ws, Lw.lkey);
  uint32_t* lpos = ws_ptr<uint32_t>(ws, Lw.lpos);
  const int mode = d.index_mode;
  const int max_cand = mode == SKV_INDEX_SKETCH_INT4 ? d.max_ctx : d.max_ctx / 4;
  const int nchunk = (max_cand + kHistChunk - 1) / kHistChunk;
  const dim3 grid(nchunk > 0 ? nchunk : 1, d.batch);
  const int S = mode == SKV_INDEX_SKETCH_INT4 ? d.n_sink : 0;
  const int L = mode == SKV_INDEX_SKETCH_INT4 ? d.n_tail : 0;
  hipLaunchKernelGGL(topk_init_kernel, dim3(d.batch), dim3(256), 0, st, hist, state);
  hipLaunchKernelGGL(topk_hist_kernel, grid, dim3(kSelThreads), 0, st, keys, ctx_len, hist, state,
                     mode, d.max_ctx, S, d.topk, L);
  hipLaunchKernelGGL(topk_collect_kernel, grid, dim3(kSelThreads), 0, st, keys, ctx_len, state,
                     lkey, lpos, mode, d.max_ctx, S, d.topk, L);
  hipLaunchKernelGGL(topk_final_kernel, dim3(d.batch), dim3(kFinalThreads), 0, st, keys, ctx_len,
                     state, lkey, lpos, idx, n_sel, flags, mode, d.max_ctx, S, d.topk, L,
                     select_capacity(d));
  return hipGetLastError();
}

}  // namespace skv
