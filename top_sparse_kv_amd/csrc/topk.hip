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
// Three kernels, none of which uses a global atomic (same-address atomics
// from many workgroups serialise in the memory system):
//   sample   one workgroup per sequence histograms a 12-bit order-preserving
//            digit of a strided sample of the keys (the digit is the key
//            rounded to fp32, so one bucket spans 1/8 of an octave) and picks
//            the bucket beta above which the sample predicts, with a margin,
//            at least k keys;
//   collect  workgroups of 2048 keys write the keys with digit >= beta into a
//            segment of their own (at most kSegCap) and their count;
//   final    one workgroup per sequence gathers the segments into LDS and runs
//            an exact MSB-first radix select over the 96-bit composite
//            (ordered key, ~position), stopping once the remaining bucket is
//            kept whole; the kept positions are marked in an LDS bitmap and
//            read back in order.
// If the candidates cannot be used (a segment overflowed, fewer than k or more
// than the LDS list holds -- degenerate data such as all-equal keys), the
// final kernel runs the same exact radix select over every key of the
// sequence in global memory and compacts in position order (slow path,
// flagged as SKV_FLAG_TOPK_SLOW).  The sample only affects speed, never the
// result.
#include "select_common.h"

namespace skv {
namespace {

constexpr int kSelThreads = 256;
constexpr int kFinalThreads = 1024;
constexpr int kKeysPerThread = kHistChunk / kSelThreads;   // 8
constexpr int kMaxSeg = 1024;                              // segments per sequence

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

__device__ __forceinline__ int ctx_of(const int32_t* ctx_len, int b, int max_ctx) {
  int T = ctx_len[b];
  return T < 0 ? 0 : (T > max_ctx ? max_ctx : T);
}

__device__ __forceinline__ double canon(double x) { return x + 0.0; }

// The sample is whole 16-key lines (128 B) taken every s lines: about 8k
// samples per sequence, every key (an exact histogram) when short.
constexpr int kLineKeys = 16;
__device__ __forceinline__ int sample_stride(int n, int k) {
  int s = n / (8 * k);
  return s < 1 ? 1 : (s > 16 ? 16 : s);
}

__global__ __launch_bounds__(kFinalThreads) void topk_sample_kernel(
    const double* __restrict__ keys, const int32_t* __restrict__ ctx_len,
    TopkState* __restrict__ state, int mode, int max_ctx, int S, int k, int L) {
  constexpr int PER = kHistBins / kFinalThreads;   // 4 bins per thread
  constexpr int UNR = 16;
  __shared__ uint32_t h[kHistBins];
  __shared__ uint32_t wsum[16];
  const int b = blockIdx.x;
  const Range r = cand_range(mode, ctx_of(ctx_len, b, max_ctx), S, k, L, max_ctx);
  if (r.dense) return;
  const int s = sample_stride(r.n, k);
  const int lines = (r.n + kLineKeys - 1) / kLineKeys;
  const int nsl = (lines + s - 1) / s;               // sampled lines
  const int nj = nsl * kLineKeys;                    // sample slots
  for (int i = threadIdx.x; i < kHistBins; i += blockDim.x) h[i] = 0u;
  __syncthreads();
  const double* kb = keys + (size_t)b * r.stride + r.lo;
  uint32_t taken = 0;
  for (int j0 = 0; j0 < nj; j0 += UNR * kFinalThreads) {
    double x[UNR];
    bool ok[UNR];
#pragma unroll
    for (int u = 0; u < UNR; ++u) {
      const int j = j0 + u * kFinalThreads + threadIdx.x;
      const int i = (j / kLineKeys) * s * kLineKeys + (j % kLineKeys);
      ok[u] = j < nj && i < r.n;
      x[u] = kb[ok[u] ? i : 0];     // unconditional load: all in flight together
    }
#pragma unroll
    for (int u = 0; u < UNR; ++u)
      if (ok[u]) {
        atomicAdd(&h[key_digit(canon(x[u]))], 1u);
        ++taken;
      }
  }
  __syncthreads();
  // samples needed above beta: exactly k when every key is sampled, else the
  // expected share of the top k plus 25% and four standard deviations
  uint32_t need;
  if (s == 1) {
    need = (uint32_t)k;
  } else {
    const float e = (float)k * (float)nsl / (float)lines;
    need = (uint32_t)ceilf(1.25f * e + 4.0f * sqrtf(e) + 8.0f);
  }
  (void)taken;
  const int top = kHistBins - PER * threadIdx.x;
  uint32_t cnt[PER];
  uint32_t mine = 0;
#pragma unroll
  for (int j = 0; j < PER; ++j) {
    cnt[j] = h[top - 1 - j];
    mine += cnt[j];
  }
  uint32_t total = 0;
  uint32_t cum = block_excl_scan(mine, wsum, &total);
  if (threadIdx.x == 0 && total < need) state[b].beta = 0u;   // keep everything
  if (cum < need && cum + mine >= need) {
#pragma unroll
    for (int j = 0; j < PER; ++j) {
      const uint32_t nxt = cum + cnt[j];
      if (cum < need && nxt >= need) state[b].beta = (uint32_t)(top - 1 - j);
      cum = nxt;
    }
  }
}

__global__ __launch_bounds__(kSelThreads) void topk_collect_kernel(
    const double* __restrict__ keys, const int32_t* __restrict__ ctx_len,
    const TopkState* __restrict__ state, uint32_t* __restrict__ segcnt,
    uint64_t* __restrict__ lkey, uint32_t* __restrict__ lpos, int n_seg, int mode, int max_ctx,
    int S, int k, int L) {
  __shared__ uint32_t wsum[16];
  const int b = blockIdx.y;
  const Range r = cand_range(mode, ctx_of(ctx_len, b, max_ctx), S, k, L, max_ctx);
  if (r.dense) return;
  const int c = blockIdx.x;
  const int i0 = c * kHistChunk;
  if (i0 >= r.n) return;
  const uint32_t beta = state[b].beta;
  const double* kb = keys + (size_t)b * r.stride + r.lo;
  const size_t seg = ((size_t)b * n_seg + c) * kSegCap;
  double x[kKeysPerThread];
#pragma unroll
  for (int u = 0; u < kKeysPerThread; ++u) {
    const int i = i0 + u * kSelThreads + threadIdx.x;
    x[u] = canon(kb[min(i, r.n - 1)]);   // unconditional load
  }
  uint32_t mine = 0;
  uint32_t selm = 0;
#pragma unroll
  for (int u = 0; u < kKeysPerThread; ++u) {
    const int i = i0 + u * kSelThreads + threadIdx.x;
    if (i < r.n && key_digit(x[u]) >= beta) {
      selm |= 1u << u;
      ++mine;
    }
  }
  uint32_t total = 0;
  uint32_t at = block_excl_scan(mine, wsum, &total);
#pragma unroll
  for (int u = 0; u < kKeysPerThread; ++u) {
    if (selm & (1u << u)) {
      if (at < (uint32_t)kSegCap) {
        lkey[seg + at] = ordered_u64(x[u]);
        lpos[seg + at] = (uint32_t)(r.lo + i0 + u * kSelThreads + threadIdx.x);
      }
      ++at;
    }
  }
  if (threadIdx.x == 0) segcnt[(size_t)b * n_seg + c] = total;
}

// ---- exact radix select over unique 96-bit composites ----------------------
// composite = (hi: order-preserving key, lo: ~position); larger composite =
// larger key, or equal key and lower position.

__device__ __forceinline__ uint32_t comp_digit(uint64_t hi, uint32_t lo, int dg) {
  return dg >= 4 ? (uint32_t)(hi >> (8 * (dg - 4))) & 0xFFu : (lo >> (8 * dg)) & 0xFFu;
}

struct SelectShared {
  uint32_t hist[256];
  uint32_t wsum[16];
  uint32_t and3[3], or3[3];
  uint64_t pre_hi, mask_hi;
  uint32_t pre_lo, mask_lo;
  int need;
  int done;
  int count;
  int fast;
  int total;
};

// MSB-first radix select of the k largest composites among n (0 < k <= n).
// On return every element with (hi & mask_hi, lo & mask_lo) lexicographically
// >= (pre_hi, pre_lo) is kept, and exactly k elements satisfy that.  The loop
// stops once the remaining bucket is kept whole.  get(i, hi, lo) reads element i.
template <class Get>
__device__ void radix_select(Get get, int n, int k, SelectShared& sh) {
  // bytes on which all n composites agree are fixed without a histogram pass
  uint32_t a0 = ~0u, a1 = ~0u, a2 = ~0u, o0 = 0u, o1 = 0u, o2 = 0u;
  for (int i = threadIdx.x; i < n; i += blockDim.x) {
    uint64_t hi;
    uint32_t lo;
    get(i, hi, lo);
    a0 &= (uint32_t)(hi >> 32); o0 |= (uint32_t)(hi >> 32);
    a1 &= (uint32_t)hi;         o1 |= (uint32_t)hi;
    a2 &= lo;                   o2 |= lo;
  }
  if (threadIdx.x == 0) {
    sh.and3[0] = sh.and3[1] = sh.and3[2] = ~0u;
    sh.or3[0] = sh.or3[1] = sh.or3[2] = 0u;
    sh.pre_hi = 0;
    sh.mask_hi = 0;
    sh.pre_lo = 0;
    sh.mask_lo = 0;
    sh.need = k;
    sh.done = (k == n);
  }
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    a0 &= __shfl_xor(a0, off); a1 &= __shfl_xor(a1, off); a2 &= __shfl_xor(a2, off);
    o0 |= __shfl_xor(o0, off); o1 |= __shfl_xor(o1, off); o2 |= __shfl_xor(o2, off);
  }
  __syncthreads();
  if ((threadIdx.x & 63) == 0) {
    atomicAnd(&sh.and3[0], a0); atomicAnd(&sh.and3[1], a1); atomicAnd(&sh.and3[2], a2);
    atomicOr(&sh.or3[0], o0);   atomicOr(&sh.or3[1], o1);   atomicOr(&sh.or3[2], o2);
  }
  __syncthreads();
  int dg0 = 11;
  {
    const uint64_t ahi = ((uint64_t)sh.and3[0] << 32) | sh.and3[1];
    const uint64_t ohi = ((uint64_t)sh.or3[0] << 32) | sh.or3[1];
    const uint32_t alo = sh.and3[2], olo = sh.or3[2];
    uint64_t ph = 0, mh = 0;
    uint32_t pl = 0, ml = 0;
    while (dg0 >= 0 && n > 0) {
      const uint32_t da = comp_digit(ahi, alo, dg0), dor = comp_digit(ohi, olo, dg0);
      if (da != dor) break;
      if (dg0 >= 4) {
        ph |= (uint64_t)da << (8 * (dg0 - 4));
        mh |= 0xFFull << (8 * (dg0 - 4));
      } else {
        pl |= da << (8 * dg0);
        ml |= 0xFFu << (8 * dg0);
      }
      --dg0;
    }
    __syncthreads();
    if (threadIdx.x == 0) {
      sh.pre_hi = ph;
      sh.mask_hi = mh;
      sh.pre_lo = pl;
      sh.mask_lo = ml;
    }
    __syncthreads();
  }
  for (int dg = dg0; dg >= 0 && !sh.done; --dg) {
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
            sh.done = (need - cum) == c4[j];
          }
          cum = nxt;
        }
      }
    }
    __syncthreads();
  }
}

__device__ __forceinline__ bool kept(uint64_t hi, uint32_t lo, const SelectShared& sh) {
  const uint64_t h = hi & sh.mask_hi;
  return h > sh.pre_hi || (h == sh.pre_hi && (lo & sh.mask_lo) >= sh.pre_lo);
}

// Output slot of the rank-th kept candidate (ascending): token mode after the
// sinks; block mode as the 4 tokens of the block.
__device__ __forceinline__ void emit_position(int32_t* out, int mode, int S, int rank, int pos) {
  if (mode == SKV_INDEX_SKETCH_INT4) {
    out[S + rank] = pos;
  } else {
#pragma unroll
    for (int j = 0; j < 4; ++j) out[4 * rank + j] = 4 * pos + j;
  }
}

__global__ __launch_bounds__(kFinalThreads) void topk_final_kernel(
    const double* __restrict__ keys, const int32_t* __restrict__ ctx_len,
    const uint32_t* __restrict__ segcnt, const uint64_t* __restrict__ lkey,
    const uint32_t* __restrict__ lpos, int32_t* __restrict__ idx, int32_t* __restrict__ n_sel,
    uint32_t* __restrict__ flags, int n_seg, int mode, int max_ctx, int S, int k, int L, int cap) {
  __shared__ uint64_t s_key[kListCap];
  __shared__ uint32_t s_pos[kListCap];
  __shared__ uint32_t s_bm[kBitmapWords];
  __shared__ uint32_t s_off[kMaxSeg + 1];
  __shared__ SelectShared sh;
  const int b = blockIdx.x;
  const int T = ctx_of(ctx_len, b, max_ctx);
  const Range r = cand_range(mode, T, S, k, L, max_ctx);
  int32_t* out = idx + (size_t)b * cap;
  if (r.dense) {
    for (int i = threadIdx.x; i < T; i += blockDim.x) out[i] = i;
    if (threadIdx.x == 0) n_sel[b] = T;
    return;
  }
  // sinks / tail / partial block
  if (mode == SKV_INDEX_SKETCH_INT4) {
    for (int i = threadIdx.x; i < S; i += blockDim.x) out[i] = i;
    for (int i = threadIdx.x; i < L; i += blockDim.x) out[S + k + i] = T - L + i;
    if (threadIdx.x == 0) n_sel[b] = S + k + L;
  } else {
    const int nb = T / 4;
    for (int i = threadIdx.x; i < T - 4 * nb; i += blockDim.x) out[4 * k + i] = 4 * nb + i;
    if (threadIdx.x == 0) n_sel[b] = 4 * k + (T - 4 * nb);
  }
  // gather the segment counts; the candidates are usable when no segment
  // overflowed and there are between k and kListCap of them
  const int n_parts = (r.n + kHistChunk - 1) / kHistChunk;
  const int words = (r.n + 31) / 32;
  {
    const int per = (n_parts + blockDim.x - 1) / blockDim.x;   // 1 unless n_parts > 1024
    uint32_t mine = 0;
    int over = 0;
    for (int j = 0; j < per; ++j) {
      const int c = threadIdx.x * per + j;
      if (c < n_parts) {
        const uint32_t v = segcnt[(size_t)b * n_seg + c];
        over |= v > (uint32_t)kSegCap;
        mine += v;
      }
    }
    if (threadIdx.x == 0) sh.fast = 1;
    uint32_t total = 0;
    uint32_t off = block_excl_scan(mine, sh.wsum, &total);
    if (over) sh.fast = 0;
    for (int j = 0; j < per; ++j) {
      const int c = threadIdx.x * per + j;
      if (c < n_parts && c <= kMaxSeg) {
        s_off[c] = off;
        off += min(segcnt[(size_t)b * n_seg + c], (uint32_t)kSegCap);
      }
    }
    if (threadIdx.x == 0) {
      s_off[min(n_parts, kMaxSeg)] = total;
      sh.total = (int)total;
    }
    __syncthreads();
    if (threadIdx.x == 0 && (total < (uint32_t)k || total > (uint32_t)kListCap || words > kBitmapWords ||
                             n_parts > kMaxSeg))
      sh.fast = 0;
    __syncthreads();
  }
  if (sh.fast) {
    const int n = sh.total;
    // 8 threads per segment, each moving up to kSegCap/8 entries with
    // unconditional loads (clamped into the segment) so they overlap
    constexpr int TPS = 8, PER = kSegCap / TPS;
    for (int c = threadIdx.x / TPS; c < n_parts; c += blockDim.x / TPS) {
      const int cnt = (int)(s_off[c + 1] - s_off[c]);   // s_off[n_parts] holds the total
      const size_t base = ((size_t)b * n_seg + c) * kSegCap;
      uint64_t kk[PER];
      uint32_t pp[PER];
#pragma unroll
      for (int j = 0; j < PER; ++j) {
        const int e = (threadIdx.x % TPS) + TPS * j;
        const int ec = e < cnt ? e : 0;
        kk[j] = lkey[base + ec];
        pp[j] = lpos[base + ec];
      }
#pragma unroll
      for (int j = 0; j < PER; ++j) {
        const int e = (threadIdx.x % TPS) + TPS * j;
        if (e < cnt) {
          s_key[s_off[c] + e] = kk[j];
          s_pos[s_off[c] + e] = pp[j];
        }
      }
    }
    for (int w = threadIdx.x; w < words; w += blockDim.x) s_bm[w] = 0u;
    __syncthreads();
    radix_select([&](int i, uint64_t& hi, uint32_t& lo) { hi = s_key[i]; lo = ~s_pos[i]; }, n, k, sh);
    for (int i = threadIdx.x; i < n; i += blockDim.x)
      if (kept(s_key[i], ~s_pos[i], sh)) {
        const int ci = (int)s_pos[i] - r.lo;
        atomicOr(&s_bm[ci >> 5], 1u << (ci & 31));
      }
    __syncthreads();
    // read the bitmap back in order: thread t owns a contiguous run of words
    const int per = (words + blockDim.x - 1) / blockDim.x;
    const int w0 = threadIdx.x * per;
    const int w1 = min(words, w0 + per);
    uint32_t cnt = 0;
    for (int w = w0; w < w1; ++w) cnt += (uint32_t)__popc(s_bm[w]);
    int rank = (int)block_excl_scan(cnt, sh.wsum, nullptr);
    for (int w = w0; w < w1; ++w) {
      uint32_t bits = s_bm[w];
      while (bits) {
        const int bit = __ffs(bits) - 1;
        bits &= bits - 1;
        if (rank < k) emit_position(out, mode, S, rank, r.lo + 32 * w + bit);
        ++rank;
      }
    }
    return;
  }
  // exact path over every candidate key in global memory
  if (threadIdx.x == 0) raise_flag(flags, SKV_FLAG_TOPK_SLOW);
  const double* kb = keys + (size_t)b * r.stride + r.lo;
  const int lo0 = r.lo;
  radix_select(
      [&](int i, uint64_t& hi, uint32_t& lo) {
        hi = ordered_u64(canon(kb[i]));
        lo = ~(uint32_t)(lo0 + i);
      },
      r.n, k, sh);
  // ordered compaction: positions come out ascending
  if (threadIdx.x == 0) sh.count = 0;
  __syncthreads();
  for (int base = 0; base < r.n; base += blockDim.x) {
    const int i = base + threadIdx.x;
    const bool sel = i < r.n && kept(ordered_u64(canon(kb[i])), ~(uint32_t)(lo0 + i), sh);
    const int before = sh.count;
    const int off = (int)block_excl_scan(sel ? 1u : 0u, sh.wsum, nullptr);
    if (sel && before + off < k) emit_position(out, mode, S, before + off, lo0 + i);
    __syncthreads();
    if (threadIdx.x == blockDim.x - 1) sh.count = before + off + (sel ? 1 : 0);
    __syncthreads();
  }
}

}  // namespace

hipError_t launch_topk(const skv_layer_desc& d, const int32_t* ctx_len, const double* keys,
                       int32_t* idx, int32_t* n_sel, void* ws, const WsLayout& Lw,
                       hipStream_t st) {
  uint32_t* flags = ws_ptr<uint32_t>(ws, Lw.flags);
  TopkState* state = ws_ptr<TopkState>(ws, Lw.state);
  uint32_t* segcnt = ws_ptr<uint32_t>(ws, Lw.segcnt);
  uint64_t* lkey = ws_ptr<uint64_t>(ws, Lw.lkey);
  uint32_t* lpos = ws_ptr<uint32_t>(ws, Lw.lpos);
  const int mode = d.index_mode;
  const int S = mode == SKV_INDEX_SKETCH_INT4 ? d.n_sink : 0;
  const int L = mode == SKV_INDEX_SKETCH_INT4 ? d.n_tail : 0;
  hipLaunchKernelGGL(topk_sample_kernel, dim3(d.batch), dim3(kFinalThreads), 0, st, keys, ctx_len,
                     state, mode, d.max_ctx, S, d.topk, L);
  hipLaunchKernelGGL(topk_collect_kernel, dim3(Lw.n_seg, d.batch), dim3(kSelThreads), 0, st, keys,
                     ctx_len, state, segcnt, lkey, lpos, Lw.n_seg, mode, d.max_ctx, S, d.topk, L);
  hipLaunchKernelGGL(topk_final_kernel, dim3(d.batch), dim3(kFinalThreads), 0, st, keys, ctx_len,
                     segcnt, lkey, lpos, idx, n_sel, flags, Lw.n_seg, mode, d.max_ctx, S, d.topk, L,
                     select_capacity(d));
  return hipGetLastError();
}

}  // namespace skv
