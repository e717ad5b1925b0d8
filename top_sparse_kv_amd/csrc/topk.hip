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
// The select works on candidates: the keys whose 12-bit digit (the key
// rounded to fp32, 1/8 octave per bucket) is at least a threshold bucket beta
// estimated from a sample of whole 16-key lines.  Candidates are stored per
// segment (256 tokens or 128 blocks, one wave each) in position order.  With
// keys already in memory (sparsekv_topk) two kernels produce them:
//   sample   one workgroup per sequence histograms the sampled digits -> beta;
//   collect  one wave per segment keeps the digits >= beta, in order.
// The fused path (score.hip) produces the same records straight from the
// index.  Then, one workgroup per sequence:
//   final    gathers the candidates into registers (position order), finds
//            the 16-bit digit bin of the k-th largest with one LDS histogram
//            (bins above it are kept whole), orders the members of that bin
//            exactly by the composite (key, ~position) -- pairwise ranks when
//            it is small, else an MSB-first radix select -- and writes the
//            kept positions by an ordered prefix sum.
// Fallbacks, flagged SKV_FLAG_TOPK_SLOW: more candidates than LDS holds ->
// the same select over the records in global memory; fewer candidates than
// the budget (the sample overestimated beta) -> the select over every key of
// the sequence (recomputed from the index in the fused path).  The sample
// only affects speed, never the result.
#include "keys_common.h"

namespace skv {
namespace {

constexpr int kSelThreads = 256;
constexpr int kFinalThreads = 1024;   // sample kernel of the keys path
constexpr int kFT = 1024;             // final select kernel
constexpr int kSegPT = kMaxSeg / kFT; // segment counts per thread
// candidates the register path holds (per thread kGPT, in registers): more
// than the LDS lists, since the capped sample of a multi-million-token
// context lets about 9,000 through at k = 4096; the threshold bin's members
// still go through an LDS list of kListCap
constexpr int kRegCap = 12288;
constexpr int kGPT = kRegCap / kFT;

// ---------------------------------------------------------------------------
// sample and collect from materialized keys
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(kFinalThreads) void topk_sample_kernel(
    const double* __restrict__ keys, const int32_t* __restrict__ ctx_len,
    TopkState* __restrict__ state, int mode, int max_ctx, int S, int k, int L) {
  constexpr int PER = kHistBins / kFinalThreads;   // 4 bins per thread
  constexpr int UNR = 16;
  __shared__ uint32_t h[kHistBins];
  __shared__ uint32_t wsum[16];
  const int b = blockIdx.x;
  const Range r = cand_range(mode, ctx_of(ctx_len, b, max_ctx), S, k, L);
  if (r.dense) return;
  const int s = sample_stride(r.n, k);
  const int nj = sample_lines(r.n, k) * kLineKeys;   // sample slots
  for (int i = threadIdx.x; i < kHistBins; i += blockDim.x) h[i] = 0u;
  __syncthreads();
  const double* kb = keys + (size_t)b * (mode == SKV_INDEX_SKETCH_INT4 ? max_ctx : max_ctx / 4) + r.lo;
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
      if (ok[u]) atomicAdd(&h[key_digit(x[u] + 0.0)], 1u);
  }
  __syncthreads();
  const uint32_t need = sample_need(r.n, k);
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
  if (total >= need && cum < need && cum + mine >= need) {
#pragma unroll
    for (int j = 0; j < PER; ++j) {
      const uint32_t nxt = cum + cnt[j];
      if (cum < need && nxt >= need) state[b].beta = (uint32_t)(top - 1 - j);
      cum = nxt;
    }
  }
}

// one wave per segment; lane l holds the KPL consecutive keys l*KPL.. of it
template <int KPL>
__global__ __launch_bounds__(kSelThreads) void topk_collect_kernel(
    const double* __restrict__ keys, const int32_t* __restrict__ ctx_len,
    const TopkState* __restrict__ state, uint32_t* __restrict__ segcnt, Cand* __restrict__ cand,
    int n_seg, int mode, int max_ctx, int S, int k, int L) {
  constexpr int SEG = 64 * KPL;
  const int b = blockIdx.y;
  const Range r = cand_range(mode, ctx_of(ctx_len, b, max_ctx), S, k, L);
  if (r.dense) return;
  const int lane = threadIdx.x & 63;
  const int seg = blockIdx.x * (kSelThreads / 64) + (threadIdx.x >> 6);
  const int i0 = seg * SEG;
  if (i0 >= r.n) return;   // wave-uniform
  const uint32_t beta = state[b].beta;
  const double* kb = keys + (size_t)b * (mode == SKV_INDEX_SKETCH_INT4 ? max_ctx : max_ctx / 4) + r.lo;
  double x[KPL];
#pragma unroll
  for (int u = 0; u < KPL; ++u) x[u] = kb[min(i0 + lane * KPL + u, r.n - 1)] + 0.0;   // unconditional
  uint32_t selm = 0, mine = 0;
#pragma unroll
  for (int u = 0; u < KPL; ++u) {
    const int i = i0 + lane * KPL + u;
    if (i < r.n && key_digit(x[u]) >= beta) {
      selm |= 1u << u;
      ++mine;
    }
  }
  const uint32_t incl = wave_incl_scan(mine);
  uint32_t at = incl - mine;
  u32x4* out = reinterpret_cast<u32x4*>(cand + ((size_t)b * n_seg + seg) * SEG);
#pragma unroll
  for (int u = 0; u < KPL; ++u) {
    if (selm & (1u << u)) {
      const uint64_t ok = ordered_u64(x[u]);
      if (at < (uint32_t)SEG)   // always true: at most one record per key
        out[at] = (u32x4){(uint32_t)ok, (uint32_t)(ok >> 32), (uint32_t)(r.lo + i0 + lane * KPL + u),
                          key_digit16(x[u])};
      ++at;
    }
  }
  if (lane == 63) segcnt[(size_t)b * n_seg + seg] = min(incl, (uint32_t)SEG);
}

// ---------------------------------------------------------------------------
// exact radix select over unique 96-bit composites
// ---------------------------------------------------------------------------
// composite = (hi: order-preserving key, lo: ~position); larger composite =
// larger key, or equal key and lower position.
__device__ __forceinline__ uint32_t comp_digit(uint64_t hi, uint32_t lo, int dg) {
  return dg >= 4 ? (uint32_t)(hi >> (8 * (dg - 4))) & 0xFFu : (lo >> (8 * dg)) & 0xFFu;
}

struct SelectShared {
  uint32_t hist[256];
  uint32_t wsum[16];
  uint32_t wred[16][6];
  uint64_t pre_hi, mask_hi;
  uint32_t pre_lo, mask_lo;
  int need;
  int done;
  int dg0;
};

// MSB-first radix select of the k largest composites among n (0 < k <= n).
// On return every element with (hi & mask_hi, lo & mask_lo) lexicographically
// >= (pre_hi, pre_lo) is kept, and exactly k elements satisfy that.  The loop
// stops once the boundary bucket is kept whole.  get(i, hi, lo) reads element
// i.  Every thread of the block must call it.
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
  a0 = wave_and(a0); a1 = wave_and(a1); a2 = wave_and(a2);
  o0 = wave_or(o0);  o1 = wave_or(o1);  o2 = wave_or(o2);
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, nw = blockDim.x >> 6;
  if (lane == 0) {
    sh.wred[wave][0] = a0; sh.wred[wave][1] = a1; sh.wred[wave][2] = a2;
    sh.wred[wave][3] = o0; sh.wred[wave][4] = o1; sh.wred[wave][5] = o2;
  }
  __syncthreads();
  if (wave == 0) {
    // lane w < nw holds wave w's values; a 16-lane DPP reduction combines them
    const int w = lane < nw ? lane : 0;
    a0 = sh.wred[w][0]; a1 = sh.wred[w][1]; a2 = sh.wred[w][2];
    o0 = sh.wred[w][3]; o1 = sh.wred[w][4]; o2 = sh.wred[w][5];
    a0 = wave_and(a0); a1 = wave_and(a1); a2 = wave_and(a2);
    o0 = wave_or(o0);  o1 = wave_or(o1);  o2 = wave_or(o2);
    if (lane == 0) {
      const uint64_t ahi = ((uint64_t)a0 << 32) | a1, ohi = ((uint64_t)o0 << 32) | o1;
      uint64_t ph = 0, mh = 0;
      uint32_t pl = 0, ml = 0;
      int dg = 11;
      while (dg >= 0) {
        const uint32_t da = comp_digit(ahi, a2, dg), dor = comp_digit(ohi, o2, dg);
        if (da != dor) break;
        if (dg >= 4) {
          ph |= (uint64_t)da << (8 * (dg - 4));
          mh |= 0xFFull << (8 * (dg - 4));
        } else {
          pl |= da << (8 * dg);
          ml |= 0xFFu << (8 * dg);
        }
        --dg;
      }
      sh.pre_hi = ph;
      sh.mask_hi = mh;
      sh.pre_lo = pl;
      sh.mask_lo = ml;
      sh.need = k;
      sh.done = (k == n) || dg < 0;
      sh.dg0 = dg;
    }
  }
  __syncthreads();
  for (int dg = sh.dg0; dg >= 0 && !sh.done; --dg) {
    if (threadIdx.x < 256) sh.hist[threadIdx.x] = 0u;
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
      uint32_t c4[4];
      uint32_t s = 0;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        c4[j] = sh.hist[255 - 4 * lane - j];
        s += c4[j];
      }
      const uint32_t incl = wave_incl_scan(s);
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
  return (h > sh.pre_hi) | ((h == sh.pre_hi) & ((lo & sh.mask_lo) >= sh.pre_lo));
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

// Writes the kept elements of [0, n) in index order (indices are in position
// order), one block-wide prefix sum per round of blockDim.x elements.
template <class Get>
__device__ void ordered_emit(Get get, int n, int k, SelectShared& sh, int32_t* out, int mode,
                             int S) {
  uint32_t before = 0;
  for (int base = 0; base < n; base += blockDim.x) {
    const int i = base + threadIdx.x;
    uint64_t hi = 0;
    uint32_t lo = 0;
    int pos = 0;
    bool sel = false;
    if (i < n) {
      get(i, hi, lo, pos);
      sel = kept(hi, lo, sh);
    }
    uint32_t tot = 0;
    const uint32_t off = block_excl_scan(sel ? 1u : 0u, sh.wsum, &tot);
    if (sel && before + off < (uint32_t)k) emit_position(out, mode, S, (int)(before + off), pos);
    before += tot;
  }
}

// segment of flattened candidate j: the last c with s_off[c] <= j (s_off is
// non-decreasing and s_off[nparts] = total > j)
__device__ __forceinline__ int seg_of(const uint32_t* s_off, int nparts, uint32_t j) {
  int lo = 0, hi = nparts - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (s_off[mid] <= j) lo = mid; else hi = mid - 1;
  }
  return lo;
}

struct NoSrc {
  static constexpr int LANES = 64;
};

// bucket sizes resolved by pairwise ranks: 16, 8, 4, 2 or 1 threads per
// member (a wider bucket takes the multi-pass radix select)
constexpr uint32_t kRankMax = 1024;

// RECOMPUTE (the fused path): keys are recomputed from the index when the
// candidates are too few.
constexpr int kFetch = 4;                   // records read with each segment count
constexpr int kFetch2 = 12;                 // records read in the second batch of a longer segment
constexpr int kOneTripSegs = 2 * kFT;       // segments the one-round-trip path covers
// LDS of the final select, shared by its paths (bytes): the one-trip path's
// candidate arrays (key, position, digit) plus a member list, or the other
// paths' register-gather lists and segment offsets
constexpr size_t kFastBytes = (size_t)kListCap * 14 + (kRankMax + 64) * 12;
constexpr size_t kOldBytes = (size_t)(kListCap + 64) * 12 + (size_t)(kMaxSeg + 1) * 4;
constexpr size_t kSelLds = kFastBytes > kOldBytes ? kFastBytes : kOldBytes;

template <class Src, bool RECOMPUTE>
__global__ __launch_bounds__(kFT) void topk_final_kernel(
    const double* __restrict__ keys_in, const void* __restrict__ iq, const void* __restrict__ ik,
    const uint16_t* __restrict__ isc, const int32_t* __restrict__ ctx_len,
    const uint32_t* __restrict__ segcnt, Cand* __restrict__ cand, const TopkState* __restrict__ state,
    int32_t* __restrict__ idx, int32_t* __restrict__ n_sel,
    uint32_t* __restrict__ flags, int n_seg, int seg_items, int mode, int max_ctx, int S, int k,
    int L, int cap, int mq) {
  __shared__ uint64_t s_mem[(kSelLds + 7) / 8];
  uint64_t* s_bhi = s_mem;                                                   // [kListCap + 64]
  uint32_t* s_blo = reinterpret_cast<uint32_t*>(s_bhi + kListCap + 64);      // [kListCap + 64]
  uint32_t* s_off = s_blo + kListCap + 64;                                   // [kMaxSeg + 1]
  __shared__ uint32_t s_hist[256 + 32];
  __shared__ SelectShared sh;
  const int b = blockIdx.x;   // virtual sequence: query b % mq of sequence b / mq
  const int T = ctx_of_query(ctx_len, b, mq, max_ctx);
  const Range r = cand_range(mode, T, S, k, L);
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
  const int n_parts = (r.n + seg_items - 1) / seg_items;
  const uint32_t* sc = segcnt + (size_t)b * n_seg;
  const Cand* cb = cand + (size_t)b * n_seg * seg_items;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;

  if (n_parts <= kOneTripSegs) {
    // ---- per 1024 segments: each thread reads one segment's count together
    // with its first kFetch records (a segment averages a few candidates), a
    // block prefix sum places them in LDS in position order, and the longer
    // segments read the rest in one more batch ----
    uint64_t* c_key = s_mem;                                                  // [kListCap]
    uint32_t* c_pos = reinterpret_cast<uint32_t*>(c_key + kListCap);          // [kListCap]
    uint16_t* c_dig = reinterpret_cast<uint16_t*>(c_pos + kListCap);          // [kListCap]
    uint64_t* m_hi = reinterpret_cast<uint64_t*>(c_dig + kListCap);           // [kRankMax + 64]
    uint32_t* m_lo = reinterpret_cast<uint32_t*>(m_hi + kRankMax + 64);       // [kRankMax + 64]
    uint32_t total = 0;
    bool fits = true;
    for (int r0 = 0; r0 < n_parts; r0 += kFT) {   // workgroup-uniform
      const int seg = r0 + (int)threadIdx.x;
      const int segc = min(seg, n_parts - 1);
      const u32x4* src = reinterpret_cast<const u32x4*>(cb + (size_t)segc * seg_items);
      uint32_t cnt = sc[segc];
      u32x4 rr[kFetch];
#pragma unroll
      for (int m = 0; m < kFetch; ++m) rr[m] = src[m];   // unconditional, inside the segment
      cnt = seg < n_parts ? min(cnt, (uint32_t)seg_items) : 0u;
      uint32_t tot = 0;
      const uint32_t off = total + block_excl_scan(cnt, sh.wsum, &tot);
      if (total + tot > (uint32_t)kListCap) {   // uniform: more candidates than LDS holds
        fits = false;
        break;
      }
#pragma unroll
      for (int m = 0; m < kFetch; ++m)
        if ((uint32_t)m < cnt) {
          c_key[off + m] = ((uint64_t)rr[m].y << 32) | rr[m].x;
          c_pos[off + m] = rr[m].z;
          c_dig[off + m] = (uint16_t)rr[m].w;
        }
      // longer segments: the next kFetch2 records in one batch, then (rare)
      // further batches
      for (uint32_t m0 = kFetch; m0 < cnt; m0 += kFetch2) {
        u32x4 r2[kFetch2];
#pragma unroll
        for (int m = 0; m < kFetch2; ++m) r2[m] = src[min(m0 + (uint32_t)m, cnt - 1)];
#pragma unroll
        for (int m = 0; m < kFetch2; ++m)
          if (m0 + (uint32_t)m < cnt) {
            c_key[off + m0 + m] = ((uint64_t)r2[m].y << 32) | r2[m].x;
            c_pos[off + m0 + m] = r2[m].z;
            c_dig[off + m0 + m] = (uint16_t)r2[m].w;
          }
      }
      total += tot;
    }
    __syncthreads();
    if (fits && total >= (uint32_t)k) {
      const int n = (int)total;
      // digits relative to the threshold every candidate passed (12-bit in
      // the keys path, 16-bit elsewhere); bins count up from it, the last bin
      // open; the bin of the k-th largest (fbin) is the only one ranked
      const uint32_t dlo = RECOMPUTE ? state[b].beta : state[b].beta << 4;
      auto bin_of = [&](uint32_t dg) -> uint32_t { return dg >= dlo ? min(dg - dlo, 255u) : 0u; };
      const int PT = (n + kFT - 1) / kFT;   // candidates per thread, a contiguous run
      const int j0 = PT * (int)threadIdx.x;
      if (threadIdx.x < 256) s_hist[threadIdx.x] = 0u;
      if (threadIdx.x == 0) s_hist[258] = 0u;
      __syncthreads();
      for (int m = 0; m < PT; ++m)
        if (j0 + m < n) atomicAdd(&s_hist[bin_of(c_dig[j0 + m])], 1u);
      __syncthreads();
      uint32_t* wr = s_hist + 256;
      if (wave == 0) {
        uint32_t c[4], t = 0;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          c[j] = s_hist[255 - 4 * lane - j];
          t += c[j];
        }
        const uint32_t incl = wave_incl_scan(t);
        const uint64_t hit = __ballot(incl >= (uint32_t)k);   // not empty: n >= k
        const int l = (int)__ffsll((unsigned long long)hit) - 1;
        uint32_t cum = incl - t, fb = 0, before = 0, fbc = 0;
        bool found = false;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          if (!found && cum + c[j] >= (uint32_t)k) {
            found = true;
            fb = (uint32_t)(255 - 4 * lane - j);
            before = cum;
            fbc = c[j];
          }
          cum += c[j];
        }
        if (lane == l) {
          wr[0] = fb;       // the bin of the k-th largest
          wr[1] = before;   // candidates in the bins above it
          wr[3] = fbc;      // members of that bin
        }
      }
      __syncthreads();
      const uint32_t fbin = wr[0], rk = (uint32_t)k - wr[1], mb = wr[3];
      if (mb <= kRankMax) {
        // the members of fbin, appended in any order, ranked pairwise
        for (int m = 0; m < PT; ++m)
          if (j0 + m < n && bin_of(c_dig[j0 + m]) == fbin) {
            const uint32_t at = atomicAdd(&wr[2], 1u);
            m_hi[at] = c_key[j0 + m];
            m_lo[at] = ~c_pos[j0 + m];
          }
        if (threadIdx.x < 64) {   // padding that never ranks above a member
          m_hi[mb + threadIdx.x] = 0ull;
          m_lo[mb + threadIdx.x] = 0u;
        }
        __syncthreads();
        const int P = mb <= 64 ? 16 : (mb <= 128 ? 8 : (mb <= 256 ? 4 : (mb <= 512 ? 2 : 1)));
        const int mm = (int)threadIdx.x / P, part = (int)threadIdx.x % P;
        uint32_t rank = 0;
        uint64_t hi = 0;
        uint32_t lo = 0;
        if (mm < (int)mb) {
          hi = m_hi[mm];
          lo = m_lo[mm];
          for (int j = part; j < (int)mb; j += 4 * P) {
            uint64_t oh[4];
            uint32_t ol[4];
#pragma unroll
            for (int u = 0; u < 4; ++u) {
              oh[u] = m_hi[j + u * P];
              ol[u] = m_lo[j + u * P];
            }
#pragma unroll
            for (int u = 0; u < 4; ++u)
              rank += (uint32_t)(oh[u] > hi) + (uint32_t)((oh[u] == hi) & (ol[u] > lo));
          }
        }
        for (int o = 1; o < P; o <<= 1) rank += (uint32_t)__shfl_xor((int)rank, o);
        if (mm < (int)mb && part == 0 && rank == rk - 1) {
          sh.pre_hi = hi;
          sh.pre_lo = lo;
        }
        if (threadIdx.x == 0) {
          sh.mask_hi = ~0ull;
          sh.mask_lo = ~0u;
        }
        __syncthreads();
      } else {
        // a wide bin: radix select over all candidates, non-members as zeros
        radix_select([&](int i, uint64_t& hi, uint32_t& lo) {
          const bool mem = bin_of(c_dig[i]) == fbin;
          hi = mem ? c_key[i] : 0ull;
          lo = mem ? ~c_pos[i] : 0u;
        }, n, (int)rk, sh);
      }
      // ordered emission of the kept candidates (runs are in position order)
      uint32_t cnt = 0;
      for (int m = 0; m < PT; ++m) {
        const int i = j0 + m;
        if (i < n) {
          const uint32_t bn = bin_of(c_dig[i]);
          cnt += (uint32_t)(bn > fbin || (bn == fbin && kept(c_key[i], ~c_pos[i], sh)));
        }
      }
      int rank = (int)block_excl_scan(cnt, sh.wsum, nullptr);
      for (int m = 0; m < PT; ++m) {
        const int i = j0 + m;
        if (i < n) {
          const uint32_t bn = bin_of(c_dig[i]);
          if (bn > fbin || (bn == fbin && kept(c_key[i], ~c_pos[i], sh))) {
            if (rank < k) emit_position(out, mode, S, rank, (int)c_pos[i]);
            ++rank;
          }
        }
      }
      return;
    }
    __syncthreads();   // the LDS is reused below
  }

  // segment offsets (n_parts <= kMaxSeg = kSegPT * blockDim.x)
  uint32_t total;
  {
    uint32_t cs[kSegPT], mine = 0;
#pragma unroll
    for (int j = 0; j < kSegPT; ++j) {
      const int c = kSegPT * threadIdx.x + j;
      const uint32_t v = sc[min(c, n_parts - 1)];   // unconditional
      cs[j] = c < n_parts ? min(v, (uint32_t)seg_items) : 0u;
      mine += cs[j];
    }
    uint32_t off = block_excl_scan(mine, sh.wsum, &total);
#pragma unroll
    for (int j = 0; j < kSegPT; ++j) {
      const int c = kSegPT * threadIdx.x + j;
      if (c < n_parts) s_off[c] = off;
      off += cs[j];
    }
    if (threadIdx.x == 0) s_off[n_parts] = total;
    __syncthreads();
  }

  if (total >= (uint32_t)k && total <= (uint32_t)kRegCap) {
    // ---- fast path: the candidates stay in registers, in position order ----
    // Thread t holds the contiguous run [kGPT*t, kGPT*(t+1)): one search for
    // its first segment, then a walk; all its loads are issued together.
    const int n = (int)total;
    const int j0 = kGPT * (int)threadIdx.x;
    u32x4 rec[kGPT];
    {
      int c = seg_of(s_off, n_parts, (uint32_t)min(j0, n - 1));
#pragma unroll
      for (int m = 0; m < kGPT; ++m) {
        const int j = min(j0 + m, n - 1);
        while (c + 1 < n_parts && (int)s_off[c + 1] <= j) ++c;
        const int e = min(max(j - (int)s_off[c], 0), seg_items - 1);   // in range by construction
        rec[m] = reinterpret_cast<const u32x4*>(cb + (size_t)c * seg_items)[e];
      }
    }
    // The 16-bit digit (rec.w) is monotone in the key.  Bins count digits
    // upward from the lowest one, the last bin takes everything from 255 up.
    // The bin of the k-th largest candidate, fbin, splits the set: larger bins
    // are kept whole, smaller ones dropped, and only the members of fbin need
    // the exact (key, position) order.
    uint32_t* wr = s_hist + 256;
    {
      uint32_t inv = 0;
#pragma unroll
      for (int m = 0; m < kGPT; ++m)
        if (j0 + m < n) inv = max(inv, 0xFFFFu - rec[m].w);
      inv = wave_max(inv);
      if (lane == 0) wr[wave] = inv;
      if (threadIdx.x < 256) s_hist[threadIdx.x] = 0u;
    }
    __syncthreads();
    const uint32_t dmin = 0xFFFFu - lds_max16(wr, kFT / 64);
    auto bin_of = [&](uint32_t dg) -> uint32_t { return min(dg - dmin, 255u); };
#pragma unroll
    for (int m = 0; m < kGPT; ++m)
      if (j0 + m < n) atomicAdd(&s_hist[bin_of(rec[m].w)], 1u);
    __syncthreads();
    if (wave == 0) {
      // lane l owns bins 255-4l .. 252-4l, counted from the top
      uint32_t c[4], s = 0;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        c[j] = s_hist[255 - 4 * lane - j];
        s += c[j];
      }
      const uint32_t incl = wave_incl_scan(s);
      const uint64_t hit = __ballot(incl >= (uint32_t)k);   // not empty: n >= k
      const int l = (int)__ffsll((unsigned long long)hit) - 1;
      uint32_t cum = incl - s, fb = 0, before = 0;
      bool found = false;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        if (!found && cum + c[j] >= (uint32_t)k) {
          found = true;
          fb = (uint32_t)(255 - 4 * lane - j);
          before = cum;
        }
        cum += c[j];
      }
      const uint32_t fsel = (uint32_t)__builtin_amdgcn_readlane((int)fb, l);
      const uint32_t bsel = (uint32_t)__builtin_amdgcn_readlane((int)before, l);
      if (lane == 0) {
        wr[16] = fsel;
        wr[17] = bsel;
      }
    }
    __syncthreads();
    const uint32_t fbin = wr[16];
    const uint32_t r = (uint32_t)k - wr[17];   // taken from bin fbin, >= 1
    // the members of fbin, in position order, as composites (key, ~position)
    uint32_t mine = 0;
#pragma unroll
    for (int m = 0; m < kGPT; ++m)
      if (j0 + m < n && bin_of(rec[m].w) == fbin) ++mine;
    uint32_t mb = 0;
    uint32_t at = block_excl_scan(mine, sh.wsum, &mb);
    if (mb <= (uint32_t)kListCap) {   // workgroup-uniform; else the path over the records below
#pragma unroll
    for (int m = 0; m < kGPT; ++m)
      if (j0 + m < n && bin_of(rec[m].w) == fbin) {
        s_bhi[at] = ((uint64_t)rec[m].y << 32) | rec[m].x;
        s_blo[at] = ~rec[m].z;
        ++at;
      }
    if (threadIdx.x < 64) {   // padding that never ranks above a member
      s_bhi[mb + threadIdx.x] = 0ull;
      s_blo[mb + threadIdx.x] = 0u;
    }
    __syncthreads();
    if (mb <= kRankMax) {
      // each member counts the members above it (P threads per member, each
      // over every P-th member); rank r-1 is the threshold
      const int P = mb <= 64 ? 16 : (mb <= 128 ? 8 : (mb <= 256 ? 4 : (mb <= 512 ? 2 : 1)));
      const int m = (int)threadIdx.x / P, part = (int)threadIdx.x % P;
      uint32_t rank = 0;
      uint64_t hi = 0;
      uint32_t lo = 0;
      if (m < (int)mb) {
        hi = s_bhi[m];
        lo = s_blo[m];
        for (int j = part; j < (int)mb; j += 4 * P) {
          uint64_t oh[4];
          uint32_t ol[4];
#pragma unroll
          for (int u = 0; u < 4; ++u) {   // past mb: zero padding, never above a member
            oh[u] = s_bhi[j + u * P];
            ol[u] = s_blo[j + u * P];
          }
          // the two cases exclude each other; added without branches
#pragma unroll
          for (int u = 0; u < 4; ++u)
            rank += (uint32_t)(oh[u] > hi) + (uint32_t)((oh[u] == hi) & (ol[u] > lo));
        }
      }
      for (int o = 1; o < P; o <<= 1) rank += (uint32_t)__shfl_xor((int)rank, o);
      if (m < (int)mb && part == 0 && rank == r - 1) {
        sh.pre_hi = hi;
        sh.pre_lo = lo;
      }
      if (threadIdx.x == 0) {
        sh.mask_hi = ~0ull;
        sh.mask_lo = ~0u;
      }
      __syncthreads();
    } else {
      radix_select([&](int i, uint64_t& hi, uint32_t& lo) {
        hi = s_bhi[i];
        lo = s_blo[i];
      }, (int)mb, (int)r, sh);
    }
    // ordered emission of the kept candidates
    uint32_t keep = 0, cnt = 0;
#pragma unroll
    for (int m = 0; m < kGPT; ++m) {
      if (j0 + m >= n) continue;
      const uint32_t bn = bin_of(rec[m].w);
      if (bn > fbin ||
          (bn == fbin && kept(((uint64_t)rec[m].y << 32) | rec[m].x, ~rec[m].z, sh))) {
        keep |= 1u << m;
        ++cnt;
      }
    }
    int rank = (int)block_excl_scan(cnt, sh.wsum, nullptr);
#pragma unroll
    for (int m = 0; m < kGPT; ++m)
      if (keep & (1u << m)) {
        if (rank < k) emit_position(out, mode, S, rank, (int)rec[m].z);
        ++rank;
      }
    return;
    }
    __syncthreads();   // the LDS is reused below
  }

  if (threadIdx.x == 0) raise_flag(flags, SKV_FLAG_TOPK_SLOW);
  if (total >= (uint32_t)k) {
    // ---- more candidates than LDS holds: the same select over the records ----
    const int n = (int)total;
    auto rec_of = [&](int j) -> u32x4 {
      const int c = seg_of(s_off, n_parts, (uint32_t)j);
      const int e = min(max(j - (int)s_off[c], 0), seg_items - 1);   // in range by construction
      return reinterpret_cast<const u32x4*>(cb + (size_t)c * seg_items)[e];
    };
    radix_select([&](int i, uint64_t& hi, uint32_t& lo) {
      const u32x4 v = rec_of(i);
      hi = ((uint64_t)v.y << 32) | v.x;
      lo = ~v.z;
    }, n, k, sh);
    ordered_emit([&](int i, uint64_t& hi, uint32_t& lo, int& pos) {
      const u32x4 v = rec_of(i);
      hi = ((uint64_t)v.y << 32) | v.x;
      lo = ~v.z;
      pos = (int)v.z;
    }, n, k, sh, out, mode, S);
    return;
  }

  // ---- fewer candidates than the budget: the select over every key ----
  const double* kb;
  if constexpr (RECOMPUTE) {
    // the sequence's record area holds 2 * n_seg * seg_items doubles >= r.n
    double* kw = reinterpret_cast<double*>(cand + (size_t)b * n_seg * seg_items);
    constexpr int N = Src::LANES, IPW = 64 / N, PER_IT = 8 * IPW;
    const int sub = lane % N, tw = lane / N;
    Src src;
    src.init(reinterpret_cast<const uint8_t*>(iq) + (size_t)b * Src::QROW, ik, isc, b / mq, max_ctx,
             sub);
    for (int base = wave * PER_IT; base < r.n; base += (kFT / 64) * PER_IT) {
      u32x4 w[8];
      uint32_t ax[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const int i = min(base + u * IPW + tw, r.n - 1);
        w[u] = src.load(r.lo + i);
        ax[u] = src.load_aux(r.lo + i);
      }
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const int i = base + u * IPW + tw;
        const double key = src.key(w[u], ax[u]);
        if (sub == 0 && i < r.n) kw[i] = key;
      }
    }
    __threadfence_block();
    __syncthreads();
    kb = kw;
  } else {
    kb = keys_in + (size_t)b * (mode == SKV_INDEX_SKETCH_INT4 ? max_ctx : max_ctx / 4) + r.lo;
  }
  const int lo0 = r.lo;
  radix_select([&](int i, uint64_t& hi, uint32_t& lo) {
    hi = ordered_u64(kb[i] + 0.0);
    lo = ~(uint32_t)(lo0 + i);
  }, r.n, k, sh);
  ordered_emit([&](int i, uint64_t& hi, uint32_t& lo, int& pos) {
    hi = ordered_u64(kb[i] + 0.0);
    lo = ~(uint32_t)(lo0 + i);
    pos = lo0 + i;
  }, r.n, k, sh, out, mode, S);
}

// d.batch counts virtual sequences (mq query tokens per sequence)
template <class Src, bool RECOMPUTE>
hipError_t launch_final(const skv_layer_desc& d, const int32_t* ctx_len, const double* keys,
                        const void* iq, const void* ik, const uint16_t* isc, int32_t* idx,
                        int32_t* n_sel, void* ws, const WsLayout& Lw, hipStream_t st, int mq = 1) {
  const int mode = d.index_mode;
  const int S = mode == SKV_INDEX_SKETCH_INT4 ? d.n_sink : 0;
  const int L = mode == SKV_INDEX_SKETCH_INT4 ? d.n_tail : 0;
  hipLaunchKernelGGL((topk_final_kernel<Src, RECOMPUTE>), dim3(d.batch), dim3(kFT), 0, st,
                     keys, iq, ik, isc, ctx_len, ws_ptr<uint32_t>(ws, Lw.segcnt),
                     ws_ptr<Cand>(ws, Lw.cand), ws_ptr<const TopkState>(ws, Lw.state), idx, n_sel,
                     ws_ptr<uint32_t>(ws, Lw.flags),
                     Lw.n_seg, Lw.seg_items, mode, d.max_ctx, S, d.topk, L, select_capacity(d), mq);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_topk(const skv_layer_desc& d, const int32_t* ctx_len, const double* keys,
                       int32_t* idx, int32_t* n_sel, void* ws, const WsLayout& Lw,
                       hipStream_t st) {
  const int mode = d.index_mode;
  const int S = mode == SKV_INDEX_SKETCH_INT4 ? d.n_sink : 0;
  const int L = mode == SKV_INDEX_SKETCH_INT4 ? d.n_tail : 0;
  TopkState* state = ws_ptr<TopkState>(ws, Lw.state);
  hipLaunchKernelGGL(topk_sample_kernel, dim3(d.batch), dim3(kFinalThreads), 0, st, keys, ctx_len,
                     state, mode, d.max_ctx, S, d.topk, L);
  const dim3 grid((Lw.n_seg + 3) / 4, d.batch);
  if (Lw.seg_items == kSegTok)
    hipLaunchKernelGGL((topk_collect_kernel<kSegTok / 64>), grid, dim3(kSelThreads), 0, st, keys,
                       ctx_len, state, ws_ptr<uint32_t>(ws, Lw.segcnt), ws_ptr<Cand>(ws, Lw.cand),
                       Lw.n_seg, mode, d.max_ctx, S, d.topk, L);
  else
    hipLaunchKernelGGL((topk_collect_kernel<kSegBlk / 64>), grid, dim3(kSelThreads), 0, st, keys,
                       ctx_len, state, ws_ptr<uint32_t>(ws, Lw.segcnt), ws_ptr<Cand>(ws, Lw.cand),
                       Lw.n_seg, mode, d.max_ctx, S, d.topk, L);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  return launch_final<NoSrc, false>(d, ctx_len, keys, nullptr, nullptr, nullptr, idx, n_sel, ws, Lw, st);
}

hipError_t launch_final_multi(const skv_layer_desc& dv, int mq, const int32_t* ctx_len,
                              const int8_t* qs, const void* ik, const uint16_t* isc, int32_t* idx,
                              int32_t* n_sel, void* ws, const WsLayout& Lw, hipStream_t st) {
  switch (dv.n_kv_heads * dv.rank / 2) {
    case 64: return launch_final<SketchSrc<4>, true>(dv, ctx_len, nullptr, qs, ik, isc, idx, n_sel, ws, Lw, st, mq);
    case 128: return launch_final<SketchSrc<8>, true>(dv, ctx_len, nullptr, qs, ik, isc, idx, n_sel, ws, Lw, st, mq);
    case 256: return launch_final<SketchSrc<16>, true>(dv, ctx_len, nullptr, qs, ik, isc, idx, n_sel, ws, Lw, st, mq);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_score_select(const skv_layer_desc& d, const int32_t* ctx_len, const void* iq,
                               const void* q, const float* basis, int8_t* qs_out, float* qscale_out,
                               const void* ik, const uint16_t* isc, int32_t* idx, int32_t* n_sel,
                               void* ws, const WsLayout& Lw, hipStream_t st) {
  hipError_t e = launch_sample_collect(d, ctx_len, iq, q, basis, qs_out, qscale_out, ik, isc, ws, Lw, st);
  if (e != hipSuccess) return e;
  const void* qrows = qs_out ? (const void*)qs_out : iq;
#define SKV_FIN(SRC) return launch_final<SRC, true>(d, ctx_len, nullptr, qrows, ik, isc, idx, n_sel, ws, Lw, st)
  if (d.index_mode == SKV_INDEX_SKETCH_INT4) {
    switch (d.n_kv_heads * d.rank / 2) {
      case 32: SKV_FIN(SketchSrc<2>);
      case 64: SKV_FIN(SketchSrc<4>);
      case 128: SKV_FIN(SketchSrc<8>);
      case 256: SKV_FIN(SketchSrc<16>);
      default: return hipErrorInvalidValue;
    }
  }
  switch (d.index_dim) {
    case 64: SKV_FIN(PooledSrc<8>);
    case 128: SKV_FIN(PooledSrc<16>);
    case 256: SKV_FIN(PooledSrc<32>);
    default: return hipErrorInvalidValue;
  }
#undef SKV_FIN
}

}  // namespace skv
