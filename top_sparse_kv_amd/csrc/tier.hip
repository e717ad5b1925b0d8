// Host-RAM KV tier with a GPU hot buffer (stage A5).
//
// Page "8 agents x 250K context on two 3090s: sparse KV decode with a rank-64
// key sketch and a host-RAM tier", section "The mechanism": the full K/V lives
// in pinned host RAM at int4 (64-dim groups, fp16 scales, 272 B per
// token-head), turned back into int8 rows when fetched; the GPU keeps the
// sinks, the recent tail and a hot buffer of 2.5% of the tokens managed by
// windowed CLOCK; a token missing from the hot buffer is fetched alone, by a
// direct GPU read of its host record across PCIe.  Page "3.14M Context on 3x 3090: The Power of an
// Architecture That Puts KV Cache in Host RAM", sections "No Need to Rewrite
// the Kernel": the GPU reads host-mapped memory directly (zero copy), which
// needs no per-layer host synchronization and keeps the step capturable.
//
// Host memory: hipHostMalloc(mapped | portable) -- pinned at allocation --
// rather than registering an existing anonymous mapping, and the kernel reads
// it through the device address hipHostGetDevicePointer returns.
//
// Per step: tier_resolve (one workgroup per sequence) marks hits, then places
// the misses; tier_fetch (many workgroups) reads the missed records over PCIe
// and writes int8 rows + fp16 scales into their slots.
//
// Placement in parallel.  Walking the slots in hand order from where the hand
// stopped, a slot is "free" if it is empty or unpinned (last <= step - W) with
// its reference bit clear, and "referenced" if it is occupied, unpinned and
// has the bit set.  The hand takes free slots and clears the bits of the
// referenced slots it passes; pinned slots (including those taken in this
// step) are skipped.  So the m-th miss (ascending position) takes the m-th
// free slot; if the misses outnumber the free slots, the hand completes the
// sweep -- every referenced slot is then clear -- and the remaining misses
// take the referenced slots in hand order; beyond those nothing can be
// evicted (flagged).  One prefix sum over the slots, in hand order, gives
// every rank at once.
//
// LRU policy (page "vLLM's Hybrid HiSparse Triples Concurrent Requests on
// Million-Token Contexts", section "Three residency states, one block pool"):
// hits refresh the slot's last use; the misses need as many victims, the
// oldest slots not used in this step.  The victims' last-use bound is found
// by a 4 x 8-bit radix select over the ages (LDS histograms), the slots at
// exactly that age are taken in slot order, and the misses fill the victims
// in slot order: two prefix sums over the slots in index order.
#include "keys_common.h"

#include <hip/hip_ext.h>

#include <algorithm>
#include <new>
#include <vector>
#include <stddef.h>
#include <string.h>

struct skv_tier {
  skv_tier_desc desc;
  int B, S, L, k, Hkv, D, n_slots, W, cap, policy;
  int T0;             // context at creation: the tail ring's anchor
  int cap_ctx;        // positions per sequence the tier can hold (layer max_ctx)
  int rec_bytes;      // per token-head: K row + V row
  int row_bytes;      // one K (or V) host row
  void* host;         // host records (host address)
  bool own_host;
  const uint8_t* host_dev;  // device address of the host records
  int64_t res_rows;   // S + L + n_slots
  int8_t* res_k;
  int8_t* res_v;
  uint16_t* res_ks;
  uint16_t* res_vs;
  int32_t* slot_pos;     // [B][n_slots]
  int32_t* slot_last;    // [B][n_slots]
  int32_t* slot_ref;     // [B][n_slots]
  int32_t* hand;         // [B]
  int32_t* slot_of_pos;  // [B][cap_ctx]
  int32_t* ctx_dev;      // [B] context of each sequence (advanced by sparsekv_tier_append)
  int64_t appends;       // sparsekv_tier_append calls
  int mstride;           // misses per sequence the arrays below hold
  int32_t* miss_pos;     // [B][mstride]
  int32_t* miss_slot;    // [B][mstride]
  int32_t* miss_count;   // [B]
  unsigned long long* counters;  // picks, hits, misses
  uint32_t* flags;
  int64_t steps;
};

namespace skv {
namespace {

constexpr int kResolveThreads = 1024;
constexpr int kMaxSlots = 12288;     // slot table held in LDS
// misses of one pick list: its middle picks (those of a later query token of a
// sequence include up to kMaxQueries - 1 of its tail positions)
constexpr int kMaxListMisses = kMaxTopk + kMaxQueries;
constexpr int kNoStep = -(1 << 30);

__global__ void tier_reset_kernel(int32_t* slot_pos, int32_t* slot_last, int32_t* slot_ref,
                                  int32_t* hand, int32_t* slot_of_pos, unsigned long long* counters,
                                  int B, int n_slots, int cap_ctx) {
  const size_t tid = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
  const size_t nth = (size_t)gridDim.x * blockDim.x;
  for (size_t i = tid; i < (size_t)B * n_slots; i += nth) {
    slot_pos[i] = -1;
    slot_last[i] = kNoStep;
    slot_ref[i] = 0;
  }
  for (size_t i = tid; i < (size_t)B * cap_ctx; i += nth) slot_of_pos[i] = -1;
  for (size_t i = tid; i < (size_t)B; i += nth) hand[i] = 0;
  if (tid < 3) counters[tid] = 0ull;
}

// MULTI: several pick lists per sequence (mq of them); one list compiles to
// straight-line code without the loop's live state
template <int POLICY, bool MULTI>
__global__ __launch_bounds__(kResolveThreads) void tier_resolve_kernel(
    const int32_t* __restrict__ idx, const int32_t* __restrict__ n_sel, int32_t* __restrict__ rows,
    int32_t* __restrict__ slot_pos, int32_t* __restrict__ slot_last, int32_t* __restrict__ slot_ref,
    int32_t* __restrict__ hand_arr, int32_t* __restrict__ slot_of_pos,
    int32_t* __restrict__ miss_pos, int32_t* __restrict__ miss_slot, int32_t* __restrict__ miss_count,
    unsigned long long* __restrict__ counters, uint32_t* __restrict__ flags,
    const int32_t* __restrict__ tier_ctx, int T0, int cap_ctx, int S, int L,
    int k, int n_slots, int W, int cap, int step, int mq, int mstride) {
  __shared__ int32_t s_pos[kMaxSlots];
  __shared__ int32_t s_last[kMaxSlots];
  __shared__ uint8_t s_ref[kMaxSlots];
  __shared__ int32_t s_miss[kMaxListMisses];   // input index of each miss
  __shared__ int32_t s_mpos[kMaxListMisses];   // its position (read by the serial placement)
  __shared__ uint32_t s_wsum[kResolveThreads / 64];
  __shared__ int s_nm, s_nmid, s_bad, s_tlast, s_hand, s_moff;
  const int b = blockIdx.x;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  int32_t* sp = slot_pos + (size_t)b * n_slots;
  int32_t* sl = slot_last + (size_t)b * n_slots;
  int32_t* sr = slot_ref + (size_t)b * n_slots;
  int32_t* sop = slot_of_pos + (size_t)b * cap_ctx;
  // scalars first: their loads overlap the slot-table copy
  const int T = tier_ctx[b];   // this sequence's context (sinks, middle, tail ring)
  int hand = hand_arr[b];
  int n_next = n_sel[(size_t)b * mq];
  int moff = 0;   // misses placed by the earlier lists
  for (int i = threadIdx.x; i < n_slots; i += blockDim.x) {
    s_pos[i] = sp[i];
    s_last[i] = sl[i];
    s_ref[i] = (uint8_t)sr[i];
  }
  if (threadIdx.x == 0) s_bad = 0;
  // The mq pick lists of the sequence (several query tokens) are resolved one
  // after another at the same step: rows placed for an earlier list are used
  // in this step, so a later list finds them (hit) and cannot evict them.
  if (!MULTI) mq = 1;
  const int km = k + mq - 1;   // middle picks of one list relative to this context
  for (int qj = 0; qj < (MULTI ? mq : 1); ++qj) {
  const int h0 = hand;
  int n = n_next;
  if (threadIdx.x == 0) {   // nobody reads these between the previous list's last barrier and the next
    s_nm = 0;
    s_nmid = 0;
    s_tlast = -1;
  }
  if (n < 0 || n > cap) {
    if (threadIdx.x == 0) raise_flag(flags, SKV_FLAG_TIER_INPUT);
    n = n < 0 ? 0 : cap;
  }
  const int32_t* ib = idx + ((size_t)b * mq + qj) * cap;
  int32_t* rb = rows + ((size_t)b * mq + qj) * cap;
  __syncthreads();

  // phase A: classify; hits refresh their slot; misses listed in input order
  const uint64_t lt_mask = lane == 0 ? 0ull : (~0ull >> (64 - lane));
  for (int base = 0; base < n; base += blockDim.x) {
    const int i = base + threadIdx.x;
    bool miss = false, mid = false;
    int p = 0;
    if (i < n) {
      p = ib[i];
      const bool sorted = i == 0 || ib[i - 1] < p;
      if (p < 0 || p >= T || !sorted) {
        s_bad = 1;
        rb[i] = 0;
      } else if (p < S) {
        rb[i] = p;
      } else if (p >= T - L) {
        const int r = (p - T0) % L;   // tail ring anchored at the creation context
        rb[i] = S + (r < 0 ? r + L : r);
      } else {
        mid = true;
        const int s = sop[p];
        if (s >= 0) {
          s_ref[s] = 1;
          s_last[s] = step;
          rb[i] = S + L + s;
        } else {
          miss = true;
        }
      }
    }
    const uint64_t m = __ballot(miss);
    const uint64_t mm = __ballot(mid);
    if (lane == 0) {
      s_wsum[wave] = (uint32_t)__popcll(m);
      atomicAdd(&s_nmid, (int)__popcll(mm));
    }
    __syncthreads();
    int off = s_nm;
    for (int w = 0; w < wave; ++w) off += (int)s_wsum[w];
    if (miss) {
      const int at = off + (int)__popcll(m & lt_mask);
      if (at < km) {
        s_miss[at] = i;
        s_mpos[at] = p;
      } else {
        rb[i] = 0;      // more middle picks than the budget: not placed, flagged
        s_bad = 1;
      }
    }
    __syncthreads();
    if (threadIdx.x == 0) {
      int tot = 0;
      for (int w = 0; w < (int)(blockDim.x >> 6); ++w) tot += (int)s_wsum[w];
      s_nm += tot;
    }
    __syncthreads();
  }
  // a victim always exists when fewer slots are pinned than exist: at most the
  // middle picks of this step plus those of the previous W-1 steps (LRU: the
  // slots not used in this step are the candidates)
  const bool fits = POLICY == SKV_TIER_LRU ? (int64_t)s_nmid <= (int64_t)n_slots
                                           : (int64_t)s_nmid < (int64_t)n_slots;
  const int nm = fits ? min(s_nm, km) : 0;
  if (!fits) {
    for (int mi = threadIdx.x; mi < min(s_nm, km); mi += blockDim.x) rb[s_miss[mi]] = 0;
    if (threadIdx.x == 0) s_bad = 1;
  }
  __syncthreads();

  constexpr int kRun = kMaxSlots / kResolveThreads;
  if constexpr (POLICY == SKV_TIER_LRU) {
    // phase B (LRU): age key u = last - kNoStep of the slots not used in this
    // step; v = the nm-th smallest u, need = how many slots of age v are taken
    __shared__ uint32_t s_hist[256];
    __shared__ uint32_t s_sel[2];
    uint32_t v = 0, need = (uint32_t)nm;
    // ages relative to the oldest candidate: leading rounds whose digit is 0
    // for every candidate are skipped (usually one round is left)
    uint32_t umin = 0xFFFFFFFFu, umax = 0u, ncand = 0u;
    for (int j = threadIdx.x; j < n_slots; j += blockDim.x)
      if (s_last[j] < step) {
        const uint32_t u = (uint32_t)(s_last[j] - kNoStep);
        umin = min(umin, u);
        umax = max(umax, u);
        ++ncand;
      }
    umin = ~wave_max(~umin);
    umax = wave_max(umax);
    ncand = wave_sum(ncand);
    if (lane == 0) {
      s_hist[wave] = umin;
      s_hist[16 + wave] = umax;
      s_hist[32 + wave] = ncand;
    }
    __syncthreads();
    ncand = 0u;
    for (int w = 0; w < (int)(blockDim.x >> 6); ++w) {
      umin = min(umin, s_hist[w]);
      umax = max(umax, s_hist[16 + w]);
      ncand += s_hist[32 + w];
    }
    __syncthreads();
    const uint32_t span = umax >= umin ? umax - umin : 0u;
    const int top_bits = span ? 32 - __clz((int)span) : 0;
    // Fewer candidates than misses (pick lists of one step that do not fit
    // together, or a reused step number): every candidate is a victim, taken
    // in slot order, and the misses left over are flagged below -- the slot
    // table that remains does not depend on anything but the inputs.
    if (nm > 0 && ncand <= (uint32_t)nm) {
      v = 0xFFFFFFFFu;
      need = 0u;
    } else if (nm > 0) {
      for (int shift = 24; shift >= 0; shift -= 8) {
        if (shift > 0 && shift >= top_bits) continue;   // digit 0 for every candidate
        for (int i = threadIdx.x; i < 256; i += blockDim.x) s_hist[i] = 0u;
        __syncthreads();
        for (int j = threadIdx.x; j < n_slots; j += blockDim.x) {
          if (s_last[j] < step) {
            const uint32_t u = (uint32_t)(s_last[j] - kNoStep) - umin;
            if (((uint64_t)(u ^ v) >> (shift + 8)) == 0) atomicAdd(&s_hist[(u >> shift) & 255u], 1u);
          }
        }
        __syncthreads();
        if (wave == 0) {
          // lane l scans bins 4l..4l+3; the lane whose range holds the need-th
          // candidate picks the bin
          const uint32_t c0 = s_hist[4 * lane], c1 = s_hist[4 * lane + 1], c2 = s_hist[4 * lane + 2],
                         c3 = s_hist[4 * lane + 3];
          const uint32_t tot = c0 + c1 + c2 + c3;
          const uint32_t incl = wave_incl_scan(tot), excl = incl - tot;
          const uint64_t hit = __ballot(excl < need && need <= incl);
          // hit is never empty: the candidates number at least need
          if (hit && lane == (int)__ffsll((unsigned long long)hit) - 1) {
            uint32_t cum = excl;
            int bin = 4 * lane;
            if (cum + c0 < need) { cum += c0; ++bin;
              if (cum + c1 < need) { cum += c1; ++bin;
                if (cum + c2 < need) { cum += c2; ++bin; } } }
            s_sel[0] = v | ((uint32_t)bin << shift);
            s_sel[1] = need - cum;
          }
        }
        __syncthreads();
        v = s_sel[0];
        need = s_sel[1];
        __syncthreads();
      }
    }
    // thread t owns slots [kRun*t, kRun*t + kRun): index order
    const int d0 = kRun * (int)threadIdx.x;
    uint32_t ltm = 0, eqm = 0;
#pragma unroll
    for (int r = 0; r < kRun; ++r) {
      const int j = d0 + r;
      if (nm > 0 && j < n_slots && s_last[j] < step) {
        const uint32_t u = (uint32_t)(s_last[j] - kNoStep) - umin;
        ltm |= (uint32_t)(u < v) << r;
        eqm |= (uint32_t)(u == v) << r;
      }
    }
    uint32_t eq_before = block_excl_scan((uint32_t)__popc(eqm), s_wsum, nullptr);
    uint32_t vm = ltm;
#pragma unroll
    for (int r = 0; r < kRun; ++r)
      if (eqm & (1u << r)) {
        if (eq_before < need) vm |= 1u << r;
        ++eq_before;
      }
    uint32_t n_victims = 0;
    uint32_t vr = block_excl_scan((uint32_t)__popc(vm), s_wsum, &n_victims);
#pragma unroll
    for (int r = 0; r < kRun; ++r) {
      if (vm & (1u << r)) {
        const int j = d0 + r, mi = (int)vr++;
        if (mi < nm) {   // the victims are exactly nm; kept as a guard
          const int p = s_mpos[mi], i = s_miss[mi];
          const int old = s_pos[j];
          if (old >= 0) sop[old] = -1;
          s_pos[j] = p;
          s_last[j] = step;
          sop[p] = j;
          rb[i] = S + L + j;
          miss_pos[(size_t)b * mstride + moff + mi] = p;
          miss_slot[(size_t)b * mstride + moff + mi] = j;
        }
      }
    }
    // fewer candidates than misses only if a step number was reused (its
    // slots then look used in this step): the rest are not placed, flagged
    const int placed = min(nm, (int)n_victims);
    for (int mi = placed + (int)threadIdx.x; mi < nm; mi += blockDim.x) rb[s_miss[mi]] = 0;
    __syncthreads();
    if (threadIdx.x == 0) {
      s_moff = moff + placed;
      s_hand = h0;
      atomicAdd(&counters[0], (unsigned long long)s_nmid);
      atomicAdd(&counters[1], (unsigned long long)(s_nmid - nm));
      atomicAdd(&counters[2], (unsigned long long)nm);
      if (placed < nm) s_bad = 1;
    }
    __syncthreads();
  } else {

  // phase B: thread t owns the slots at hand distance [kRun*t, kRun*t + kRun)
  const int old_limit = step - W;   // last <= step - W: outside the window
  const int d0 = kRun * (int)threadIdx.x;
  uint32_t fmask = 0, rmask = 0;
#pragma unroll
  for (int r = 0; r < kRun; ++r) {
    const int t = d0 + r;
    if (t < n_slots) {
      const int j = h0 + t < n_slots ? h0 + t : h0 + t - n_slots;
      const int ps = s_pos[j];
      const bool unp = s_last[j] <= old_limit;
      const int rf = s_ref[j];
      fmask |= (uint32_t)(ps < 0 || (unp && rf == 0)) << r;
      rmask |= (uint32_t)(ps >= 0 && unp && rf == 1) << r;
    }
  }
  uint32_t both = 0;
  const uint32_t pre = block_excl_scan((uint32_t)__popc(fmask) | ((uint32_t)__popc(rmask) << 16), s_wsum,
                                       &both);
  const int nfree = (int)(both & 0xFFFFu), nref = (int)(both >> 16);
  const bool sweep = nm > nfree;   // the hand goes all the way round
  const int placed = min(nm, nfree + nref);
  int fr = (int)(pre & 0xFFFFu), rr = (int)(pre >> 16);
  auto take = [&](int mi, int j, int t) {
    const int p = s_mpos[mi], i = s_miss[mi];
    const int old = s_pos[j];
    if (old >= 0) sop[old] = -1;
    s_pos[j] = p;
    s_ref[j] = 1;
    s_last[j] = step;
    sop[p] = j;
    rb[i] = S + L + j;
    miss_pos[(size_t)b * mstride + moff + mi] = p;
    miss_slot[(size_t)b * mstride + moff + mi] = j;
    if (mi == placed - 1) s_tlast = t;
  };
  uint32_t rleft = 0;   // referenced slots not taken
#pragma unroll
  for (int r = 0; r < kRun; ++r) {
    const int t = d0 + r;
    const int j = h0 + t < n_slots ? h0 + t : h0 + t - n_slots;
    if (fmask & (1u << r)) {
      if (fr < placed) take(fr, j, t);
      ++fr;
    } else if (rmask & (1u << r)) {
      const int mi = nfree + rr;
      if (sweep && mi < placed) take(mi, j, t);
      else rleft |= 1u << r;
      ++rr;
    }
  }
  __syncthreads();
  // bits of the referenced slots the hand passed are cleared
  const int tlast = s_tlast;
#pragma unroll
  for (int r = 0; r < kRun; ++r) {
    const int t = d0 + r;
    if ((rleft & (1u << r)) && (sweep || t < tlast)) {
      const int j = h0 + t < n_slots ? h0 + t : h0 + t - n_slots;
      s_ref[j] = 0;
    }
  }
  // misses nothing could be evicted for (cannot happen when the slots
  // outnumber the picks of W steps)
  for (int mi = placed + (int)threadIdx.x; mi < nm; mi += blockDim.x) rb[s_miss[mi]] = 0;
  if (threadIdx.x == 0) {
    if (placed < nm) s_bad = 1;
    s_hand = placed > 0 ? (h0 + tlast + 1 < n_slots ? h0 + tlast + 1 : h0 + tlast + 1 - n_slots) : h0;
    s_moff = moff + placed;
    atomicAdd(&counters[0], (unsigned long long)s_nmid);
    atomicAdd(&counters[1], (unsigned long long)(s_nmid - nm));
    atomicAdd(&counters[2], (unsigned long long)nm);
  }
  __syncthreads();
  }   // policy
  hand = s_hand;
  moff = s_moff;
  if (qj + 1 < mq) n_next = n_sel[(size_t)b * mq + qj + 1];
  }   // pick lists
  if (threadIdx.x == 0) {
    miss_count[b] = moff;
    hand_arr[b] = hand;
    if (s_bad) raise_flag(flags, SKV_FLAG_TIER_INPUT);
  }
  for (int i = threadIdx.x; i < n_slots; i += blockDim.x) {
    sp[i] = s_pos[i];
    sl[i] = s_last[i];
    sr[i] = (int32_t)s_ref[i];
  }
}

// Reads missed host records over PCIe and writes int8 rows into their slots.
// One wave per (miss, KV head): lanes 0-31 the K row, 32-63 the V row, 8 dims each.
__global__ __launch_bounds__(256) void tier_fetch_kernel(
    const uint8_t* __restrict__ host, const int32_t* __restrict__ miss_pos,
    const int32_t* __restrict__ miss_slot, const int32_t* __restrict__ miss_count,
    int8_t* __restrict__ res_k, int8_t* __restrict__ res_v, uint16_t* __restrict__ res_ks,
    uint16_t* __restrict__ res_vs, int64_t host_ctx, int Hkv, int mstride, int64_t res_rows, int res_off) {
  constexpr int D = 256;
  constexpr int ROWB = D / 2 + 2 * (D / 64);   // 136
  const int b = blockIdx.y;
  const int lane = threadIdx.x & 63;
  const int half = lane >> 5, ln = lane & 31;
  const int nm = miss_count[b];
  const int nwaves = gridDim.x * (blockDim.x >> 6);
  for (int task = blockIdx.x * (blockDim.x >> 6) + (threadIdx.x >> 6); task < nm * Hkv; task += nwaves) {
    const int mi = task / Hkv, h = task % Hkv;
    const int p = miss_pos[(size_t)b * mstride + mi];
    const int slot = miss_slot[(size_t)b * mstride + mi];
    const uint8_t* row = host + (((size_t)b * host_ctx + p) * Hkv + h) * (2 * ROWB) + half * ROWB;
    const uint32_t codes = *reinterpret_cast<const uint32_t*>(row + 4 * ln);
    const uint2 sc = *reinterpret_cast<const uint2*>(row + D / 2);
    const float g0 = half_bits_to_float((uint16_t)(sc.x & 0xFFFF));
    const float g1 = half_bits_to_float((uint16_t)(sc.x >> 16));
    const float g2 = half_bits_to_float((uint16_t)(sc.y & 0xFFFF));
    const float g3 = half_bits_to_float((uint16_t)(sc.y >> 16));
    const float gmax = fmaxf(fmaxf(g0, g1), fmaxf(g2, g3));
    // fp32 quotients via one fp64 divide + one rounding (= correctly rounded fp32)
    const __half sp_h = __float2half_rn((float)((double)(gmax * 7.0f) / 127.0));
    const float spf = __half2float(sp_h);
    const int grp = ln >> 3;    // 8 dims per lane, 64 dims per group
    const float gs = grp == 0 ? g0 : (grp == 1 ? g1 : (grp == 2 ? g2 : g3));
    uint32_t out[2] = {0u, 0u};
    if (spf != 0.0f) {
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        int c = (int)((codes >> (4 * e)) & 0xFu);
        c = (c ^ 8) - 8;
        float r = rintf((float)((double)((float)c * gs) / (double)spf));
        r = fminf(fmaxf(r, -127.0f), 127.0f);
        out[e >> 2] |= ((uint32_t)(uint8_t)(int8_t)(int)r) << (8 * (e & 3));
      }
    }
    const size_t rr = ((size_t)b * res_rows + res_off + slot) * Hkv + h;
    int8_t* dst = (half ? res_v : res_k) + rr * D + 8 * ln;
    *reinterpret_cast<uint2*>(dst) = make_uint2(out[0], out[1]);
    if (ln == 0) (half ? res_vs : res_ks)[rr] = __half_as_ushort(sp_h);
  }
}

}  // namespace
}  // namespace skv

// ---------------------------------------------------------------------------
// host side
// ---------------------------------------------------------------------------
namespace skv {
skv_status set_error(skv_status s, const char* fmt, ...);
skv_status validate_desc(const skv_layer_desc* d);
}  // namespace skv

using skv::set_error;

static void tier_free(skv_tier* t) {
  if (!t) return;
  void* dev[] = {t->res_k, t->res_v, t->res_ks, t->res_vs, t->slot_pos, t->slot_last, t->slot_ref,
                 t->hand, t->slot_of_pos, t->ctx_dev, t->miss_pos, t->miss_slot, t->miss_count,
                 t->counters, t->flags};
  for (void* p : dev)
    if (p) (void)hipFree(p);
  if (t->own_host && t->host) (void)hipHostFree(t->host);
  delete t;
}

extern "C" skv_status sparsekv_tier_create(const skv_tier_desc* d, skv_tier** out) {
  if (!d || !out) return set_error(SKV_ERR_INVALID, "tier_create: NULL argument");
  *out = nullptr;
  constexpr size_t kMinDesc = offsetof(skv_tier_desc, policy);
  if (d->struct_size < kMinDesc)
    return set_error(SKV_ERR_INVALID, "tier_create: struct_size %u < %zu", d->struct_size, kMinDesc);
  const int policy = d->struct_size >= sizeof(skv_tier_desc) ? d->policy : SKV_TIER_CLOCK;
  if (policy != SKV_TIER_CLOCK && policy != SKV_TIER_LRU)
    return set_error(SKV_ERR_INVALID, "tier_create: policy %d unknown", policy);
  skv_status s = skv::validate_desc(&d->layer);
  if (s != SKV_OK) return s;
  const skv_layer_desc& L = d->layer;
  if (L.index_mode != SKV_INDEX_SKETCH_INT4 || L.kv_dtype != SKV_KV_I8_ROWSCALE || L.head_dim != 256)
    return set_error(SKV_ERR_UNSUPPORTED, "tier: needs token mode, int8 K/V rows and head_dim 256");
  if (d->ctx < 1 || d->ctx > L.max_ctx)
    return set_error(SKV_ERR_INVALID, "tier: ctx %d outside [1, max_ctx=%d]", d->ctx, L.max_ctx);
  if (policy == SKV_TIER_LRU) {
    if (d->n_slots < L.topk || d->n_slots > skv::kMaxSlots)
      return set_error(SKV_ERR_INVALID, "tier: n_slots %d must be in [topk = %d, %d]", d->n_slots,
                       L.topk, skv::kMaxSlots);
  } else {
    if (d->window < 1) return set_error(SKV_ERR_INVALID, "tier: window %d < 1", d->window);
    if ((int64_t)d->n_slots <= (int64_t)d->window * L.topk || d->n_slots > skv::kMaxSlots)
      return set_error(SKV_ERR_INVALID, "tier: n_slots %d must exceed window*topk = %lld and be <= %d",
                       d->n_slots, (long long)d->window * L.topk, skv::kMaxSlots);
  }
  skv_tier* t = new (std::nothrow) skv_tier();
  if (!t) return set_error(SKV_ERR_OOM, "tier: host allocation failed");
  memset(t, 0, sizeof(*t));
  memcpy(&t->desc, d, std::min<size_t>(d->struct_size, sizeof(skv_tier_desc)));
  t->policy = policy;
  t->B = L.batch; t->T0 = d->ctx; t->cap_ctx = L.max_ctx; t->S = L.n_sink; t->L = L.n_tail; t->k = L.topk;
  t->Hkv = L.n_kv_heads; t->D = L.head_dim; t->n_slots = d->n_slots; t->W = d->window;
  t->cap = skv::select_capacity(L);
  t->mstride = skv::kMaxQueries * (t->k + skv::kMaxQueries);
  t->row_bytes = t->D / 2 + 2 * (t->D / 64);
  t->rec_bytes = 2 * t->row_bytes;
  t->res_rows = (int64_t)t->S + t->L + t->n_slots;
  const size_t host_bytes = (size_t)t->B * t->cap_ctx * t->Hkv * t->rec_bytes;
  if (d->host_records) {
    t->host = d->host_records;
    t->own_host = false;
  } else {
    if (hipHostMalloc(&t->host, host_bytes, hipHostMallocMapped | hipHostMallocPortable) != hipSuccess) {
      t->host = nullptr;
      tier_free(t);
      return set_error(SKV_ERR_OOM, "tier: hipHostMalloc of %zu bytes failed", host_bytes);
    }
    t->own_host = true;
    memset(t->host, 0, host_bytes);
  }
  void* hd = nullptr;
  if (hipHostGetDevicePointer(&hd, t->host, 0) != hipSuccess || !hd) {
    (void)hipGetLastError();
    tier_free(t);
    return set_error(SKV_ERR_HOST_MEMORY, "tier: host records are not pinned and device-mapped");
  }
  t->host_dev = (const uint8_t*)hd;
  const size_t rr = (size_t)t->B * t->res_rows * t->Hkv;
  const size_t ns = (size_t)t->B * t->n_slots;
  bool ok = hipMalloc(&t->res_k, rr * t->D) == hipSuccess &&
            hipMalloc(&t->res_v, rr * t->D) == hipSuccess &&
            hipMalloc(&t->res_ks, rr * 2) == hipSuccess &&
            hipMalloc(&t->res_vs, rr * 2) == hipSuccess &&
            hipMalloc(&t->slot_pos, ns * 4) == hipSuccess &&
            hipMalloc(&t->slot_last, ns * 4) == hipSuccess &&
            hipMalloc(&t->slot_ref, ns * 4) == hipSuccess &&
            hipMalloc(&t->hand, (size_t)t->B * 4) == hipSuccess &&
            hipMalloc(&t->slot_of_pos, (size_t)t->B * t->cap_ctx * 4) == hipSuccess &&
            hipMalloc(&t->ctx_dev, (size_t)t->B * 4) == hipSuccess &&
            hipMalloc(&t->miss_pos, (size_t)t->B * t->mstride * 4) == hipSuccess &&
            hipMalloc(&t->miss_slot, (size_t)t->B * t->mstride * 4) == hipSuccess &&
            hipMalloc(&t->miss_count, (size_t)t->B * 4) == hipSuccess &&
            hipMalloc(&t->counters, 3 * sizeof(unsigned long long)) == hipSuccess &&
            hipMalloc(&t->flags, 256) == hipSuccess;
  if (!ok) {
    (void)hipGetLastError();
    tier_free(t);
    return set_error(SKV_ERR_OOM, "tier: device allocation failed");
  }
  if (hipMemset(t->res_k, 0, rr * t->D) != hipSuccess || hipMemset(t->res_v, 0, rr * t->D) != hipSuccess ||
      hipMemset(t->res_ks, 0, rr * 2) != hipSuccess || hipMemset(t->res_vs, 0, rr * 2) != hipSuccess ||
      hipMemset(t->flags, 0, 256) != hipSuccess) {
    tier_free(t);
    return set_error(SKV_ERR_HIP, "tier: initial clear failed");
  }
  {
    std::vector<int32_t> c0((size_t)t->B, t->T0);
    if (hipMemcpy(t->ctx_dev, c0.data(), c0.size() * 4, hipMemcpyHostToDevice) != hipSuccess) {
      tier_free(t);
      return set_error(SKV_ERR_HIP, "tier: context upload failed");
    }
  }
  hipLaunchKernelGGL(skv::tier_reset_kernel, dim3(256), dim3(256), 0, 0, t->slot_pos, t->slot_last,
                     t->slot_ref, t->hand, t->slot_of_pos, t->counters, t->B, t->n_slots, t->cap_ctx);
  if (hipGetLastError() != hipSuccess || hipDeviceSynchronize() != hipSuccess) {
    tier_free(t);
    return set_error(SKV_ERR_HIP, "tier: reset kernel failed");
  }
  *out = t;
  return SKV_OK;
}

extern "C" void* sparsekv_tier_host_records(skv_tier* t) { return t ? t->host : nullptr; }

extern "C" skv_status sparsekv_tier_resident(skv_tier* t, skv_kv_view* v) {
  if (!t || !v) return set_error(SKV_ERR_INVALID, "tier_resident: NULL argument");
  v->k = t->res_k;
  v->v = t->res_v;
  v->k_scale = t->res_ks;
  v->v_scale = t->res_vs;
  v->rows = t->res_rows;
  return SKV_OK;
}

extern "C" skv_status sparsekv_tier_load_resident(skv_tier* t, const int8_t* k, const int8_t* v,
                                                  const uint16_t* ks, const uint16_t* vs,
                                                  void* stream) {
  if (!t || !k || !v || !ks || !vs) return set_error(SKV_ERR_INVALID, "tier_load_resident: NULL argument");
  if (t->appends)
    return set_error(SKV_ERR_STATE, "tier_load_resident: the tier has appended tokens (load the creation context only)");
  hipStream_t st = (hipStream_t)stream;
  const size_t nres = (size_t)(t->S + t->L);
  if (nres == 0) return SKV_OK;
  const size_t rowb = (size_t)t->Hkv * t->D;   // bytes of one resident row (all heads)
  const size_t sclb = (size_t)t->Hkv * 2;
  for (int b = 0; b < t->B; ++b) {
    const size_t dst = (size_t)b * t->res_rows;
    const size_t src = (size_t)b * nres;
    if (hipMemcpyAsync(t->res_k + dst * rowb, k + src * rowb, nres * rowb, hipMemcpyDeviceToDevice, st) != hipSuccess ||
        hipMemcpyAsync(t->res_v + dst * rowb, v + src * rowb, nres * rowb, hipMemcpyDeviceToDevice, st) != hipSuccess ||
        hipMemcpyAsync(t->res_ks + dst * t->Hkv, ks + src * t->Hkv, nres * sclb, hipMemcpyDeviceToDevice, st) != hipSuccess ||
        hipMemcpyAsync(t->res_vs + dst * t->Hkv, vs + src * t->Hkv, nres * sclb, hipMemcpyDeviceToDevice, st) != hipSuccess)
      return set_error(SKV_ERR_HIP, "tier_load_resident: copy failed");
  }
  return SKV_OK;
}

static skv_status tier_resolve_lists(skv_tier* t, int32_t n_query, const int32_t* idx,
                                     const int32_t* n_sel, int32_t step, int32_t* rows,
                                     void* stream) {
  if (!t || !idx || !n_sel || !rows) return set_error(SKV_ERR_INVALID, "tier_resolve: NULL argument");
  if (n_query < 1 || n_query > skv::kMaxQueries)
    return set_error(SKV_ERR_UNSUPPORTED, "tier_resolve: n_query %d outside [1, %d]", n_query,
                     skv::kMaxQueries);
  hipStream_t st = (hipStream_t)stream;
#define SKV_RESOLVE(POL)                                                                           \
  hipLaunchKernelGGL((skv::tier_resolve_kernel<POL, MUL>), dim3(t->B), dim3(skv::kResolveThreads), 0, st, \
                     idx, n_sel, rows, t->slot_pos, t->slot_last, t->slot_ref, t->hand,            \
                     t->slot_of_pos, t->miss_pos, t->miss_slot, t->miss_count, t->counters,        \
                     t->flags, t->ctx_dev, t->T0, t->cap_ctx, t->S, t->L, t->k, t->n_slots, t->W,  \
                     t->cap, step, n_query, t->mstride)
  if (n_query == 1) {
    constexpr bool MUL = false;
    if (t->policy == SKV_TIER_LRU) SKV_RESOLVE(SKV_TIER_LRU);
    else SKV_RESOLVE(SKV_TIER_CLOCK);
  } else {
    constexpr bool MUL = true;
    if (t->policy == SKV_TIER_LRU) SKV_RESOLVE(SKV_TIER_LRU);
    else SKV_RESOLVE(SKV_TIER_CLOCK);
  }
#undef SKV_RESOLVE
  if (hipGetLastError() != hipSuccess) return set_error(SKV_ERR_HIP, "tier_resolve: launch failed");
  hipEvent_t ev0 = nullptr, ev1 = nullptr;
  if (skv::timer_next(skv::kTimerStream, &ev0, &ev1))   // diagnostic timer (sparsekv_timer_enable)
    hipExtLaunchKernelGGL(skv::tier_fetch_kernel, dim3(128, t->B), dim3(256), 0, st, ev0, ev1, 0,
                          t->host_dev, t->miss_pos, t->miss_slot, t->miss_count, t->res_k, t->res_v,
                          t->res_ks, t->res_vs, (int64_t)t->cap_ctx, t->Hkv, t->mstride, t->res_rows,
                          t->S + t->L);
  else
    hipLaunchKernelGGL(skv::tier_fetch_kernel, dim3(128, t->B), dim3(256), 0, st, t->host_dev,
                       t->miss_pos, t->miss_slot, t->miss_count, t->res_k, t->res_v, t->res_ks,
                       t->res_vs, (int64_t)t->cap_ctx, t->Hkv, t->mstride, t->res_rows, t->S + t->L);
  if (hipGetLastError() != hipSuccess) return set_error(SKV_ERR_HIP, "tier_fetch: launch failed");
  t->steps += 1;
  return SKV_OK;
}

extern "C" skv_status sparsekv_tier_resolve(skv_tier* t, const int32_t* idx, const int32_t* n_sel,
                                            int32_t step, int32_t* rows, void* stream) {
  return tier_resolve_lists(t, 1, idx, n_sel, step, rows, stream);
}

extern "C" skv_status sparsekv_tier_resolve_multi(skv_tier* t, int32_t n_query, const int32_t* idx,
                                                  const int32_t* n_sel, int32_t step, int32_t* rows,
                                                  void* stream) {
  return tier_resolve_lists(t, n_query, idx, n_sel, step, rows, stream);
}

extern "C" skv_status sparsekv_tier_append(skv_tier* t, int32_t* ctx_len, const void* k_new,
                                           const void* v_new, const float* basis, void* index_keys,
                                           uint16_t* index_scale, void* stream) {
  if (!t || !ctx_len || !k_new || !v_new || !basis || !index_keys || !index_scale)
    return set_error(SKV_ERR_INVALID, "tier_append: NULL argument");
  const skv::AppendTarget tg{t->ctx_dev, const_cast<uint8_t*>(t->host_dev), (int64_t)t->cap_ctx, t->S,
                             t->L, t->T0};
  skv_kv_view res;
  res.k = t->res_k;
  res.v = t->res_v;
  res.k_scale = t->res_ks;
  res.v_scale = t->res_vs;
  res.rows = t->res_rows;
  if (skv::launch_tier_append(t->desc.layer, ctx_len, k_new, v_new, basis, res, index_keys,
                              index_scale, t->flags, tg, (hipStream_t)stream) != hipSuccess)
    return set_error(SKV_ERR_HIP, "tier_append: launch failed");
  t->appends += 1;
  return SKV_OK;
}

extern "C" skv_status sparsekv_tier_stats(skv_tier* t, skv_tier_stats* out, void* stream) {
  if (!t || !out) return set_error(SKV_ERR_INVALID, "tier_stats: NULL argument");
  unsigned long long c[3] = {0, 0, 0};
  uint32_t fl = 0;
  if (hipStreamSynchronize((hipStream_t)stream) != hipSuccess ||
      hipMemcpy(c, t->counters, sizeof(c), hipMemcpyDeviceToHost) != hipSuccess ||
      hipMemcpy(&fl, t->flags, 4, hipMemcpyDeviceToHost) != hipSuccess)
    return set_error(SKV_ERR_HIP, "tier_stats: readback failed");
  out->steps = t->steps;
  out->picks = (int64_t)c[0];
  out->hits = (int64_t)c[1];
  out->misses = (int64_t)c[2];
  out->host_bytes = (int64_t)c[2] * t->Hkv * t->rec_bytes;
  if (fl) return set_error(SKV_ERR_STATE, "tier: device flags 0x%x (invalid selection or append input)", fl);
  return SKV_OK;
}

extern "C" skv_status sparsekv_tier_slots(skv_tier* t, int32_t* slot_pos_host, void* stream) {
  if (!t || !slot_pos_host) return set_error(SKV_ERR_INVALID, "tier_slots: NULL argument");
  if (hipStreamSynchronize((hipStream_t)stream) != hipSuccess ||
      hipMemcpy(slot_pos_host, t->slot_pos, (size_t)t->B * t->n_slots * 4, hipMemcpyDeviceToHost) != hipSuccess)
    return set_error(SKV_ERR_HIP, "tier_slots: readback failed");
  return SKV_OK;
}

extern "C" skv_status sparsekv_tier_reset(skv_tier* t, void* stream) {
  if (!t) return set_error(SKV_ERR_INVALID, "tier_reset: NULL argument");
  hipLaunchKernelGGL(skv::tier_reset_kernel, dim3(256), dim3(256), 0, (hipStream_t)stream,
                     t->slot_pos, t->slot_last, t->slot_ref, t->hand, t->slot_of_pos, t->counters,
                     t->B, t->n_slots, t->cap_ctx);
  if (hipGetLastError() != hipSuccess) return set_error(SKV_ERR_HIP, "tier_reset: launch failed");
  t->steps = 0;
  return SKV_OK;
}

extern "C" void sparsekv_tier_destroy(skv_tier* t) {
  if (!t) return;
  (void)hipDeviceSynchronize();
  tier_free(t);
}
