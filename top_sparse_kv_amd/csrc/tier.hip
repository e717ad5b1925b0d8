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
// Residency states (page "vLLM's Hybrid HiSparse Triples Concurrent Requests
// on Million-Token Contexts", section "Three residency states, one block
// pool"): a page table per sequence maps pages of P positions to blocks of a
// device pool (full residency: every page mapped; mixed: some; none: no page).
// A middle pick of a mapped page is read where it sits in the pool; the other
// middle picks go through the hot buffer.
//
// Per step one kernel -- the single fused resolver the residency section
// describes -- with 1 + F workgroups per sequence.  The first resolves the
// picks (in place, hit, miss) and places the misses; the other F read the
// missed records over PCIe and write them into their slots as int8 rows +
// fp16 scales.  Host reads need many compute units in flight (one workgroup
// alone pulls a few GB/s), so the fetch is spread; the resolver publishes the
// misses' positions as soon as they are classified, so the PCIe reads overlap
// the placement, then their slots.  A fetch workgroup only ever waits for the
// resolver of its own sequence, which has a lower workgroup id and is
// dispatched before it; the wait is bounded (a flag is raised if it ends
// without the resolver's word), and the last workgroup of a sequence to
// finish clears the sequence's hand-off words for the next call.
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
  uint32_t* hot_bits;    // [B][hot_words]: bit p set while position p is in the hot buffer
  int hot_words;         // ceil(cap_ctx / 32)
  int32_t* ctx_dev;      // [B] context of each sequence (advanced by sparsekv_tier_append)
  int64_t appends;       // sparsekv_tier_append calls
  int P, page_shift;     // page size (positions, a power of two) and its log2; 0 / 0: no page table
  int pool_pages;        // pool blocks per sequence
  int n_pages;           // pages per sequence: ceil(cap_ctx / P)
  int64_t pool_row0;     // first pool row of a sequence in the resident rows
  int32_t* page_block;   // [B][n_pages] pool block of each page, -1: host only (device)
  int32_t* page_host;    // host mirror of page_block
  int32_t* block_page;   // [B][pool_pages] page held by each block, -1: free (host)
  int n_fetch;           // fetch workgroups per sequence
  int mstride;           // misses per sequence the arrays below hold
  int32_t* miss_pos;     // [B][mstride] resolver -> fetch workgroups
  int32_t* miss_slot;    // [B][mstride]
  int32_t* miss_n;       // [B]
  int32_t* sync;         // [B][4]: positions listed, slots placed, arrivals
  unsigned long long* counters;  // picks, hits, misses, in place
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
                                  int32_t* hand, int32_t* slot_of_pos, uint32_t* hot_bits,
                                  unsigned long long* counters, int B, int n_slots, int cap_ctx,
                                  int hot_words) {
  const size_t tid = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
  const size_t nth = (size_t)gridDim.x * blockDim.x;
  for (size_t i = tid; i < (size_t)B * n_slots; i += nth) {
    slot_pos[i] = -1;
    slot_last[i] = kNoStep;
    slot_ref[i] = 0;
  }
  for (size_t i = tid; i < (size_t)B * cap_ctx; i += nth) slot_of_pos[i] = -1;
  for (size_t i = tid; i < (size_t)B * hot_words; i += nth) hot_bits[i] = 0u;
  for (size_t i = tid; i < (size_t)B; i += nth) hand[i] = 0;
  if (tid < 4) counters[tid] = 0ull;
}

// ---- hand-off between the resolver and the fetch workgroups of a sequence ----
// Words w[0] (miss positions listed), w[1] (slots placed), w[2] (arrivals).
// Everything handed over (positions, slots, counts, the words) is written and
// read with device-scope atomic accesses, which are coherent across the XCDs'
// L2 caches by themselves; so no release or acquire fence is needed.  (A
// device-scope release fence writes the XCD's whole L2 back and here queues
// behind the fetch workgroups' host reads; an acquire fence invalidates it.)
constexpr uint64_t kWaitTicks = 5000000;   // 50 ms of the 100 MHz constant clock

__device__ __forceinline__ void put(int32_t* p, int32_t v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ int32_t get(const int32_t* p) {
  return __hip_atomic_load(const_cast<int32_t*>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// every thread's earlier put()s complete, then word = 1
__device__ __forceinline__ void publish(int32_t* word) {
  __builtin_amdgcn_s_waitcnt(0);   // this thread's stores are acknowledged
  __syncthreads();
  if (threadIdx.x == 0) put(word, 1);
}

// thread 0 polls the word (bounded); false if it never became 1
__device__ __forceinline__ bool wait_word(int32_t* word, uint32_t* flags, int* s_ok) {
  if (threadIdx.x == 0) {
    const uint64_t t0 = wall_clock64();
    int ok = 1;
    while (get(word) == 0) {
      if (wall_clock64() - t0 > kWaitTicks) {
        ok = 0;
        raise_flag(flags, SKV_FLAG_WAIT);
        break;
      }
      __builtin_amdgcn_s_sleep(8);
    }
    *s_ok = ok;
  }
  __syncthreads();
  return *s_ok != 0;
}

// one more workgroup of the sequence done (thread 0); the last of the 1 + F
// clears the words for the next call
__device__ __forceinline__ void arrive(int32_t* w, int n_fetch) {
  const int old = atomicAdd(w + 2, 1);
  if (old == n_fetch) {
    w[0] = 0;
    w[1] = 0;
    w[2] = 0;
  }
}

// Fetch workgroup `part` of F.  Task t = (miss, KV head) = (t / H_kv, t % H_kv);
// round r, batch slot u, workgroup part p, wave w take task
// ((r * BATCH + u) * F + p) * W + w (W waves per workgroup), so every round
// covers BATCH * F * W consecutive tasks; lanes 0-31 handle the K row and
// 32-63 the V row, 8 dims each.  A round reads and converts its records, then
// (first round only) waits for the slots, then stores.  The round count is the
// same for every wave of the workgroup, so the waits' barriers line up.
constexpr int kFetchBatch = 4;
template <int BATCH>
__device__ void fetch_part(const uint8_t* __restrict__ host, const int32_t* mpos, const int32_t* mslot,
                           const int32_t* mcount, int32_t* w, uint32_t* flags, int part, int n_fetch, int b,
                           int64_t host_ctx, int Hkv, int8_t* __restrict__ res_k, int8_t* __restrict__ res_v,
                           uint16_t* __restrict__ res_ks, uint16_t* __restrict__ res_vs, int64_t res_rows,
                           int res_off) {
  constexpr int D = 256;
  constexpr int ROWB = D / 2 + 2 * (D / 64);   // 136
  __shared__ int s_ok[2];   // one word per wait: no wave reads one while thread 0 writes the other
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, nw = (int)(blockDim.x >> 6);
  const int half = lane >> 5, ln = lane & 31;
  const bool listed = wait_word(w + 0, flags, &s_ok[0]);
  const int ntask = listed ? get(mcount) * Hkv : 0;
  const int per_round = BATCH * n_fetch * nw;
  const int rounds = (ntask + per_round - 1) / per_round;   // the same in every wave
  for (int r = 0; r < rounds; ++r) {
    uint2 rowv[BATCH];
    uint16_t sbits[BATCH];
#pragma unroll
    for (int u = 0; u < BATCH; ++u) {
      const int task = ((r * BATCH + u) * n_fetch + part) * nw + wave;
      rowv[u] = make_uint2(0u, 0u);
      sbits[u] = 0;
      if (task < ntask) {
        const int mi = task / Hkv, h = task - mi * Hkv;
        const uint8_t* row = host + (((size_t)b * host_ctx + get(mpos + mi)) * Hkv + h) * (2 * ROWB) + half * ROWB;
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
        uint32_t o2[2] = {0u, 0u};
        if (spf != 0.0f) {
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            int c = (int)((codes >> (4 * e)) & 0xFu);
            c = (c ^ 8) - 8;
            float q = rintf((float)((double)((float)c * gs) / (double)spf));
            q = fminf(fmaxf(q, -127.0f), 127.0f);
            o2[e >> 2] |= ((uint32_t)(uint8_t)(int8_t)(int)q) << (8 * (e & 3));
          }
        }
        rowv[u] = make_uint2(o2[0], o2[1]);
        sbits[u] = __half_as_ushort(sp_h);
      }
    }
    if (r == 0 && !wait_word(w + 1, flags, &s_ok[1])) break;   // workgroup-uniform
#pragma unroll
    for (int u = 0; u < BATCH; ++u) {
      const int task = ((r * BATCH + u) * n_fetch + part) * nw + wave;
      if (task >= ntask) continue;
      const int mi = task / Hkv, h = task - mi * Hkv;
      const int slot = get(mslot + mi);
      if (slot < 0) continue;   // not placed (flagged by the resolver)
      const size_t rr = ((size_t)b * res_rows + res_off + slot) * Hkv + h;
      int8_t* dst = (half ? res_v : res_k) + rr * D + 8 * ln;
      *reinterpret_cast<uint2*>(dst) = rowv[u];
      if (ln == 0) (half ? res_vs : res_ks)[rr] = sbits[u];
    }
  }
  __syncthreads();
  if (threadIdx.x == 0) arrive(w, n_fetch);
}

__global__ void tier_set_page_kernel(int32_t* page_block, int64_t at, int32_t block) {
  page_block[at] = block;
}

// MULTI: several pick lists per sequence (mq of them); one list compiles to
// straight-line code without the loop's live state
template <int POLICY, bool MULTI>
__global__ __launch_bounds__(kResolveThreads) void tier_resolve_kernel(
    const int32_t* __restrict__ idx, const int32_t* __restrict__ n_sel, int32_t* __restrict__ rows,
    int32_t* __restrict__ slot_pos, int32_t* __restrict__ slot_last, int32_t* __restrict__ slot_ref,
    int32_t* __restrict__ hand_arr, int32_t* __restrict__ slot_of_pos,
    uint32_t* __restrict__ hot_bits, int hot_words,
    unsigned long long* __restrict__ counters, uint32_t* __restrict__ flags,
    const int32_t* __restrict__ tier_ctx, int T0, int cap_ctx, int S, int L,
    int k, int n_slots, int W, int cap, int step, int mq,
    const int32_t* __restrict__ page_block, int n_pages, int page_shift, int64_t pool_row0,
    const uint8_t* __restrict__ host, int8_t* __restrict__ res_k, int8_t* __restrict__ res_v,
    uint16_t* __restrict__ res_ks, uint16_t* __restrict__ res_vs, int64_t res_rows, int Hkv,
    int32_t* __restrict__ miss_pos, int32_t* __restrict__ miss_slot, int32_t* __restrict__ miss_n,
    int32_t* __restrict__ sync, int mstride, int n_fetch) {
  __shared__ int32_t s_pos[kMaxSlots];
  __shared__ int32_t s_last[kMaxSlots];
  __shared__ uint8_t s_ref[kMaxSlots];
  __shared__ int32_t s_miss[kMaxListMisses];   // input index of each miss; its slot once placed
  __shared__ int32_t s_mpos[kMaxListMisses];   // its position (read by the serial placement)
  __shared__ uint16_t s_hit[kMaxListMisses];   // one pick list: input index of each hit
  __shared__ uint32_t s_wsum[kResolveThreads / 64];
  // per-wave counts of a classification round (misses, hits, middle, in
  // place), two buffers used by alternate rounds: one barrier per round
  __shared__ __align__(16) uint32_t s_cnt[2][kResolveThreads / 64][4];
  __shared__ int s_nm, s_nh, s_nmid, s_ninp, s_bad, s_tlast, s_hand, s_placed;
  const int b = blockIdx.x / (1 + n_fetch), role = blockIdx.x % (1 + n_fetch);
  if (role != 0) {   // a fetch workgroup (workgroup-uniform, before any barrier of the resolver)
    fetch_part<MULTI ? kFetchBatch / 2 : kFetchBatch>(host, miss_pos + (size_t)b * mstride,
                                                      miss_slot + (size_t)b * mstride, miss_n + b,
                                                      sync + 4 * b, flags, role - 1, n_fetch, b, cap_ctx,
                                                      Hkv, res_k, res_v, res_ks, res_vs, res_rows, S + L);
    return;
  }
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  int32_t* sp = slot_pos + (size_t)b * n_slots;
  int32_t* sl = slot_last + (size_t)b * n_slots;
  int32_t* sr = slot_ref + (size_t)b * n_slots;
  int32_t* sop = slot_of_pos + (size_t)b * cap_ctx;
  uint32_t* hb = hot_bits + (size_t)b * hot_words;
  const int32_t* pgb = page_block ? page_block + (size_t)b * n_pages : nullptr;
  const int pmask = (1 << page_shift) - 1;
  // scalars first: their loads overlap the slot-table copy
  const int T = tier_ctx[b];   // this sequence's context (sinks, middle, tail ring)
  int hand = hand_arr[b];
  int n_next = n_sel[(size_t)b * mq];
  int moff = 0;   // misses handed to the fetch workgroups by the earlier lists
  if constexpr (MULTI) {
    // several lists: the slot table first (one list loads it once the misses
    // are handed over, off the fetch's critical path)
    for (int i = threadIdx.x; i < n_slots; i += blockDim.x) {
      s_pos[i] = sp[i];
      s_last[i] = sl[i];
      s_ref[i] = (uint8_t)sr[i];
    }
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
    s_nh = 0;
    s_nmid = 0;
    s_ninp = 0;
    s_tlast = -1;
  }
  if (n < 0 || n > cap) {
    if (threadIdx.x == 0) raise_flag(flags, SKV_FLAG_TIER_INPUT);
    n = n < 0 ? 0 : cap;
  }
  const int32_t* ib = idx + ((size_t)b * mq + qj) * cap;
  int32_t* rb = rows + ((size_t)b * mq + qj) * cap;
  __syncthreads();

  // phase A: classify; hits refresh their slot; misses listed in input order.
  // The picks of the first kPre rounds and their slot / page lookups are
  // loaded together first (the lookups do not change before the placement),
  // so the rounds cost one pair of dependent round trips, not one each.
  // One list: the hot test reads the bitmap of hot positions instead of the
  // slot of each pick (the picks ascend, so a 64-byte line of bits serves
  // several of them: about a quarter of the scattered lines), and the hits
  // are only listed; their slots are looked up once the misses are handed
  // over.
  constexpr int kPre = 4;
  int pp[kPre], pq[kPre], ps[kPre], pg[kPre];
#pragma unroll
  for (int r = 0; r < kPre; ++r) {
    const int i = r * (int)blockDim.x + (int)threadIdx.x;
    pp[r] = i < n ? ib[i] : -1;
    pq[r] = (i < n && i > 0) ? ib[i - 1] : INT32_MIN;
  }
#pragma unroll
  for (int r = 0; r < kPre; ++r) {
    const int p = pp[r];
    const bool midr = p >= S && p < T - L;   // then 0 <= p < T <= cap_ctx
    if constexpr (MULTI) ps[r] = midr ? sop[p] : -1;
    else ps[r] = midr ? (int)hb[p >> 5] : 0;   // the bitmap word of p
    pg[r] = (midr && pgb) ? pgb[p >> page_shift] : -1;
  }
  const uint64_t lt_mask = lane == 0 ? 0ull : (~0ull >> (64 - lane));
  int round = 0;
  int nm_run = 0, nh_run = 0, nmid_run = 0, ninp_run = 0;   // the same in every thread
  for (int base = 0; base < n; base += blockDim.x, ++round) {
    const int i = base + threadIdx.x;
    bool miss = false, mid = false, inpl = false;
    int p = pp[0], prev = pq[0], s_pre = ps[0], blk_pre = pg[0];
#pragma unroll
    for (int u = 0; u + 1 < kPre; ++u) {   // static indices: the next round moves to slot 0
      pp[u] = pp[u + 1];
      pq[u] = pq[u + 1];
      ps[u] = ps[u + 1];
      pg[u] = pg[u + 1];
    }
    if (round >= kPre && i < n) {   // rounds past the prefetched ones load here
      p = ib[i];
      prev = i > 0 ? ib[i - 1] : INT32_MIN;
      const bool midr = p >= S && p < T - L;
      if constexpr (MULTI) s_pre = midr ? sop[p] : -1;
      else s_pre = midr ? (int)hb[p >> 5] : 0;
      blk_pre = (midr && pgb) ? pgb[p >> page_shift] : -1;
    }
    bool hit = false;
    if (i < n) {
      const bool sorted = i == 0 || prev < p;
      if (p < 0 || p >= T || !sorted) {
        s_bad = 1;
        rb[i] = 0;
      } else if (p < S) {
        rb[i] = p;
      } else if (p >= T - L) {
        const int r = (p - T0) % L;   // tail ring anchored at the creation context
        rb[i] = S + (r < 0 ? r + L : r);
      } else {
        // a mapped page wins over the hot buffer
        const int blk = blk_pre;
        const int s = s_pre;
        if (blk >= 0) {
          inpl = true;
          rb[i] = (int)(pool_row0 + ((int64_t)blk << page_shift) + (p & pmask));
        } else if (MULTI ? s >= 0 : (((uint32_t)s >> (p & 31)) & 1u) != 0u) {
          mid = true;
          if constexpr (MULTI) {
            s_ref[s] = 1;
            s_last[s] = step;
            rb[i] = S + L + s;
          } else {
            hit = true;
          }
        } else {
          mid = true;
          miss = true;
        }
      }
    }
    const uint64_t m = __ballot(miss);
    const uint64_t mm = __ballot(mid);
    const uint64_t mi_ = __ballot(inpl);
    const uint64_t mh = MULTI ? 0ull : __ballot(hit);
    uint32_t (*cnt)[4] = s_cnt[round & 1];
    if (lane == 0)
      *reinterpret_cast<u32x4*>(cnt[wave]) = (u32x4){(uint32_t)__popcll(m), (uint32_t)__popcll(mh),
                                                     (uint32_t)__popcll(mm), (uint32_t)__popcll(mi_)};
    __syncthreads();
    // every wave's counts: lane l < 16 reads wave l's, four wave scans give
    // this wave's offsets (the prefix before it) and the round's totals
    int off, hoff;
    {
      constexpr int NW = kResolveThreads / 64;   // the workgroup is always this size
      const u32x4 c = lane < NW ? *reinterpret_cast<const u32x4*>(cnt[lane]) : (u32x4){0u, 0u, 0u, 0u};
      const uint32_t ix = wave_incl_scan(c.x), iy = wave_incl_scan(c.y);
      const uint32_t iz = wave_incl_scan(c.z), iw = wave_incl_scan(c.w);
      const int wv = __builtin_amdgcn_readfirstlane(wave);
      off = nm_run + (wv > 0 ? __builtin_amdgcn_readlane((int)ix, wv - 1) : 0);
      hoff = nh_run + (wv > 0 ? __builtin_amdgcn_readlane((int)iy, wv - 1) : 0);
      nm_run += __builtin_amdgcn_readlane((int)ix, 63);
      nh_run += __builtin_amdgcn_readlane((int)iy, 63);
      nmid_run += __builtin_amdgcn_readlane((int)iz, 63);
      ninp_run += __builtin_amdgcn_readlane((int)iw, 63);
    }
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
    if constexpr (!MULTI) {
      if (hit) {
        const int at = hoff + (int)__popcll(mh & lt_mask);
        if (at < kMaxListMisses) {
          s_hit[at] = (uint16_t)i;
        } else {
          rb[i] = 0;      // more middle picks than a list holds: flagged
          s_bad = 1;
        }
      }
    }
  }
  if (threadIdx.x == 0) {
    s_nm = nm_run;
    s_nh = nh_run;
    s_nmid = nmid_run;
    s_ninp = ninp_run;
  }
  __syncthreads();
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
  if constexpr (!MULTI) {
    // one pick list: the misses' positions go to the fetch workgroups now, so
    // their host reads overlap the placement below
    for (int mi = threadIdx.x; mi < nm; mi += blockDim.x) put(miss_pos + (size_t)b * mstride + mi, s_mpos[mi]);
    if (threadIdx.x == 0) put(miss_n + b, nm);
    publish(sync + 4 * b + 0);
    // now the slot table, then the hits: each refreshes its slot and takes
    // its row (the slot lookups of up to four hits per thread in flight)
    for (int j = threadIdx.x; j < n_slots; j += blockDim.x) {
      s_pos[j] = sp[j];
      s_last[j] = sl[j];
      s_ref[j] = (uint8_t)sr[j];
    }
    __syncthreads();
    const int nh = min(s_nh, kMaxListMisses);
    for (int h0 = 0; h0 < nh; h0 += 4 * (int)blockDim.x) {
      int hi[4], hs[4];
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int h = h0 + u * (int)blockDim.x + (int)threadIdx.x;
        hi[u] = h < nh ? (int)s_hit[h] : -1;
      }
      int hp[4];
#pragma unroll
      for (int u = 0; u < 4; ++u) hp[u] = hi[u] >= 0 ? ib[hi[u]] : 0;
#pragma unroll
      for (int u = 0; u < 4; ++u) hs[u] = hi[u] >= 0 ? sop[hp[u]] : -1;
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        if (hi[u] < 0) continue;
        const int sl_ = hs[u];
        if (sl_ >= 0 && sl_ < n_slots) {
          s_ref[sl_] = 1;
          s_last[sl_] = step;
          rb[hi[u]] = S + L + sl_;
        } else {   // the bitmap and the slot map disagree: cannot happen; flagged
          rb[hi[u]] = 0;
          s_bad = 1;
        }
      }
    }
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
          if (old >= 0) {
            sop[old] = -1;
            atomicAnd(hb + (old >> 5), ~(1u << (old & 31)));
          }
          s_pos[j] = p;
          s_last[j] = step;
          sop[p] = j;
          atomicOr(hb + (p >> 5), 1u << (p & 31));
          rb[i] = S + L + j;
          s_miss[mi] = j;   // its slot, for the fetch
        }
      }
    }
    // fewer candidates than misses only if a step number was reused (its
    // slots then look used in this step): the rest are not placed, flagged
    const int placed = min(nm, (int)n_victims);
    for (int mi = placed + (int)threadIdx.x; mi < nm; mi += blockDim.x) rb[s_miss[mi]] = 0;
    __syncthreads();
    if (threadIdx.x == 0) {
      s_placed = placed;
      s_hand = h0;
      atomicAdd(&counters[0], (unsigned long long)(s_nmid + s_ninp));
      atomicAdd(&counters[1], (unsigned long long)(s_nmid - nm));
      atomicAdd(&counters[2], (unsigned long long)nm);
      atomicAdd(&counters[3], (unsigned long long)s_ninp);
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
    if (old >= 0) {
      sop[old] = -1;
      atomicAnd(hb + (old >> 5), ~(1u << (old & 31)));
    }
    s_pos[j] = p;
    s_ref[j] = 1;
    s_last[j] = step;
    sop[p] = j;
    atomicOr(hb + (p >> 5), 1u << (p & 31));
    rb[i] = S + L + j;
    s_miss[mi] = j;   // its slot, for the fetch
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
    s_placed = placed;
    atomicAdd(&counters[0], (unsigned long long)(s_nmid + s_ninp));
    atomicAdd(&counters[1], (unsigned long long)(s_nmid - nm));
    atomicAdd(&counters[2], (unsigned long long)nm);
    atomicAdd(&counters[3], (unsigned long long)s_ninp);
  }
  __syncthreads();
  }   // policy
  hand = s_hand;
  // the slots of this list's misses (-1: not placed, nothing written); with
  // several lists also their positions, after those of the earlier lists
  for (int mi = threadIdx.x; mi < nm; mi += blockDim.x) {
    if (MULTI) put(miss_pos + (size_t)b * mstride + moff + mi, s_mpos[mi]);
    put(miss_slot + (size_t)b * mstride + moff + mi, mi < s_placed ? s_miss[mi] : -1);
  }
  if (MULTI) moff += nm;
  __syncthreads();   // s_mpos / s_miss are reused by the next list
  if (qj + 1 < mq) n_next = n_sel[(size_t)b * mq + qj + 1];
  }   // pick lists
  if constexpr (MULTI) {
    if (threadIdx.x == 0) put(miss_n + b, moff);
    publish(sync + 4 * b + 0);
  }
  publish(sync + 4 * b + 1);
  if (threadIdx.x == 0) {
    hand_arr[b] = hand;
    if (s_bad) raise_flag(flags, SKV_FLAG_TIER_INPUT);
    arrive(sync + 4 * b, n_fetch);
  }
  for (int i = threadIdx.x; i < n_slots; i += blockDim.x) {
    sp[i] = s_pos[i];
    sl[i] = s_last[i];
    sr[i] = (int32_t)s_ref[i];
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
                 t->hand, t->slot_of_pos, t->hot_bits, t->ctx_dev, t->page_block, t->counters, t->flags,
                 t->miss_pos, t->miss_slot, t->miss_n, t->sync};
  for (void* p : dev)
    if (p) (void)hipFree(p);
  if (t->own_host && t->host) (void)hipHostFree(t->host);
  delete[] t->page_host;
  delete[] t->block_page;
  delete t;
}

extern "C" skv_status sparsekv_tier_create(const skv_tier_desc* d, skv_tier** out) {
  if (!d || !out) return set_error(SKV_ERR_INVALID, "tier_create: NULL argument");
  *out = nullptr;
  constexpr size_t kMinDesc = offsetof(skv_tier_desc, policy);
  constexpr size_t kPagedDesc = offsetof(skv_tier_desc, pool_pages) + sizeof(int32_t);
  if (d->struct_size < kMinDesc)
    return set_error(SKV_ERR_INVALID, "tier_create: struct_size %u < %zu", d->struct_size, kMinDesc);
  const int policy = d->struct_size >= offsetof(skv_tier_desc, policy) + sizeof(int32_t) ? d->policy
                                                                                         : SKV_TIER_CLOCK;
  const int P = d->struct_size >= kPagedDesc ? d->page_tokens : 0;
  const int pool_pages = d->struct_size >= kPagedDesc ? d->pool_pages : 0;
  if (P != 0 && (P < 16 || P > 4096 || (P & (P - 1))))
    return set_error(SKV_ERR_INVALID, "tier_create: page_tokens %d is not 0 or a power of two in [16, 4096]", P);
  if (pool_pages < 0 || (pool_pages > 0 && P == 0))
    return set_error(SKV_ERR_INVALID, "tier_create: pool_pages %d needs page_tokens", pool_pages);
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
  t->B = L.batch; t->T0 = d->ctx; t->cap_ctx = L.max_ctx; t->hot_words = (L.max_ctx + 31) / 32; t->S = L.n_sink; t->L = L.n_tail; t->k = L.topk;
  t->Hkv = L.n_kv_heads; t->D = L.head_dim; t->n_slots = d->n_slots; t->W = d->window;
  t->cap = skv::select_capacity(L);
  t->row_bytes = t->D / 2 + 2 * (t->D / 64);
  t->rec_bytes = 2 * t->row_bytes;
  t->P = P;
  t->page_shift = P ? __builtin_ctz((unsigned)P) : 0;
  t->pool_pages = pool_pages;
  t->n_pages = P ? (t->cap_ctx + P - 1) / P : 0;
  t->pool_row0 = (int64_t)t->S + t->L + t->n_slots;
  // about one workgroup per compute unit: F fetch workgroups per sequence
  t->n_fetch = std::max(1, std::min(63, 256 / t->B - 1));
  t->mstride = skv::kMaxQueries * skv::kMaxListMisses;
  t->res_rows = t->pool_row0 + (int64_t)pool_pages * P;
  if (t->res_rows > INT32_MAX) {
    tier_free(t);
    return set_error(SKV_ERR_INVALID, "tier_create: %lld resident rows per sequence exceed int32 row ids",
                     (long long)t->res_rows);
  }
  if (P) {
    t->page_host = new (std::nothrow) int32_t[(size_t)t->B * t->n_pages];
    t->block_page = new (std::nothrow) int32_t[(size_t)t->B * (pool_pages > 0 ? pool_pages : 1)];
    if (!t->page_host || !t->block_page) {
      tier_free(t);
      return set_error(SKV_ERR_OOM, "tier: host allocation failed");
    }
    std::fill(t->page_host, t->page_host + (size_t)t->B * t->n_pages, -1);
    std::fill(t->block_page, t->block_page + (size_t)t->B * (pool_pages > 0 ? pool_pages : 1), -1);
  }
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
            hipMalloc(&t->hot_bits, (size_t)t->B * t->hot_words * 4) == hipSuccess &&
            hipMalloc(&t->ctx_dev, (size_t)t->B * 4) == hipSuccess &&
            (!P || hipMalloc(&t->page_block, (size_t)t->B * t->n_pages * 4) == hipSuccess) &&
            hipMalloc(&t->counters, 4 * sizeof(unsigned long long)) == hipSuccess &&
            hipMalloc(&t->miss_pos, (size_t)t->B * t->mstride * 4) == hipSuccess &&
            hipMalloc(&t->miss_slot, (size_t)t->B * t->mstride * 4) == hipSuccess &&
            hipMalloc(&t->miss_n, (size_t)t->B * 4) == hipSuccess &&
            hipMalloc(&t->sync, (size_t)t->B * 16) == hipSuccess &&
            hipMalloc(&t->flags, 256) == hipSuccess;
  if (!ok) {
    (void)hipGetLastError();
    tier_free(t);
    return set_error(SKV_ERR_OOM, "tier: device allocation failed");
  }
  if (hipMemset(t->res_k, 0, rr * t->D) != hipSuccess || hipMemset(t->res_v, 0, rr * t->D) != hipSuccess ||
      hipMemset(t->res_ks, 0, rr * 2) != hipSuccess || hipMemset(t->res_vs, 0, rr * 2) != hipSuccess ||
      hipMemset(t->flags, 0, 256) != hipSuccess || hipMemset(t->sync, 0, (size_t)t->B * 16) != hipSuccess ||
      (P && hipMemset(t->page_block, 0xFF, (size_t)t->B * t->n_pages * 4) != hipSuccess)) {
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
                     t->slot_ref, t->hand, t->slot_of_pos, t->hot_bits, t->counters, t->B, t->n_slots,
                     t->cap_ctx, t->hot_words);
  if (hipGetLastError() != hipSuccess || hipDeviceSynchronize() != hipSuccess) {
    tier_free(t);
    return set_error(SKV_ERR_HIP, "tier: reset kernel failed");
  }
  *out = t;
  return SKV_OK;
}

extern "C" void* sparsekv_tier_host_records(skv_tier* t) { return t ? t->host : nullptr; }
extern "C" void* sparsekv_tier_host_ptr(skv_tier* t) { return t ? t->host : nullptr; }

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
  hipEvent_t ev0 = nullptr, ev1 = nullptr;
  const bool timed = skv::timer_next(skv::kTimerStream, &ev0, &ev1);   // diagnostic timer
#define SKV_RESOLVE_ARGS                                                                           \
  idx, n_sel, rows, t->slot_pos, t->slot_last, t->slot_ref, t->hand, t->slot_of_pos, t->hot_bits, \
      t->hot_words, t->counters,                                                                   \
      t->flags, t->ctx_dev, t->T0, t->cap_ctx, t->S, t->L, t->k, t->n_slots, t->W, t->cap, step,    \
      n_query, t->page_block, t->n_pages, t->page_shift, t->pool_row0, t->host_dev, t->res_k,       \
      t->res_v, t->res_ks, t->res_vs, t->res_rows, t->Hkv, t->miss_pos, t->miss_slot, t->miss_n, t->sync, \
      t->mstride, t->n_fetch
  const dim3 grid((unsigned)(t->B * (1 + t->n_fetch)));
#define SKV_RESOLVE(POL)                                                                           \
  do {                                                                                             \
    if (timed)                                                                                     \
      hipExtLaunchKernelGGL((skv::tier_resolve_kernel<POL, MUL>), grid, dim3(skv::kResolveThreads),         \
                            0, st, ev0, ev1, 0, SKV_RESOLVE_ARGS);                                 \
    else                                                                                           \
      hipLaunchKernelGGL((skv::tier_resolve_kernel<POL, MUL>), grid, dim3(skv::kResolveThreads), 0,         \
                         st, SKV_RESOLVE_ARGS);                                                    \
  } while (0)
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
#undef SKV_RESOLVE_ARGS
  if (hipGetLastError() != hipSuccess) return set_error(SKV_ERR_HIP, "tier_resolve: launch failed");
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
  unsigned long long c[4] = {0, 0, 0, 0};
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
  out->in_place = (int64_t)c[3];
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

extern "C" skv_status sparsekv_tier_map_page(skv_tier* t, int32_t seq, int32_t page, int32_t block,
                                             const int8_t* k, const int8_t* v, const uint16_t* ks,
                                             const uint16_t* vs, void* stream) {
  if (!t) return set_error(SKV_ERR_INVALID, "tier_map_page: NULL tier");
  if (!t->P || t->pool_pages < 1) return set_error(SKV_ERR_STATE, "tier_map_page: the tier has no page pool");
  if (seq < 0 || seq >= t->B || page < 0 || page >= t->n_pages || block < 0 || block >= t->pool_pages)
    return set_error(SKV_ERR_INVALID, "tier_map_page: seq %d / page %d / block %d out of range", seq, page, block);
  const size_t pi = (size_t)seq * t->n_pages + page, bi = (size_t)seq * t->pool_pages + block;
  if (t->page_host[pi] >= 0)
    return set_error(SKV_ERR_STATE, "tier_map_page: page %d of sequence %d is already mapped", page, seq);
  if (t->block_page[bi] >= 0)
    return set_error(SKV_ERR_STATE, "tier_map_page: block %d of sequence %d holds page %d", block, seq,
                     t->block_page[bi]);
  if ((k != nullptr) != (v != nullptr) || (k != nullptr) != (ks != nullptr) || (k != nullptr) != (vs != nullptr))
    return set_error(SKV_ERR_INVALID, "tier_map_page: give all of k, v, k_scale, v_scale or none");
  hipStream_t st = (hipStream_t)stream;
  if (k) {
    const size_t row0 = (size_t)seq * t->res_rows + (size_t)t->pool_row0 + (size_t)block * t->P;
    const size_t rows = (size_t)t->P * t->Hkv;   // (row, head) pairs of the page
    if (hipMemcpyAsync(t->res_k + row0 * t->Hkv * t->D, k, rows * t->D, hipMemcpyDeviceToDevice, st) != hipSuccess ||
        hipMemcpyAsync(t->res_v + row0 * t->Hkv * t->D, v, rows * t->D, hipMemcpyDeviceToDevice, st) != hipSuccess ||
        hipMemcpyAsync(t->res_ks + row0 * t->Hkv, ks, rows * 2, hipMemcpyDeviceToDevice, st) != hipSuccess ||
        hipMemcpyAsync(t->res_vs + row0 * t->Hkv, vs, rows * 2, hipMemcpyDeviceToDevice, st) != hipSuccess)
      return set_error(SKV_ERR_HIP, "tier_map_page: copy failed");
  }
  hipLaunchKernelGGL(skv::tier_set_page_kernel, dim3(1), dim3(1), 0, st, t->page_block, (int64_t)pi, block);
  if (hipGetLastError() != hipSuccess) return set_error(SKV_ERR_HIP, "tier_map_page: launch failed");
  t->page_host[pi] = block;
  t->block_page[bi] = page;
  return SKV_OK;
}

extern "C" skv_status sparsekv_tier_unmap_page(skv_tier* t, int32_t seq, int32_t page, void* stream) {
  if (!t) return set_error(SKV_ERR_INVALID, "tier_unmap_page: NULL tier");
  if (!t->P || t->pool_pages < 1) return set_error(SKV_ERR_STATE, "tier_unmap_page: the tier has no page pool");
  if (seq < 0 || seq >= t->B || page < 0 || page >= t->n_pages)
    return set_error(SKV_ERR_INVALID, "tier_unmap_page: seq %d / page %d out of range", seq, page);
  const size_t pi = (size_t)seq * t->n_pages + page;
  const int32_t block = t->page_host[pi];
  if (block < 0) return set_error(SKV_ERR_STATE, "tier_unmap_page: page %d of sequence %d is not mapped", page, seq);
  hipLaunchKernelGGL(skv::tier_set_page_kernel, dim3(1), dim3(1), 0, (hipStream_t)stream, t->page_block,
                     (int64_t)pi, -1);
  if (hipGetLastError() != hipSuccess) return set_error(SKV_ERR_HIP, "tier_unmap_page: launch failed");
  t->page_host[pi] = -1;
  t->block_page[(size_t)seq * t->pool_pages + block] = -1;
  return SKV_OK;
}

extern "C" skv_status sparsekv_tier_attend(skv_tier* t, const void* q, const int32_t* rows,
                                           const int32_t* n_sel, float sm_scale, float* out, void* ws,
                                           size_t ws_bytes, void* stream) {
  if (!t) return set_error(SKV_ERR_INVALID, "tier_attend: NULL tier");
  skv_kv_view v;
  v.k = t->res_k;
  v.v = t->res_v;
  v.k_scale = t->res_ks;
  v.v_scale = t->res_vs;
  v.rows = t->res_rows;
  return sparsekv_attend(&t->desc.layer, q, &v, rows, n_sel, sm_scale, out, ws, ws_bytes, stream);
}

extern "C" skv_status sparsekv_tier_reset(skv_tier* t, void* stream) {
  if (!t) return set_error(SKV_ERR_INVALID, "tier_reset: NULL argument");
  hipLaunchKernelGGL(skv::tier_reset_kernel, dim3(256), dim3(256), 0, (hipStream_t)stream,
                     t->slot_pos, t->slot_last, t->slot_ref, t->hand, t->slot_of_pos, t->hot_bits,
                     t->counters, t->B, t->n_slots, t->cap_ctx, t->hot_words);
  if (hipGetLastError() != hipSuccess) return set_error(SKV_ERR_HIP, "tier_reset: launch failed");
  t->steps = 0;
  return SKV_OK;
}

extern "C" void sparsekv_tier_destroy(skv_tier* t) {
  if (!t) return;
  (void)hipDeviceSynchronize();
  tier_free(t);
}
