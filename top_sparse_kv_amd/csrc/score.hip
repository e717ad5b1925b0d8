// Stage A2: exact ranking keys, and the streaming half of stage A3.
//
// Token mode -- page "8 agents x 250K context on two 3090s: sparse KV decode
// with a rank-64 key sketch and a host-RAM tier", section "The mechanism":
// each token carries an int4 sketch (H_kv*R codes) and one fp16 scale; the
// score is the integer dot product with the int8 query sketch.  The ranking
// key is that dot times the token's fp16 scale, computed exactly in fp64
// (at most 19 + 11 significant bits), so keys rank like q.k would.
//
// Block mode -- page "3.14M Context on 3x 3090: The Power of an Architecture
// That Puts KV Cache in Host RAM", sections "Why" and "What Needs to Stay in
// VRAM": every complete 4-token block has a 128-dim bf16 pooled key that is
// scored against the bf16 indexer query each step; the sum is accumulated in
// fp64, which is exact when the bf16 inputs lie in [2^-8, 2^8) or are 0.
//
// The index (130 B/token at H_kv*R = 256, or 256 B/block) is the only array
// read in full, so it is streamed once, with 16-byte loads spread over the
// lanes of a candidate so that every wavefront load covers 1 KB of
// consecutive memory; each wave keeps two batches of eight such loads in
// flight.  The kernels:
//   score_kernel<keys>     writes every key (sparsekv_score);
//   front_kernel           the 16-bit digits (key rounded to fp32, 1/128
//                          octave per bucket) of a sample of whole 16-candidate
//                          lines, written to the workspace (token mode: after
//                          quantizing the projected query sketch);
//   beta_kernel            one workgroup per sequence finds, from the sampled
//                          digits, the threshold digit beta (a 256-bin LDS
//                          histogram window slid down from the largest digit);
//   score_kernel<collect>  every wave keeps, per 256-token (128-block)
//                          segment, the candidates whose digit is >= beta, in
//                          position order (ballot + popcount), as (key,
//                          position) records; keys are never stored.
// No workgroup waits for another and no atomics are used.
#include "keys_common.h"

#include <hip/hip_ext.h>

namespace skv {
namespace {

constexpr int kThreads = 256;
constexpr int kUnroll = 8;

// The collect launches one workgroup per segment, one load batch per wave,
// where a segment is exactly four batches: the token sketch at 8 lanes per
// token (transposed collect) and the pooled key at 16 lanes per block.
template <class Src>
constexpr bool segment_per_workgroup() {
  constexpr int per_it = kUnroll * (64 / Src::LANES);
  return Src::HAS_AUX ? Src::LANES == 8 : per_it * (kThreads / 64) == kSegBlk;
}

// candidates whose key sparsekv_score writes (not restricted by the dense rule)
__device__ __forceinline__ void key_range(int mode, int T, int S, int L, int& lo, int& n) {
  if (mode == SKV_INDEX_SKETCH_INT4) {
    lo = S;
    n = T - L > S ? T - L - S : 0;
  } else {
    lo = 0;
    n = T / 4;
  }
}

template <class Src, bool COLLECT>
__global__ __launch_bounds__(kThreads) void score_kernel(
    const void* __restrict__ iq, const void* __restrict__ ik, const uint16_t* __restrict__ isc,
    const int32_t* __restrict__ ctx_len, double* __restrict__ keys,
    const TopkState* __restrict__ state, Cand* __restrict__ cand, uint32_t* __restrict__ segcnt,
    uint32_t* __restrict__ flags, int mode, int max_ctx, int S, int k, int L, int n_seg,
    int seg_items) {
  constexpr int N = Src::LANES, IPW = 64 / N, PER_IT = kUnroll * IPW;
  constexpr bool TRANS = COLLECT && Src::HAS_AUX && N == 8;   // see the transposed collect below
  constexpr bool SPLIT = COLLECT && !Src::HAS_AUX && segment_per_workgroup<Src>();   // pooled, one batch per wave
  const int b = blockIdx.y;
  const int T = clamp_ctx(ctx_len, b, max_ctx, blockIdx.x == 0 ? flags : nullptr);
  int lo, n;
  if (COLLECT) {
    const Range r = cand_range(mode, T, S, k, L);
    if (r.dense) return;
    lo = r.lo;
    n = r.n;
  } else {
    key_range(mode, T, S, L, lo, n);
  }
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  // transposed collect: one workgroup per segment, one batch per wave;
  // otherwise one segment per wave
  const int seg = TRANS || SPLIT ? blockIdx.x : blockIdx.x * (kThreads / 64) + wave;
  const int i0 = seg * seg_items;
  if (i0 >= n) return;   // workgroup-uniform (transposed) or wave-uniform (no barrier below)
  const int i1 = min(n, i0 + seg_items);
  const int first = TRANS || SPLIT ? i0 + PER_IT * wave : i0;
  const int sub = lane % N, tw = lane / N;
  Src src;
  src.init(reinterpret_cast<const uint8_t*>(iq) + (size_t)b * Src::QROW, ik, isc, b, max_ctx, sub);
  u32x4 w[kUnroll];
  uint32_t ax[kUnroll];
  // loads issued unconditionally (past the end they re-read the last
  // candidate; those results are dropped), so a batch is in flight together
  auto load_batch = [&](int base, u32x4* wv, uint32_t* av) {
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      const int i = min(base + u * IPW + tw, i1 - 1);
      wv[u] = src.load(lo + i);
      if constexpr (!TRANS) av[u] = src.load_aux(lo + i);
    }
  };
  load_batch(first, w, ax);
  const uint32_t beta = COLLECT ? state[b].beta : 0u;   // read while the first loads fly
  double* kout = keys + (size_t)b * (mode == SKV_INDEX_SKETCH_INT4 ? max_ctx : max_ctx / 4) + lo;
  u32x4* cseg = reinterpret_cast<u32x4*>(cand + ((size_t)b * n_seg + seg) * seg_items);
  const uint64_t lt = lanemask_lt();
  uint32_t cnt = 0;
  if constexpr (TRANS) {
    // Transposed collect: the 8 partial dots of a lane (one per load) are
    // reduced over the 8 lanes of its group by a butterfly (mirror / quad
    // swaps), which leaves lane (tw, sub) with the whole dot of load sub, i.e.
    // candidate o = 8*sub + tw of the wave's batch.  Digit, selection and
    // ballot then run once, and the ballot is transposed (8x8 bits) into
    // candidate order for the ranks.  Each lane reads the scale of its own
    // candidate.  The four waves of the workgroup cover the segment's four
    // batches; their counts are exchanged in LDS so that the records land in
    // position order.  Short per-wave work (8 KB) lets the dispatcher keep
    // the HBM queues full to the end of the stream.
    static_assert(PER_IT * (kThreads / 64) == kSegTok, "one batch per wave");
    __shared__ uint32_t s_cnt[kThreads / 64];
    const int o = 8 * sub + tw;
    const uint32_t sc = src.load_aux(lo + min(first + o, i1 - 1));
    const uint32_t b2 = (sub >> 2) & 1, b1 = (sub >> 1) & 1, b0 = sub & 1;
    const uint64_t below = (1ull << o) - 1ull;
    int p[kUnroll];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) p[u] = src.partial(w[u]);
#pragma unroll
    for (int j = 0; j < 4; ++j) {   // partner 7 - sub: opposite bit 2
      const int keep = b2 ? p[j + 4] : p[j], send = b2 ? p[j] : p[j + 4];
      p[j] = keep + (int)dpp_u32<0x141>((uint32_t)send);
    }
#pragma unroll
    for (int j = 0; j < 2; ++j) {   // partner sub ^ 2
      const int keep = b1 ? p[j + 2] : p[j], send = b1 ? p[j] : p[j + 2];
      p[j] = keep + (int)dpp_u32<0x4E>((uint32_t)send);
    }
    {                               // partner sub ^ 1
      const int keep = b0 ? p[1] : p[0], send = b0 ? p[0] : p[1];
      p[0] = keep + (int)dpp_u32<0xB1>((uint32_t)send);
    }
    const int dt = p[0] >> 4;
    const int i = first + o;
    const uint32_t dig = src.digit_of(dt, sc);
    const bool sel = i < i1 && dig >= beta;
    uint64_t x = __ballot(sel);   // bit 8*tw + sub
    uint64_t t = (x ^ (x >> 7)) & 0x00AA00AA00AA00AAull;
    x = x ^ t ^ (t << 7);
    t = (x ^ (x >> 14)) & 0x0000CCCC0000CCCCull;
    x = x ^ t ^ (t << 14);
    t = (x ^ (x >> 28)) & 0x00000000F0F0F0F0ull;
    x = x ^ t ^ (t << 28);          // bit o = 8*sub + tw
    if (lane == 0) s_cnt[wave] = (uint32_t)__popcll(x);
    __syncthreads();
    uint32_t off = 0, tot = 0;
#pragma unroll
    for (int v = 0; v < kThreads / 64; ++v) {
      const uint32_t c = s_cnt[v];
      off += v < wave ? c : 0u;
      tot += c;
    }
    if (sel) {
      const uint64_t ok = ordered_u64(src.key_of(dt, sc));
      cseg[off + (uint32_t)__popcll(x & below)] =
          (u32x4){(uint32_t)ok, (uint32_t)(ok >> 32), (uint32_t)(lo + i), dig};
    }
    if (threadIdx.x == 0) segcnt[(size_t)b * n_seg + seg] = tot;
    return;
  }
  if constexpr (SPLIT) {
    // Pooled keys, one workgroup per 128-block segment: wave w scores the
    // segment's batch w (32 blocks); the four counts go through LDS so that
    // the records stay in position order.  Short per-wave work keeps more
    // loads in flight when the batch holds few sequences.
    __shared__ uint32_t s_cnt2[kThreads / 64];
    uint64_t mu[kUnroll], oku[kUnroll];
    uint32_t digu[kUnroll], tot_w = 0;
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      const int i = first + u * IPW + tw;
      const double key = src.key(w[u], ax[u]);
      digu[u] = key_digit16(key);
      oku[u] = ordered_u64(key);
      mu[u] = __ballot(sub == 0 && i < i1 && digu[u] >= beta);
      tot_w += (uint32_t)__popcll(mu[u]);
    }
    if (lane == 0) s_cnt2[wave] = tot_w;
    __syncthreads();
    uint32_t run = 0, tot = 0;
#pragma unroll
    for (int v = 0; v < kThreads / 64; ++v) {
      const uint32_t c = s_cnt2[v];
      run += v < wave ? c : 0u;
      tot += c;
    }
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      if ((mu[u] >> lane) & 1ull)
        cseg[run + (uint32_t)__popcll(mu[u] & lt)] =
            (u32x4){(uint32_t)oku[u], (uint32_t)(oku[u] >> 32), (uint32_t)(lo + first + u * IPW + tw), digu[u]};
      run += (uint32_t)__popcll(mu[u]);
    }
    if (threadIdx.x == 0) segcnt[(size_t)b * n_seg + seg] = tot;
    return;
  }
  for (int base = i0; base < i1; base += PER_IT) {
    u32x4 wn[kUnroll];
    uint32_t an[kUnroll];
    if (base + PER_IT < i1) load_batch(base + PER_IT, wn, an);   // next batch in flight
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      const int i = base + u * IPW + tw;
      if constexpr (!COLLECT) {
        const double key = src.key(w[u], ax[u]);
        if (sub == 0 && i < i1) kout[i] = key;
      } else if constexpr (Src::HAS_AUX) {
        // token sketch: the digit from the fp32 product; the exact fp64 key
        // only for the kept candidates
        const int dt = src.dot(w[u]);
        const uint32_t dig = src.digit_of(dt, ax[u]);
        const bool sel = sub == 0 && i < i1 && dig >= beta;
        const uint64_t m = __ballot(sel);
        if (sel) {
          const uint64_t ok = ordered_u64(src.key_of(dt, ax[u]));
          const uint32_t rank = cnt + (uint32_t)__popcll(m & lt);
          cseg[rank] = (u32x4){(uint32_t)ok, (uint32_t)(ok >> 32), (uint32_t)(lo + i), dig};
        }
        cnt += (uint32_t)__popcll(m);
      } else {
        const double key = src.key(w[u], ax[u]);
        const uint32_t dig = key_digit16(key);
        const bool sel = sub == 0 && i < i1 && dig >= beta;
        const uint64_t m = __ballot(sel);
        if (sel) {
          const uint64_t ok = ordered_u64(key);
          const uint32_t rank = cnt + (uint32_t)__popcll(m & lt);
          cseg[rank] = (u32x4){(uint32_t)ok, (uint32_t)(ok >> 32), (uint32_t)(lo + i), dig};
        }
        cnt += (uint32_t)__popcll(m);
      }
    }
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      w[u] = wn[u];
      ax[u] = an[u];
    }
  }
  if (COLLECT && lane == 0) segcnt[(size_t)b * n_seg + seg] = cnt;
}

// Front of the fused step: the sample of the threshold estimate.  Workgroup w
// of sequence b reads sample lines [w*LPG, (w+1)*LPG) (line j = candidates
// [16*s*j, 16*s*j + 16)), issuing those loads first.  Token mode with
// FROM_PROJ: the fp32 query sketch in the workspace is quantized here (one
// int8 scale per sequence) and workgroup 0 writes it out.  Then the 16-bit
// digits of its sampled keys, written in line order (empty sample slots as
// digit 0); the threshold kernel takes the need-th largest digit of the
// sequence's sample.
template <class Src, bool FROM_PROJ>
__global__ __launch_bounds__(kFrontThreads) void front_kernel(
    const void* __restrict__ iq, const float* __restrict__ sproj, int8_t* __restrict__ qs_out,
    float* __restrict__ qscale_out, const void* __restrict__ ik, const uint16_t* __restrict__ isc,
    const int32_t* __restrict__ ctx_len, uint16_t* __restrict__ sdig, int sdig_stride, int mode,
    int max_ctx, int S, int k, int L) {
  constexpr int N = Src::LANES, IPW = 64 / N, FU = kFrontUnroll, PER_IT = FU * IPW;
  constexpr int LPW = PER_IT / kLineKeys;                   // sample lines per wave
  constexpr int NWV = kFrontThreads / 64;
  constexpr int LPG = LPW * NWV;                            // sample lines per workgroup
  constexpr int MW = LPG * kLineKeys;                       // sample slots per workgroup
  constexpr int NQ = 32 * N;                                // int8 query sketch values (token mode)
  static_assert(LPG == front_lines(N), "front geometry");
  // token mode (the only FROM_PROJ caller) has N <= 16: NQ <= 512 = 2 * kFrontThreads
  __shared__ int8_t q8[512];
  __shared__ uint32_t s_red[32];
  const int b = blockIdx.y, w = blockIdx.x;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const Range r = cand_range(mode, ctx_of(ctx_len, b, max_ctx), S, k, L);
  const int s = r.dense ? 1 : sample_stride(r.n, k);
  const int nsl = r.dense ? 0 : sample_lines(r.n, k);
  const int nwg = front_wgs(nsl, N);
  if (w >= nwg && !(FROM_PROJ && w == 0)) return;   // workgroup-uniform
  const int sub = lane % N, tw = lane / N;
  Src src;
  src.init_data(ik, isc, b, max_ctx, sub);
  // the sample loads go out first (clamped: past the sample they re-read a
  // valid candidate, dropped below)
  const int j0 = (w * NWV + wave) * LPW;
  u32x4 wv[FU];
  uint32_t ax[FU];
  bool ok[FU];
#pragma unroll
  for (int u = 0; u < FU; ++u) {
    const int o = u * IPW + tw;
    const int j = j0 + o / kLineKeys;
    const int i = j * s * kLineKeys + o % kLineKeys;
    ok[u] = j < nsl && i < r.n;
    const int ic = ok[u] ? i : (r.n > 0 ? r.n - 1 : 0);
    wv[u] = src.load(r.lo + ic);
    ax[u] = src.load_aux(r.lo + ic);
  }
  const void* qrow;
  if constexpr (FROM_PROJ) {
    const float scale = quantize_sketch(sproj + (size_t)b * NQ, NQ, q8, s_red);
    if (w == 0) {
      for (int i = threadIdx.x; i < NQ; i += kFrontThreads) qs_out[(size_t)b * NQ + i] = q8[i];
      if (threadIdx.x == 0) qscale_out[b] = scale;
    }
    if (w >= nwg) return;   // workgroup-uniform: dense sequence, sketch written
    qrow = q8;
  } else {
    qrow = reinterpret_cast<const uint8_t*>(iq) + (size_t)b * Src::QROW;
  }
  src.init_query(qrow, sub);
  uint16_t* dg = sdig + (size_t)b * sdig_stride + (size_t)w * MW;   // this workgroup's lines
#pragma unroll
  for (int u = 0; u < FU; ++u) {
    uint32_t dig;
    if constexpr (Src::HAS_AUX) dig = src.digit_of(src.dot(wv[u]), ax[u]);
    else dig = key_digit16(src.key(wv[u], ax[u]));
    if (sub == 0) dg[wave * PER_IT + u * IPW + tw] = ok[u] ? (uint16_t)dig : (uint16_t)0u;
  }
}

// Threshold digit of each (virtual) sequence from its sampled digits.  With
// mq query tokens per sequence the sample is laid out for the last query's
// (largest) candidate range, shared by the sequence's queries.
__global__ __launch_bounds__(1024) void beta_kernel(const uint16_t* __restrict__ sdig, int n_samp,
                                                     const int32_t* __restrict__ ctx_len,
                                                     TopkState* __restrict__ state, int mode,
                                                     int max_ctx, int S, int k, int L, int mq) {
  __shared__ uint32_t red[256 + 32];
  const int b = blockIdx.x;
  if (cand_range(mode, ctx_of_query(ctx_len, b, mq, max_ctx), S, k, L).dense) return;
  const Range r = cand_range(mode, ctx_of(ctx_len, b / mq, max_ctx), S, k, L);
  const uint32_t beta = wg_beta(sdig + (size_t)b * n_samp * kLineKeys,
                                sample_lines(r.n, k) * kLineKeys, sample_need(r.n, k), red);
  if (threadIdx.x == 0) state[b].beta = beta;
}

template <class Src>
hipError_t launch_token_or_block(const skv_layer_desc& d, const int32_t* ctx_len, const void* iq,
                                 const void* q, const float* basis, int8_t* qs_out,
                                 float* qscale_out, const void* ik, const uint16_t* isc, double* keys,
                                 void* ws, const WsLayout* Lw, uint32_t* flags, bool collect,
                                 hipStream_t st) {
  const int mode = d.index_mode;
  const int S = mode == SKV_INDEX_SKETCH_INT4 ? d.n_sink : 0;
  const int L = mode == SKV_INDEX_SKETCH_INT4 ? d.n_tail : 0;
  const int seg_items = mode == SKV_INDEX_SKETCH_INT4 ? kSegTok : kSegBlk;
  const int n_seg = (max_candidates(d) + seg_items - 1) / seg_items;
  constexpr int kWaves = kThreads / 64;   // one segment per wave
  dim3 grid((n_seg + kWaves - 1) / kWaves > 0 ? (n_seg + kWaves - 1) / kWaves : 1, d.batch);
  if (!collect) {
    hipLaunchKernelGGL((score_kernel<Src, false>), grid, dim3(kThreads), 0, st, iq, ik, isc,
                       ctx_len, keys, nullptr, nullptr, nullptr, flags, mode, d.max_ctx, S, d.topk,
                       L, n_seg, seg_items);
    return hipGetLastError();
  }
  // the front kernel: grid wide enough for the largest sample of a sequence
  const dim3 fgrid(front_wgs(Lw->n_samp, Src::LANES), d.batch);
  uint16_t* sdig = ws_ptr<uint16_t>(ws, Lw->sdig);
  const int sdig_stride = Lw->sdig_stride;
  TopkState* state = ws_ptr<TopkState>(ws, Lw->state);
  if (qs_out)
    hipLaunchKernelGGL((front_kernel<Src, true>), fgrid, dim3(kFrontThreads), 0, st, nullptr,
                       ws_ptr<const float>(ws, Lw->sproj), qs_out, qscale_out, ik, isc, ctx_len, sdig,
                       sdig_stride, mode, d.max_ctx, S, d.topk, L);
  else
    hipLaunchKernelGGL((front_kernel<Src, false>), fgrid, dim3(kFrontThreads), 0, st, iq, nullptr,
                       nullptr, nullptr, ik, isc, ctx_len, sdig, sdig_stride, mode, d.max_ctx, S,
                       d.topk, L);
  // the threshold: one 1024-thread workgroup per sequence over its sample
  hipLaunchKernelGGL(beta_kernel, dim3(d.batch), dim3(1024), 0, st, (const uint16_t*)sdig,
                     sdig_stride / kLineKeys, ctx_len, state, mode, d.max_ctx, S, d.topk, L, 1);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const void* iq_score = qs_out ? (const void*)qs_out : iq;
  // the transposed token collect and the 16-lane pooled collect run one
  // workgroup per segment
  if (segment_per_workgroup<Src>()) grid.x = Lw->n_seg;
  hipEvent_t ev0 = nullptr, ev1 = nullptr;
  if (timer_next(kTimerStream, &ev0, &ev1))
    hipExtLaunchKernelGGL((score_kernel<Src, true>), grid, dim3(kThreads), 0, st, ev0, ev1, 0,
                          iq_score, ik, isc, ctx_len, (double*)nullptr, (const TopkState*)state,
                          ws_ptr<Cand>(ws, Lw->cand), ws_ptr<uint32_t>(ws, Lw->segcnt), flags, mode,
                          d.max_ctx, S, d.topk, L, Lw->n_seg, Lw->seg_items);
  else
    hipLaunchKernelGGL((score_kernel<Src, true>), grid, dim3(kThreads), 0, st, iq_score, ik, isc,
                       ctx_len, nullptr, state, ws_ptr<Cand>(ws, Lw->cand),
                       ws_ptr<uint32_t>(ws, Lw->segcnt), flags, mode, d.max_ctx, S, d.topk, L,
                       Lw->n_seg, Lw->seg_items);
  return hipGetLastError();
}

hipError_t launch_any(const skv_layer_desc& d, const int32_t* ctx_len, const void* iq, const void* q,
                      const float* basis, int8_t* qs_out, float* qscale_out, const void* ik,
                      const uint16_t* isc, double* keys, void* ws, const WsLayout* Lw, uint32_t* flags,
                      bool collect, hipStream_t st) {
#define SKV_GO(SRC) return launch_token_or_block<SRC>(d, ctx_len, iq, q, basis, qs_out, qscale_out, ik, isc, keys, ws, Lw, flags, collect, st)
  if (d.index_mode == SKV_INDEX_SKETCH_INT4) {
    switch (d.n_kv_heads * d.rank / 2) {   // sketch bytes per token = 16 * lanes
      case 32: SKV_GO(SketchSrc<2>);
      case 64: SKV_GO(SketchSrc<4>);
      case 128: SKV_GO(SketchSrc<8>);
      case 256: SKV_GO(SketchSrc<16>);
      default: return hipErrorInvalidValue;
    }
  }
  switch (d.index_dim) {   // pooled key bytes = 16 * lanes
    case 64: SKV_GO(PooledSrc<8>);
    case 128: SKV_GO(PooledSrc<16>);
    case 256: SKV_GO(PooledSrc<32>);
    default: return hipErrorInvalidValue;
  }
#undef SKV_GO
}

}  // namespace

hipError_t launch_score(const skv_layer_desc& d, const int32_t* ctx_len, const void* iq,
                        const void* ik, const uint16_t* isc, double* keys, uint32_t* flags,
                        hipStream_t st) {
  return launch_any(d, ctx_len, iq, nullptr, nullptr, nullptr, nullptr, ik, isc, keys, nullptr, nullptr,
                    flags, false, st);
}

hipError_t launch_sample_collect(const skv_layer_desc& d, const int32_t* ctx_len, const void* iq,
                                 const void* q, const float* basis, int8_t* qs_out, float* qscale_out,
                                 const void* ik, const uint16_t* isc, void* ws, const WsLayout& L,
                                 hipStream_t st) {
  return launch_any(d, ctx_len, iq, q, basis, qs_out, qscale_out, ik, isc, nullptr, ws, &L,
                    ws_ptr<uint32_t>(ws, L.flags), true, st);
}

hipError_t launch_beta(const skv_layer_desc& dv, int mq, const int32_t* ctx_len, void* ws,
                       const WsLayout& L, hipStream_t st) {
  const int mode = dv.index_mode;
  const int S = mode == SKV_INDEX_SKETCH_INT4 ? dv.n_sink : 0;
  const int Lt = mode == SKV_INDEX_SKETCH_INT4 ? dv.n_tail : 0;
  hipLaunchKernelGGL(beta_kernel, dim3(dv.batch), dim3(1024), 0, st, ws_ptr<const uint16_t>(ws, L.sdig),
                     L.n_samp, ctx_len, ws_ptr<TopkState>(ws, L.state), mode, dv.max_ctx, S, dv.topk,
                     Lt, mq);
  return hipGetLastError();
}

}  // namespace skv
