// Stages A1-A3 for a step that carries several query tokens per sequence.
//
// Page "8 agents x 250K context on two 3090s: sparse KV decode with a rank-64
// key sketch and a host-RAM tier", section "What shipped": the model decodes
// with MTP-7 speculation, so one step verifies the drafted tokens together
// with the current one; page "vLLM's Hybrid HiSparse Triples Concurrent
// Requests on Million-Token Contexts", section "Where the tradeoffs bite":
// every verification token has its own pick.  Query j of M (the cache's last
// M positions) sees the causal context T - M + 1 + j and is scored, ranked
// and attended exactly as a single decode query at that length.
//
// All queries of a sequence read the same sketch, so it is streamed once: for
// every token the codes meet up to 16 int8 query sketches, a dense int8
// contraction [tokens x H_kv*R] x [H_kv*R x queries] that runs on the matrix
// cores (v_mfma_i32_16x16x64_i8: 16 tokens x 16 queries x 64 dims).  The
// int4 codes of a lane's 16 bytes become two int8 operands holding 16x the
// codes (high nibbles masked in place, low nibbles shifted up), so the
// accumulator is 16x the exact integer dot.
//
// Operand layout (checked on the GPU against a host product): lane l supplies
// row l%16 of A and column l%16 of B over the same 16 k values, chosen by
// l/16, and receives C[4*(l/16) + i][l%16] in element i.  A row is a token:
// lane l reads bytes [16g + 64m, +16) of token l%16's code row (g = l/16,
// m < TB/64), i.e. dims [32g + 128m, +32); its B operands hold query l%16's
// codes of the same dims, the even dims against the low nibbles and the odd
// dims against the high ones.  The lane then owns tokens 4g..4g+3 of the
// tile for query l%16.
//
// Kernels (the threshold kernel is the single-query one, per query):
//   sample_multi_kernel   quantizes the M query sketches and writes the
//                         digits of a sample of 16-token lines per query
//                         (the lines of the last query's candidate range);
//   score_multi_kernel    one workgroup per 256-token segment, one 64-token
//                         batch (four 16-token tiles) per wave; per query,
//                         the candidates at or above its threshold are kept
//                         in position order as (key, position, digit)
//                         records, the per-wave counts exchanged in LDS.
#include "keys_common.h"

#include <hip/hip_ext.h>

namespace skv {
namespace {

typedef int v4i __attribute__((ext_vector_type(4)));
constexpr int kThreads = 256;
constexpr int kTiles = 4;                 // 16-token tiles per wave
static_assert(kTiles * 16 * (kThreads / 64) == kSegTok, "one 64-token batch per wave");

template <int TB>   // sketch bytes per token: 64, 128 or 256
struct MqTile {
  static constexpr int NL = TB / 64;      // 16-byte loads per lane per tile
  v4i bq[NL][2];                          // query operands: even dims, odd dims

  // q8: LDS rows of 2*TB int8 query codes, one per query (zero rows for the
  // unused queries of the 16)
  __device__ __forceinline__ void init(const int8_t* q8, int lane) {
    const int j = lane & 15, g = lane >> 4;
#pragma unroll
    for (int m = 0; m < NL; ++m) {
      const uint32_t* p = reinterpret_cast<const uint32_t*>(q8 + j * 2 * TB + 32 * g + 128 * m);
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        const uint32_t x0 = p[2 * t], x1 = p[2 * t + 1];   // query dims 8t .. 8t+7
        bq[m][0][t] = (int)((x0 & 0xFFu) | ((x0 >> 8) & 0xFF00u) | ((x1 & 0xFFu) << 16) |
                            ((x1 << 8) & 0xFF000000u));
        bq[m][1][t] = (int)(((x0 >> 8) & 0xFFu) | ((x0 >> 16) & 0xFF00u) | ((x1 << 8) & 0xFF0000u) |
                            (x1 & 0xFF000000u));
      }
    }
  }
  // 16x the integer dots of the tile's 16 tokens (rows) with the 16 queries
  __device__ __forceinline__ v4i mma(const u32x4* w) const {
    v4i c = {0, 0, 0, 0};
#pragma unroll
    for (int m = 0; m < NL; ++m) {
      v4i lo, hi;
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        lo[t] = (int)((w[m][t] << 4) & 0xF0F0F0F0u);
        hi[t] = (int)(w[m][t] & 0xF0F0F0F0u);
      }
      c = __builtin_amdgcn_mfma_i32_16x16x64_i8(lo, bq[m][0], c, 0, 0, 0);
      c = __builtin_amdgcn_mfma_i32_16x16x64_i8(hi, bq[m][1], c, 0, 0, 0);
    }
    return c;
  }
};

// The same 16x dots on the vector ALUs (a measurement aid): lane (query j =
// l%16, group g = l/16) computes tokens 4g..4g+3 of a tile against query j
// itself, reading the tile's code rows from LDS (staged there by the wave) and
// holding query j's codes as even-dim and odd-dim dwords, with 4-way int8 dot
// instructions against the nibbles masked (odd dims) or shifted (even dims)
// into the high half of each byte, as in the matrix-core operands.
template <int TB>
struct MqTileValu {
  static constexpr int NU = TB / 4;       // code dwords per token
  static constexpr int RS = TB + 16;      // LDS row stride (bytes): 4 rows, 4 bank groups
  int qe[NU], qo[NU];

  __device__ __forceinline__ void init(const int8_t* q8, int lane) {
    const uint32_t* p = reinterpret_cast<const uint32_t*>(q8 + (lane & 15) * 2 * TB);
#pragma unroll
    for (int u = 0; u < NU; ++u) {
      const uint32_t x0 = p[2 * u], x1 = p[2 * u + 1];   // query dims 8u .. 8u+7
      qe[u] = (int)((x0 & 0xFFu) | ((x0 >> 8) & 0xFF00u) | ((x1 & 0xFFu) << 16) | ((x1 << 8) & 0xFF000000u));
      qo[u] = (int)(((x0 >> 8) & 0xFFu) | ((x0 >> 16) & 0xFF00u) | ((x1 << 8) & 0xFF0000u) | (x1 & 0xFF000000u));
    }
  }
  // rows: the tile's 16 code rows in LDS; element e = token 4g + e
  __device__ __forceinline__ v4i dots(const uint8_t* rows, int lane) const {
    const int g = lane >> 4;
    v4i c;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const u32x4* rp = reinterpret_cast<const u32x4*>(rows + (4 * g + e) * RS);
      int acc = 0;
#pragma unroll
      for (int x = 0; x < NU / 4; ++x) {
        const u32x4 w = rp[x];
#pragma unroll
        for (int t = 0; t < 4; ++t) {
          acc = __builtin_amdgcn_sdot4((int)((w[t] << 4) & 0xF0F0F0F0u), qe[4 * x + t], acc, false);
          acc = __builtin_amdgcn_sdot4((int)(w[t] & 0xF0F0F0F0u), qo[4 * x + t], acc, false);
        }
      }
      c[e] = acc;
    }
    return c;
  }
};

// the digit and the exact key of a token from its dot and fp16 scale (the same
// formulas as the single-query stream)
__device__ __forceinline__ uint32_t mq_digit(int d, uint32_t sc) {
  return ordered_u32((float)d * half_bits_to_float((uint16_t)sc) + 0.0f) >> 16;
}
__device__ __forceinline__ double mq_key(int d, uint32_t sc) {
  return (double)d * (double)half_bits_to_float((uint16_t)sc) + 0.0;
}

// candidates of query j: its middle range and whether it is ranked at all
struct QueryRange {
  int n;          // candidates [S, S + n)
  bool active;    // a query token of this step whose sequence is not dense
};
__device__ __forceinline__ QueryRange query_range(int T, int mq, int j, int S, int k, int L) {
  QueryRange q{0, false};
  if (j < mq) {
    const int Tj = T - (mq - 1 - j);
    const Range r = cand_range(SKV_INDEX_SKETCH_INT4, Tj < 0 ? 0 : Tj, S, k, L);
    q.active = !r.dense;
    q.n = r.n;
  }
  return q;
}

template <int TB>
__global__ __launch_bounds__(kThreads) void sample_multi_kernel(
    const float* __restrict__ sproj, int8_t* __restrict__ qs_out, float* __restrict__ qscale_out,
    int mq, const uint8_t* __restrict__ ik, const uint16_t* __restrict__ isc,
    const int32_t* __restrict__ ctx_len, uint16_t* __restrict__ sdig, int n_samp, int max_ctx,
    int S, int k, int L) {
  constexpr int NQ = 2 * TB, NL = TB / 64;
  __shared__ __align__(16) int8_t s_q[kMaxQueries * NQ];
  const int b = blockIdx.y;
  // the M query sketches of the sequence, one int8 scale each (the rule of
  // quantize_sketch: scale = amax / 127 rounded once, codes rint(v / scale)
  // clamped to +-127): wave w quantizes queries w, w + 4, ..., all of their
  // values loaded first, the maximum taken over the wave
  {
    constexpr int VPL = NQ / 64, RPW = kMaxQueries / (kThreads / 64);
    const int ln = threadIdx.x & 63, wv = threadIdx.x >> 6;
    float v[RPW][VPL];
#pragma unroll
    for (int u = 0; u < RPW; ++u) {
      const int j = min(wv + u * (kThreads / 64), mq - 1);   // unconditional
#pragma unroll
      for (int e = 0; e < VPL; ++e) v[u][e] = sproj[((size_t)b * mq + j) * NQ + ln + 64 * e];
    }
#pragma unroll
    for (int u = 0; u < RPW; ++u) {
      const int j = wv + u * (kThreads / 64);
      if (j >= mq) break;   // wave-uniform
      uint32_t am = 0;
#pragma unroll
      for (int e = 0; e < VPL; ++e) am = max(am, __float_as_uint(fabsf(v[u][e])));
      const float amax = __uint_as_float(wave_max(am));
      const float scale = amax == 0.0f ? 0.0f : (float)((double)amax / 127.0);
#pragma unroll
      for (int e = 0; e < VPL; ++e) {
        int8_t c = 0;
        if (amax != 0.0f) {
          float rr = rintf((float)((double)v[u][e] / (double)scale));
          c = (int8_t)(int)fminf(fmaxf(rr, -127.0f), 127.0f);
        }
        s_q[j * NQ + ln + 64 * e] = c;
        if (blockIdx.x == 0) qs_out[((size_t)b * mq + j) * NQ + ln + 64 * e] = c;
      }
      if (blockIdx.x == 0 && ln == 0) qscale_out[(size_t)b * mq + j] = scale;
    }
  }
  for (int i = threadIdx.x; i < (kMaxQueries - mq) * NQ; i += kThreads) s_q[mq * NQ + i] = 0;
  __syncthreads();
  const int T = ctx_of(ctx_len, b, max_ctx);
  const Range r = cand_range(SKV_INDEX_SKETCH_INT4, T, S, k, L);   // the last query's range
  if (r.dense) return;
  const int s = sample_stride(r.n, k);
  const int nsl = sample_lines(r.n, k);
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int l0 = (blockIdx.x * (kThreads / 64) + wave) * kTiles;   // first sample line of the wave
  if (l0 >= nsl) return;   // wave-uniform; no barrier below
  const int j = lane & 15, g = lane >> 4;
  const uint8_t* cb = ik + (size_t)b * max_ctx * TB + 16 * g;
  const uint16_t* sb = isc + (size_t)b * max_ctx + r.lo;
  u32x4 w[kTiles][NL];
#pragma unroll
  for (int t = 0; t < kTiles; ++t) {
    const int i = min(16 * s * (l0 + t) + j, r.n - 1);   // past the end: re-read, dropped below
#pragma unroll
    for (int m = 0; m < NL; ++m)
      w[t][m] = __builtin_nontemporal_load(
          reinterpret_cast<const u32x4*>(cb + (size_t)(r.lo + i) * TB + 64 * m));
  }
  // lane l fetches the scale of token l%16 of line l0 + l/16
  const uint32_t sc_l = sb[min(16 * s * (l0 + g) + j, r.n - 1)];
  MqTile<TB> tile;
  tile.init(s_q, lane);
  const QueryRange qr = query_range(T, mq, j, S, k, L);
  uint16_t* dg = sdig + ((size_t)b * mq + j) * n_samp * kLineKeys;
#pragma unroll
  for (int t = 0; t < kTiles; ++t) {
    const v4i c = tile.mma(w[t]);
    uint32_t d4[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const uint32_t sc = __shfl(sc_l, 16 * t + 4 * g + e);
      const int i = 16 * s * (l0 + t) + 4 * g + e;
      d4[e] = i < qr.n ? mq_digit(c[e] >> 4, sc) : 0u;   // 0: empty sample slot
    }
    if (qr.active && l0 + t < nsl)
      *reinterpret_cast<uint2*>(dg + (size_t)(l0 + t) * kLineKeys + 4 * g) =
          make_uint2(d4[0] | (d4[1] << 16), d4[2] | (d4[3] << 16));
  }
}

// VALU: the dots on the vector ALUs (MqTileValu), else on the matrix cores
template <int TB, bool VALU>
__global__ __launch_bounds__(kThreads) void score_multi_kernel(
    const int8_t* __restrict__ qs, const uint8_t* __restrict__ ik, const uint16_t* __restrict__ isc,
    const int32_t* __restrict__ ctx_len, const TopkState* __restrict__ state,
    Cand* __restrict__ cand, uint32_t* __restrict__ segcnt, uint32_t* __restrict__ flags,
    int max_ctx, int S, int k, int L, int n_seg, int mq) {
  constexpr int NQ = 2 * TB, NL = TB / 64;
  __shared__ __align__(16) int8_t s_q[kMaxQueries * NQ];
  __shared__ uint32_t s_cnt[kThreads / 64][16];
  // VALU: each wave's 64 code rows (row stride TB + 16 bytes)
  __shared__ __align__(16) uint8_t s_w[VALU ? (kThreads / 64) * 64 * (TB + 16) : 16];
  const int b = blockIdx.y, seg = blockIdx.x;
  const int T = clamp_ctx(ctx_len, b, max_ctx, seg == 0 ? flags : nullptr);
  const Range r = cand_range(SKV_INDEX_SKETCH_INT4, T, S, k, L);   // the last query's range
  if (r.dense) return;
  const int i0 = seg * kSegTok;
  if (i0 >= r.n) return;   // workgroup-uniform
  const int i1 = min(r.n, i0 + kSegTok);
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int j = lane & 15, g = lane >> 4;
  const int first = i0 + 64 * wave;
  // the scale, the query rows and then the wave's 64 tokens: loads return in
  // order, so the LDS staging before the barrier waits only for the first
  // ones and the tiles can start as their codes arrive
  const uint32_t sc_l = isc[(size_t)b * max_ctx + r.lo + min(first + lane, i1 - 1)];
  const QueryRange qr = query_range(T, mq, j, S, k, L);
  const uint32_t beta = qr.active ? state[(size_t)b * mq + j].beta : 0xFFFFFFFFu;
  {
    const uint32_t* src = reinterpret_cast<const uint32_t*>(qs + (size_t)b * mq * NQ);
    uint32_t* dst = reinterpret_cast<uint32_t*>(s_q);
#pragma unroll
    for (int u = 0; u < kMaxQueries * NQ / 4 / kThreads; ++u) {
      const int i = threadIdx.x + u * kThreads;
      const uint32_t v = src[min(i, mq * NQ / 4 - 1)];   // unconditional
      dst[i] = i < mq * NQ / 4 ? v : 0u;
    }
  }
  const uint8_t* cb = ik + (size_t)b * max_ctx * TB + 16 * g;
  u32x4 w[kTiles][NL];
#pragma unroll
  for (int t = 0; t < kTiles; ++t) {
    const int i = min(first + 16 * t + j, i1 - 1);   // past the end: re-read, dropped below
#pragma unroll
    for (int m = 0; m < NL; ++m)
      w[t][m] = __builtin_nontemporal_load(
          reinterpret_cast<const u32x4*>(cb + (size_t)(r.lo + i) * TB + 64 * m));
  }
  if constexpr (VALU) {
    // lane (j, g) holds bytes [16g + 64m, +16) of token 16t + j of the batch
#pragma unroll
    for (int t = 0; t < kTiles; ++t)
#pragma unroll
      for (int m = 0; m < NL; ++m)
        *reinterpret_cast<u32x4*>(s_w + (wave * 64 + 16 * t + j) * (TB + 16) + 16 * g + 64 * m) = w[t][m];
  }
  __syncthreads();
  MqTile<TB> tile;
  MqTileValu<TB> vtile;
  if constexpr (VALU) vtile.init(s_q, lane);
  else tile.init(s_q, lane);

  // pass 1: digits and selection; bit 4t+e of mask = token 16t + 4g + e of the batch
  v4i c[kTiles];
  uint32_t scs[kTiles][4];
  uint32_t mask = 0;
#pragma unroll
  for (int t = 0; t < kTiles; ++t) {
    if constexpr (VALU) c[t] = vtile.dots(s_w + (wave * 64 + 16 * t) * (TB + 16), lane);
    else c[t] = tile.mma(w[t]);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      scs[t][e] = __shfl(sc_l, 16 * t + 4 * g + e);
      const int i = first + 16 * t + 4 * g + e;
      const bool sel = i < qr.n && mq_digit(c[t][e] >> 4, scs[t][e]) >= beta;
      mask |= (sel ? 1u : 0u) << (4 * t + e);
    }
  }
  // the masks of the four lanes of this query (tokens 4g'..4g'+3 of each tile)
  uint32_t mg[4];
#pragma unroll
  for (int q = 0; q < 4; ++q) mg[q] = (uint32_t)__shfl((int)mask, j + 16 * q);
  const uint32_t wave_tot = __popc(mg[0]) + __popc(mg[1]) + __popc(mg[2]) + __popc(mg[3]);
  if (g == 0) s_cnt[wave][j] = wave_tot;
  __syncthreads();
  uint32_t off = 0, tot = 0;
#pragma unroll
  for (int v = 0; v < kThreads / 64; ++v) {
    const uint32_t n = s_cnt[v][j];
    off += v < wave ? n : 0u;
    tot += n;
  }
  // pass 2: records in position order (tiles, then lanes of the query, then e)
  if (j < mq) {
    u32x4* cseg = reinterpret_cast<u32x4*>(cand + (((size_t)b * mq + j) * n_seg + seg) * kSegTok);
    uint32_t before = off;
#pragma unroll
    for (int t = 0; t < kTiles; ++t) {
      uint32_t grp = 0, tile_n = 0;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const uint32_t nq = __popc((mg[q] >> (4 * t)) & 0xFu);
        grp += q < g ? nq : 0u;
        tile_n += nq;
      }
      const uint32_t mine = (mask >> (4 * t)) & 0xFu;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        if (mine & (1u << e)) {
          const int dt = c[t][e] >> 4;
          const uint64_t okey = ordered_u64(mq_key(dt, scs[t][e]));
          const uint32_t rank = before + grp + __popc(mine & ((1u << e) - 1u));
          cseg[rank] = (u32x4){(uint32_t)okey, (uint32_t)(okey >> 32),
                               (uint32_t)(r.lo + first + 16 * t + 4 * g + e), mq_digit(dt, scs[t][e])};
        }
      }
      before += tile_n;
    }
    if (wave == 0 && g == 0) segcnt[((size_t)b * mq + j) * n_seg + seg] = tot;
  }
}

template <int TB>
hipError_t launch_multi_tb(const skv_layer_desc& dv, int mq, const int32_t* ctx_len, int8_t* qs_out,
                           float* qscale_out, const uint8_t* ik, const uint16_t* isc, void* ws,
                           const WsLayout& L, hipStream_t st) {
  const int B = dv.batch / mq;
  const dim3 sgrid((L.n_samp + kTiles * (kThreads / 64) - 1) / (kTiles * (kThreads / 64)), B);
  hipLaunchKernelGGL((sample_multi_kernel<TB>), sgrid, dim3(kThreads), 0, st,
                     ws_ptr<const float>(ws, L.sproj), qs_out, qscale_out, mq, ik, isc, ctx_len,
                     ws_ptr<uint16_t>(ws, L.sdig), L.n_samp, dv.max_ctx, dv.n_sink, dv.topk,
                     dv.n_tail);
  hipError_t e = hipGetLastError();
  if (e == hipSuccess) e = launch_beta(dv, mq, ctx_len, ws, L, st);
  if (e != hipSuccess) return e;
  const dim3 grid(L.n_seg, B);
  hipEvent_t ev0 = nullptr, ev1 = nullptr;
  const bool timed = timer_next(kTimerStream, &ev0, &ev1);
#define SKV_SM(VV)                                                                                 \
  do {                                                                                             \
    if (timed)                                                                                     \
      hipExtLaunchKernelGGL((score_multi_kernel<TB, VV>), grid, dim3(kThreads), 0, st, ev0, ev1, 0, \
                            (const int8_t*)qs_out, ik, isc, ctx_len,                               \
                            ws_ptr<const TopkState>(ws, L.state), ws_ptr<Cand>(ws, L.cand),        \
                            ws_ptr<uint32_t>(ws, L.segcnt), ws_ptr<uint32_t>(ws, L.flags),         \
                            dv.max_ctx, dv.n_sink, dv.topk, dv.n_tail, L.n_seg, mq);               \
    else                                                                                           \
      hipLaunchKernelGGL((score_multi_kernel<TB, VV>), grid, dim3(kThreads), 0, st,                \
                         (const int8_t*)qs_out, ik, isc, ctx_len,                                  \
                         ws_ptr<const TopkState>(ws, L.state), ws_ptr<Cand>(ws, L.cand),           \
                         ws_ptr<uint32_t>(ws, L.segcnt), ws_ptr<uint32_t>(ws, L.flags),            \
                         dv.max_ctx, dv.n_sink, dv.topk, dv.n_tail, L.n_seg, mq);                  \
  } while (0)
  // the vector-ALU variant (a measurement aid) for sketch rows up to 128 bytes
  if constexpr (TB <= 128) {
    if (g_contract_path == SKV_PATH_VALU) SKV_SM(true);
    else SKV_SM(false);
  } else {
    SKV_SM(false);
  }
#undef SKV_SM
  return hipGetLastError();
}

}  // namespace

hipError_t launch_sample_collect_multi(const skv_layer_desc& dv, int mq, const int32_t* ctx_len,
                                       int8_t* qs_out, float* qscale_out, const void* ik,
                                       const uint16_t* isc, void* ws, const WsLayout& L,
                                       hipStream_t st) {
  if (mq < 1 || mq > kMaxQueries || dv.batch % mq || dv.index_mode != SKV_INDEX_SKETCH_INT4)
    return hipErrorInvalidValue;
  const uint8_t* ikb = reinterpret_cast<const uint8_t*>(ik);
  switch (dv.n_kv_heads * dv.rank / 2) {
    case 64: return launch_multi_tb<64>(dv, mq, ctx_len, qs_out, qscale_out, ikb, isc, ws, L, st);
    case 128: return launch_multi_tb<128>(dv, mq, ctx_len, qs_out, qscale_out, ikb, isc, ws, L, st);
    case 256: return launch_multi_tb<256>(dv, mq, ctx_len, qs_out, qscale_out, ikb, isc, ws, L, st);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace skv
