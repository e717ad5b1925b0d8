// Device pieces shared by the score and select stages: the exact ranking key
// of one candidate (token sketch or pooled block key), the candidate range of
// a sequence, the sampling rule of the threshold estimate, candidate records
// and DPP wave reductions / scans.
#pragma once

#include "skv_internal.h"

namespace skv {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int kLineKeys = 16;          // candidates per sample line
constexpr int kSampleCap = 16384;      // sampled candidates per sequence, at most (+16)

// Threshold digit of an exact key: the top 16 bits of the order-preserving
// image of the key rounded to fp32 (rounding is monotone, so digits are
// ordered); a bucket spans 1/128 of an octave.  Finite keys have digits in
// [0x0080, 0xFF7F], so 0 marks an empty sample slot: it sorts below every
// sample and only matters when the samples are fewer than needed.
__device__ __forceinline__ uint32_t key_digit16(double x) {
  return ordered_u32(__double2float_rn(x)) >> 16;
}

// ---------------------------------------------------------------------------
// candidate range of a sequence
// ---------------------------------------------------------------------------
// Token mode ranks the middle tokens [S, T-L) (page "8 agents x 250K context
// on two 3090s ...", section "The mechanism": the sinks and the tail are always
// kept); block mode ranks the floor(T/4) complete blocks (page "3.14M Context
// on 3x 3090 ...", section "Why": dense until T > 4*block_topk+3).
struct Range {
  int T, lo, n;   // candidates are positions lo .. lo+n (tokens or blocks)
  bool dense;
};

__device__ __forceinline__ Range cand_range(int mode, int T, int S, int k, int L) {
  Range r;
  r.T = T;
  if (mode == SKV_INDEX_SKETCH_INT4) {
    r.dense = T <= S + k + L;
    r.lo = S;
    r.n = r.dense ? 0 : T - S - L;
  } else {
    const int nb = T / 4;
    r.dense = nb <= k;
    r.lo = 0;
    r.n = r.dense ? 0 : nb;
  }
  return r;
}

__device__ __forceinline__ int ctx_of(const int32_t* ctx_len, int b, int max_ctx) {
  const int T = ctx_len[b];
  return T < 0 ? 0 : (T > max_ctx ? max_ctx : T);
}

// A step with mq query tokens per sequence (the last mq positions of the
// cache, which ctx_len counts): virtual sequence v is query j = v % mq of
// sequence v / mq, whose causal context is T - mq + 1 + j tokens (0 when the
// cache is shorter than the step).  mq = 1 is the ordinary decode step.
__device__ __forceinline__ int ctx_of_query(const int32_t* ctx_len, int v, int mq, int max_ctx) {
  const int T = ctx_of(ctx_len, v / mq, max_ctx) - (mq - 1 - v % mq);
  return T < 0 ? 0 : T;
}

// Sample: whole lines of 16 candidates, one line in every s; about 4k lines'
// worth of keys, at most about 16K, and at least every (k/256)-th line, so
// that a sample never holds more than about 256 keys of the top k expected
// (every key when the sequence is short and k <= 256).
__host__ __device__ __forceinline__ int sample_stride(int n, int k) {
  int s = n / (4 * k);
  const int s2 = (n + kSampleCap - 1) / kSampleCap;
  const int s3 = (k + 255) / 256;
  s = s > s2 ? s : s2;
  s = s > s3 ? s : s3;
  return s < 1 ? 1 : s;
}
__host__ __device__ __forceinline__ int sample_lines(int n, int k) {
  const int lines = (n + kLineKeys - 1) / kLineKeys;
  const int s = sample_stride(n, k);
  return (lines + s - 1) / s;
}

// Samples that must lie at or above the threshold bucket: k when every key is
// sampled, else the expected share of the top k plus 25%, four standard
// deviations and 8 (the sample only steers speed; the select stays exact).
// The stride rule above keeps it at most about 420.
__host__ __device__ __forceinline__ uint32_t sample_need(int n, int k) {
  const int s = sample_stride(n, k);
  if (s == 1) return (uint32_t)k;
  const int lines = (n + kLineKeys - 1) / kLineKeys;
  const int nsl = (lines + s - 1) / s;
  const float e = (float)k * (float)nsl / (float)lines;
  return (uint32_t)ceilf(1.25f * e + 4.0f * sqrtf(e) + 8.0f);
}

// ---------------------------------------------------------------------------
// front of the fused step: the sample is read by workgroups of kFrontThreads,
// 8 loads per lane, each covering front_lines(LANES) consecutive sample lines
// (4 to 32): the sample is spread over many compute units, each of which
// gathers only a few lines; every sampled digit is written out and the
// threshold is the need-th largest of them
// ---------------------------------------------------------------------------
constexpr int kFrontThreads = 256;
constexpr int kFrontUnroll = 8;
__host__ __device__ constexpr int front_lines(int lanes) {   // sample lines per front workgroup
  return (kFrontThreads / 64) * kFrontUnroll * (64 / lanes) / kLineKeys;
}
__host__ __device__ __forceinline__ int front_wgs(int nsl, int lanes) {
  return (nsl + front_lines(lanes) - 1) / front_lines(lanes);
}

// ---------------------------------------------------------------------------
// candidate records: (order-preserving key, position, 16-bit digit), 16 bytes
// ---------------------------------------------------------------------------
struct alignas(16) Cand {
  uint32_t klo, khi, pos, digit;
};
__device__ __forceinline__ uint64_t cand_key(const Cand& c) { return ((uint64_t)c.khi << 32) | c.klo; }

// ---------------------------------------------------------------------------
// DPP helpers (all 64 lanes of the wave must be active)
// ---------------------------------------------------------------------------
template <int CTRL, int ROWMASK = 0xF>
__device__ __forceinline__ uint32_t dpp_u32(uint32_t v) {
  return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, CTRL, ROWMASK, 0xF, true);
}

// inclusive prefix sum over the 64 lanes
__device__ __forceinline__ uint32_t wave_incl_scan(uint32_t v) {
  v += dpp_u32<0x111>(v);           // row_shr:1
  v += dpp_u32<0x112>(v);           // row_shr:2
  v += dpp_u32<0x114>(v);           // row_shr:4
  v += dpp_u32<0x118>(v);           // row_shr:8
  v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x142, 0xA, 0xF, false);  // row_bcast:15
  v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x143, 0xC, 0xF, false);  // row_bcast:31
  return v;
}

// bitwise AND / OR / max over the 64 lanes, returned in every lane
__device__ __forceinline__ uint32_t wave_and(uint32_t v) {
  v &= dpp_u32<0xB1>(v);
  v &= dpp_u32<0x4E>(v);
  v &= dpp_u32<0x141>(v);
  v &= dpp_u32<0x140>(v);
  return (uint32_t)__builtin_amdgcn_readlane((int)v, 0) & (uint32_t)__builtin_amdgcn_readlane((int)v, 16) &
         (uint32_t)__builtin_amdgcn_readlane((int)v, 32) & (uint32_t)__builtin_amdgcn_readlane((int)v, 48);
}
__device__ __forceinline__ uint32_t wave_or(uint32_t v) {
  v |= dpp_u32<0xB1>(v);
  v |= dpp_u32<0x4E>(v);
  v |= dpp_u32<0x141>(v);
  v |= dpp_u32<0x140>(v);
  return (uint32_t)__builtin_amdgcn_readlane((int)v, 0) | (uint32_t)__builtin_amdgcn_readlane((int)v, 16) |
         (uint32_t)__builtin_amdgcn_readlane((int)v, 32) | (uint32_t)__builtin_amdgcn_readlane((int)v, 48);
}
__device__ __forceinline__ uint32_t wave_sum(uint32_t v) {
  v += dpp_u32<0xB1>(v);
  v += dpp_u32<0x4E>(v);
  v += dpp_u32<0x141>(v);
  v += dpp_u32<0x140>(v);
  return (uint32_t)__builtin_amdgcn_readlane((int)v, 0) + (uint32_t)__builtin_amdgcn_readlane((int)v, 16) +
         (uint32_t)__builtin_amdgcn_readlane((int)v, 32) + (uint32_t)__builtin_amdgcn_readlane((int)v, 48);
}

__device__ __forceinline__ uint32_t wave_max(uint32_t v) {
  v = max(v, dpp_u32<0xB1>(v));
  v = max(v, dpp_u32<0x4E>(v));
  v = max(v, dpp_u32<0x141>(v));
  v = max(v, dpp_u32<0x140>(v));
  return max(max((uint32_t)__builtin_amdgcn_readlane((int)v, 0), (uint32_t)__builtin_amdgcn_readlane((int)v, 16)),
             max((uint32_t)__builtin_amdgcn_readlane((int)v, 32), (uint32_t)__builtin_amdgcn_readlane((int)v, 48)));
}

// lanes below this one, as a 64-bit mask
__device__ __forceinline__ uint64_t lanemask_lt() {
  const int lane = threadIdx.x & 63;
  return lane == 0 ? 0ull : (~0ull >> (64 - lane));
}

// Per-wave partials in LDS (16 slots; slots of absent waves are ignored) are
// combined with all 16 reads issued at once -- a loop bounded by the wave
// count would wait for each read in turn.
__device__ __forceinline__ uint32_t lds_sum16(const uint32_t* red, int nw) {
  uint32_t s = 0;
#pragma unroll
  for (int w = 0; w < 16; ++w) {
    const uint32_t v = red[w];
    s += w < nw ? v : 0u;
  }
  return s;
}
__device__ __forceinline__ uint32_t lds_max16(const uint32_t* red, int nw) {
  uint32_t s = 0;
#pragma unroll
  for (int w = 0; w < 16; ++w) {
    const uint32_t v = red[w];
    s = max(s, w < nw ? v : 0u);
  }
  return s;
}

// Block-wide exclusive prefix sum of one value per thread, in thread order
// (blockDim.x a multiple of 64, <= 1024).  `wsum` is LDS scratch of 16 words.
// Contains barriers: every thread of the block must call it.
__device__ __forceinline__ uint32_t block_excl_scan(uint32_t v, uint32_t* wsum, uint32_t* total) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int nw = blockDim.x >> 6;
  const uint32_t incl = wave_incl_scan(v);
  __syncthreads();
  if (lane == 63) wsum[wave] = incl;
  __syncthreads();
  uint32_t base = 0, tot = 0;
#pragma unroll
  for (int w = 0; w < 16; ++w) {
    const uint32_t s = wsum[w];
    base += w < wave ? s : 0u;
    tot += w < nw ? s : 0u;
  }
  if (total) *total = tot;
  return base + incl - v;
}

// ---------------------------------------------------------------------------
// exact keys
// ---------------------------------------------------------------------------
// Sum over aligned groups of N lanes (N in {2,4,8,16}); every lane of the
// group ends with the group total.
template <int N>
__device__ __forceinline__ int group_sum_i32(int v) {
  v += __builtin_amdgcn_update_dpp(0, v, 0xB1, 0xF, 0xF, false);                // quad_perm [1,0,3,2]
  if (N >= 4) v += __builtin_amdgcn_update_dpp(0, v, 0x4E, 0xF, 0xF, false);    // quad_perm [2,3,0,1]
  if (N >= 8) v += __builtin_amdgcn_update_dpp(0, v, 0x141, 0xF, 0xF, false);   // row_half_mirror
  if (N >= 16) v += __builtin_amdgcn_update_dpp(0, v, 0x140, 0xF, 0xF, false);  // row_mirror
  return v;
}

template <int CTRL>
__device__ __forceinline__ double dpp_add_f64(double v) {
  const long long u = __double_as_longlong(v);
  const int lo = __builtin_amdgcn_update_dpp(0, (int)(u & 0xFFFFFFFF), CTRL, 0xF, 0xF, false);
  const int hi = __builtin_amdgcn_update_dpp(0, (int)(u >> 32), CTRL, 0xF, 0xF, false);
  return v + __longlong_as_double(((long long)hi << 32) | (unsigned)lo);
}

template <int N>
__device__ __forceinline__ double group_sum_f64(double x) {
  x = dpp_add_f64<0xB1>(x);
  if (N >= 4) x = dpp_add_f64<0x4E>(x);
  if (N >= 8) x = dpp_add_f64<0x141>(x);
  if (N >= 16) x = dpp_add_f64<0x140>(x);
  if (N >= 32) x += __shfl_xor(x, 16);
  return x;
}

// int4 x int8 dot of 32 codes held in one 16-byte load.  The nibbles of each
// 32-bit word are moved to the high half of their byte (x16, still a signed
// int8), dotted with the matching query bytes, and the sum is divided by 16
// at the end (exact: every term is a multiple of 16).
__device__ __forceinline__ int dot32_i4(const u32x4 w, const uint32_t qe[4], const uint32_t qo[4], int acc) {
  const uint32_t ws[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
  for (int m = 0; m < 4; ++m) {
    acc = __builtin_amdgcn_sdot4((int)qe[m], (int)((ws[m] << 4) & 0xF0F0F0F0u), acc, false);
    acc = __builtin_amdgcn_sdot4((int)qo[m], (int)(ws[m] & 0xF0F0F0F0u), acc, false);
  }
  return acc;
}

// Token sketch source: a candidate is a token whose H_kv*R int4 codes (16*N
// bytes) are read by N lanes, 16 bytes each, plus its fp16 scale.  The key is
// the integer dot with the int8 query sketch times the scale, exact in fp64.
template <int N>
struct SketchSrc {
  static constexpr int LANES = N;
  static constexpr bool HAS_AUX = true;    // integer dot times a per-token fp16 scale
  static constexpr int QROW = 32 * N;      // bytes of one sequence's query row
  uint32_t qe[4], qo[4];
  const uint8_t* cbase;     // this lane's 16 bytes of token 0 of the sequence
  const uint16_t* sbase;    // scales of the sequence

  // qrow: the sequence's 32*N int8 query codes (global or LDS)
  __device__ __forceinline__ void init(const void* qrow, const void* ik, const uint16_t* isc, int b,
                                       int max_ctx, int sub) {
    init_data(ik, isc, b, max_ctx, sub);
    init_query(qrow, sub);
  }
  __device__ __forceinline__ void init_data(const void* ik, const uint16_t* isc, int b, int max_ctx,
                                            int sub) {
    constexpr int TB = 16 * N;
    cbase = reinterpret_cast<const uint8_t*>(ik) + (size_t)b * max_ctx * TB + 16 * sub;
    sbase = isc + (size_t)b * max_ctx;
  }
  __device__ __forceinline__ void init_query(const void* qrow, int sub) {
    // this lane's 32 query codes: even code positions of each 8-code word in
    // qe, odd ones in qo (matching the low / high nibbles of the code bytes)
    const uint8_t* qp = reinterpret_cast<const uint8_t*>(qrow) + 32 * sub;
#pragma unroll
    for (int m = 0; m < 4; ++m) {
      uint32_t e = 0, o = 0;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        e |= (uint32_t)qp[8 * m + 2 * j] << (8 * j);
        o |= (uint32_t)qp[8 * m + 2 * j + 1] << (8 * j);
      }
      qe[m] = e;
      qo[m] = o;
    }
  }
  // raw data of candidate at position p (token index)
  __device__ __forceinline__ u32x4 load(int p) const {
    return __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(cbase + (size_t)p * (16 * N)));
  }
  __device__ __forceinline__ uint32_t load_aux(int p) const { return sbase[p]; }
  // this lane's share of 16x the integer dot (its 32 codes)
  __device__ __forceinline__ int partial(const u32x4 w) const { return dot32_i4(w, qe, qo, 0); }
  // the integer dot; every lane of the candidate's group must call it (DPP sum)
  __device__ __forceinline__ int dot(const u32x4 w) const {
    return group_sum_i32<N>(partial(w)) >> 4;
  }
  // the key from the dot: exact in fp64 (at most 19 + 11 significant bits)
  __device__ __forceinline__ double key_of(int d, uint32_t aux) const {
    return (double)d * (double)half_bits_to_float((uint16_t)aux) + 0.0;  // -0 -> +0
  }
  // the key's 16-bit digit without fp64: the key rounded to fp32 equals the
  // fp32 product of the (exact) fp32 dot and scale, which is rounded once
  __device__ __forceinline__ uint32_t digit_of(int d, uint32_t aux) const {
    return ordered_u32((float)d * half_bits_to_float((uint16_t)aux) + 0.0f) >> 16;
  }
  __device__ __forceinline__ double key(const u32x4 w, uint32_t aux) const { return key_of(dot(w), aux); }
};

// Pooled block source: a candidate is a complete 4-token block whose bf16
// pooled key (8*N values) is read by N lanes, 8 values each.  The key is the
// fp64 sum of the exact fp32 products (exact in the bf16 domain [2^-8, 2^8)).
template <int N>
struct PooledSrc {
  static constexpr int LANES = N;
  static constexpr bool HAS_AUX = false;
  static constexpr int QROW = 16 * N;      // bytes of one sequence's query row
  double qd[8];
  const uint16_t* kb;

  // qrow: the sequence's 8*N bf16 indexer query values
  __device__ __forceinline__ void init(const void* qrow, const void* ik, const uint16_t* isc, int b,
                                       int max_ctx, int sub) {
    init_data(ik, isc, b, max_ctx, sub);
    init_query(qrow, sub);
  }
  __device__ __forceinline__ void init_data(const void* ik, const uint16_t*, int b, int max_ctx, int sub) {
    constexpr int ID = 8 * N;
    kb = reinterpret_cast<const uint16_t*>(ik) + (size_t)b * (max_ctx / 4) * ID + 8 * sub;
  }
  __device__ __forceinline__ void init_query(const void* qrow, int sub) {
    const uint16_t* q = reinterpret_cast<const uint16_t*>(qrow);
#pragma unroll
    for (int e = 0; e < 8; ++e) qd[e] = (double)bf16_bits_to_float(q[8 * sub + e]);
  }
  __device__ __forceinline__ u32x4 load(int p) const {
    return __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(kb + (size_t)p * (8 * N)));
  }
  __device__ __forceinline__ uint32_t load_aux(int) const { return 0u; }
  __device__ __forceinline__ double key(const u32x4 w, uint32_t) const {
    const uint32_t ws[4] = {w.x, w.y, w.z, w.w};
    double acc = 0.0;
#pragma unroll
    for (int m = 0; m < 4; ++m) {
      acc = fma((double)__uint_as_float(ws[m] << 16), qd[2 * m], acc);
      acc = fma((double)__uint_as_float(ws[m] & 0xFFFF0000u), qd[2 * m + 1], acc);
    }
    return group_sum_f64<N>(acc) + 0.0;   // -0 -> +0
  }
};

// ---------------------------------------------------------------------------
// query sketch quantization (page "8 agents x 250K ...", section "The
// mechanism": the query sketch is an int8 vector): one scale per sequence,
// max|s|/127 correctly rounded to fp32, codes rint(s/scale) clamped to +-127,
// the quotients computed in fp64 and rounded once (exact fp32 division).
// ---------------------------------------------------------------------------
// The n <= 2*blockDim.x values at sp (global) become codes q8[0..n) in LDS;
// returns the scale.  Every thread of the block must call it.
__device__ __forceinline__ float quantize_sketch(const float* sp, int n, int8_t* q8, uint32_t* red) {
  const int t = threadIdx.x, nb = blockDim.x;
  const float v0 = sp[min(t, n - 1)], v1 = sp[min(t + nb, n - 1)];   // unconditional loads
  const bool ok0 = t < n, ok1 = t + nb < n;
  // |x| >= 0, so its bit pattern orders like the value
  uint32_t am = max(ok0 ? __float_as_uint(fabsf(v0)) : 0u, ok1 ? __float_as_uint(fabsf(v1)) : 0u);
  am = wave_max(am);
  if ((t & 63) == 0) red[t >> 6] = am;
  __syncthreads();
  am = lds_max16(red, nb >> 6);
  const float amax = __uint_as_float(am);
  const float scale = amax == 0.0f ? 0.0f : (float)((double)amax / 127.0);
  auto code = [&](float v) -> int8_t {
    if (amax == 0.0f) return 0;
    float r = rintf((float)((double)v / (double)scale));
    r = fminf(fmaxf(r, -127.0f), 127.0f);
    return (int8_t)(int)r;
  };
  if (ok0) q8[t] = code(v0);
  if (ok1) q8[t + nb] = code(v1);
  __syncthreads();
  return scale;
}

// ---------------------------------------------------------------------------
// threshold digit from the sampled digits
// ---------------------------------------------------------------------------
// dg: the sequence's ns sampled digits (16 bits, 0 = empty slot), ns a
// multiple of 8 and at most 16 * blockDim.x.  Returns the need-th largest
// digit, which is the largest beta with at least `need` samples at or above
// it -- or 0 (keep everything) when fewer than `need` samples exist, since
// empty slots count as digit 0.
// The sampled top of the distribution is narrow, so it is found in a window
// of 256 digit values (two octaves) below the largest sample: an LDS
// histogram of the samples in the window (they spread over many bins, so
// the atomics hardly collide), then one scan from the top.  If the window
// holds fewer than the remaining count, the next window starts at the
// largest sample below it.  Every thread of the block must call it; red is
// LDS scratch of 256 + 32 words.
__device__ __forceinline__ uint32_t wg_beta(const uint16_t* dg, int ns, uint32_t need, uint32_t* red) {
  const int nv = ns / 8;   // 16-byte chunks
  const int t = threadIdx.x, nb = blockDim.x, nw = nb >> 6, lane = t & 63, wave = t >> 6;
  uint32_t* hist = red;          // [256], bin i = digit top - i
  uint32_t* wr = red + 256;      // [16] per-wave partials, [16..18] broadcast
  uint32_t d[8];                 // 16 digits, two per word
#pragma unroll
  for (int m = 0; m < 2; ++m) {
    const int c = t + m * nb;
    u32x4 v = reinterpret_cast<const u32x4*>(dg)[min(c, nv - 1)];   // unconditional
    if (c >= nv) v = (u32x4){0u, 0u, 0u, 0u};
    d[4 * m + 0] = v.x;
    d[4 * m + 1] = v.y;
    d[4 * m + 2] = v.z;
    d[4 * m + 3] = v.w;
  }
  // largest digit strictly below `lim` (0 if none), over the block
  auto max_below = [&](uint32_t lim) -> uint32_t {
    uint32_t m = 0;
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      const uint32_t x = (e & 1) ? d[e >> 1] >> 16 : d[e >> 1] & 0xFFFFu;
      m = max(m, x < lim ? x : 0u);
    }
    m = wave_max(m);
    __syncthreads();
    if (lane == 0) wr[wave] = m;
    __syncthreads();
    return lds_max16(wr, nw);
  };
  uint32_t top = max_below(0x10000u), rem = need;
  for (;;) {
    for (int i = t; i < 256; i += nb) hist[i] = 0u;
    __syncthreads();
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      const uint32_t x = (e & 1) ? d[e >> 1] >> 16 : d[e >> 1] & 0xFFFFu;
      const uint32_t dist = top - x;            // wraps for x > top
      if (dist < 256u) atomicAdd(&hist[dist], 1u);
    }
    __syncthreads();
    if (wave == 0) {
      // lane l holds bins 4l..4l+3 (digits top-4l .. top-4l-3), top first
      uint32_t c[4], s = 0;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        c[j] = hist[4 * lane + j];
        s += c[j];
      }
      const uint32_t incl = wave_incl_scan(s);
      const uint32_t tot = (uint32_t)__builtin_amdgcn_readlane((int)incl, 63);
      const uint64_t m = __ballot(incl >= rem);
      const int l = m ? (int)__ffsll((unsigned long long)m) - 1 : 0;
      uint32_t cum = incl - s, dist = 0;
      bool found = false;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        if (!found && cum + c[j] >= rem) {
          found = true;
          dist = (uint32_t)(4 * lane + j);
        }
        cum += c[j];
      }
      const uint32_t dsel = (uint32_t)__builtin_amdgcn_readlane((int)dist, l);
      if (lane == 0) {
        wr[16] = m ? 1u : 0u;              // reached inside this window
        wr[17] = top - dsel;               // the digit, if reached
        wr[18] = tot;                      // samples in the window
      }
    }
    __syncthreads();
    const uint32_t hit = wr[16], val = wr[17], tot = wr[18];
    __syncthreads();
    if (hit) return val;
    rem -= tot;
    if (top < 256u) return 0u;             // every sample counted: fewer than need
    top = max_below(top - 255u);
  }
}

}  // namespace skv
