// The decode-step append: the new token of every sequence is written into the
// caches the step reads.
//
// Page "8 agents x 250K context on two 3090s: sparse KV decode with a rank-64
// key sketch and a host-RAM tier", section "The mechanism": every token has
// int8 K/V rows with a per-row scale and an int4 rank-64 sketch of its keys on
// a frozen basis with one fp16 scale.  Page "3.14M Context on 3x 3090: The
// Power of an Architecture That Puts KV Cache in Host RAM", section "No Need
// to Rewrite the Kernel": the paged cache update writes the new rows in place
// each step.
//
// Encodings (the pages give none; the plainest rounding, in a fixed fp32
// order so the integer codes are reproducible bit for bit):
//   int8 row   scale = fp16(fp32(amax / 127)), codes = clamp(rint(x / scale), +-127)
//   key sketch v[h*R + r] = sum over d ascending of k_h[d] * B_h[d][r] (fp32,
//              product and sum rounded separately); scale = fp16(fp32(amax / 7))
//              over all H_kv*R values; codes clamp(rint(v / scale), +-7), element
//              2j in the low nibble of byte j
//   position   row ctx_len[b], then ctx_len[b] += 1 (a full sequence is left as
//              it is and flagged)
// Quotients are computed in fp64 and rounded once, which is the correctly
// rounded fp32 quotient.
//
// One workgroup of 512 threads per sequence: the 2*H_kv rows go to the waves
// (a row's amax by a DPP max over the wave), then thread i computes sketch
// value i from the K rows staged in LDS.
//
// Host tier (same page, same section: every token's K/V also lives in host RAM
// as int4 in 64-dim groups with fp16 group scales; the GPU keeps sinks and
// tail): the same kernel then also writes the token's host record (group
// scale fp16(fp32(amax / 7)), codes clamp(rint(x / g), +-7), the D/2 code
// bytes then the D/64 scales, K row then V row) through the device address of
// the mapped host memory, and writes the int8 rows into the tail ring of the
// resident rows (position p at row S + ((p - anchor) mod L)) instead of row p
// of a full cache.  The tier's own per-sequence context must equal ctx_len;
// both advance together.
#include "keys_common.h"

#include <hip/hip_ext.h>

namespace skv {
namespace {

constexpr int kAppThreads = 512;
constexpr int kAppMaxHkv = 32;   // H_kv * R <= 512 with R >= 16

__device__ __forceinline__ float quot_rn(float a, float c) { return (float)((double)a / (double)c); }


// TIER: also the host record and the tail ring (AppendTarget); the plain
// cache append compiles without those paths
template <int D, bool I8, bool TIER>
__global__ __launch_bounds__(kAppThreads) void append_kernel(
    int32_t* __restrict__ ctx_len, const __half* __restrict__ k_new, const __half* __restrict__ v_new,
    const float* __restrict__ basis, uint8_t* __restrict__ kc, uint8_t* __restrict__ vc,
    uint16_t* __restrict__ ksc, uint16_t* __restrict__ vsc, int64_t rows,
    uint8_t* __restrict__ codes, uint16_t* __restrict__ sk_scale, int Hkv, int R, int max_ctx,
    uint32_t* __restrict__ flags, AppendTarget tg) {
#pragma clang fp contract(off)
  constexpr int PL = D / 64;   // row values per lane
  constexpr int HROW = D / 2 + 2 * (D / 64);   // host bytes of one K (or V) row
  __shared__ float s_k[kAppMaxHkv * D];
  __shared__ int8_t s_c[kAppThreads];
  __shared__ uint32_t s_red[16];
  const int b = blockIdx.x;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, nw = kAppThreads / 64;
  const int t = ctx_len[b];
  if (t < 0 || t >= max_ctx) {   // the same t in every thread: the whole workgroup leaves
    if (threadIdx.x == 0) raise_flag(flags, SKV_FLAG_CTX_RANGE);
    return;
  }
  if (TIER && tg.tier_ctx[b] != t) {   // the tier and the caller disagree
    if (threadIdx.x == 0) raise_flag(flags, SKV_FLAG_TIER_INPUT);
    return;
  }
  // cache row of position t: row t of a full cache, a ring row of a tier's
  // tail, or none (a tier without a tail)
  int crow = t;
  if (!TIER) {
  } else if (tg.ring_len == 0) {
    crow = -1;
  } else if (tg.ring_len > 0) {
    int r = (t - tg.ring_anchor) % tg.ring_len;
    crow = tg.ring_base + (r < 0 ? r + tg.ring_len : r);
  }
  // ---- K and V rows: wave w takes rows w, w + nw, ... (K rows first) ----
  for (int row = wave; row < 2 * Hkv; row += nw) {
    const bool isv = row >= Hkv;
    const int h = isv ? row - Hkv : row;
    const __half* src = (isv ? v_new : k_new) + ((size_t)b * Hkv + h) * D + lane * PL;
    float x[PL];
#pragma unroll
    for (int e = 0; e < PL; ++e) x[e] = __half2float(src[e]);
    if (!isv) {
#pragma unroll
      for (int e = 0; e < PL; ++e) s_k[h * D + lane * PL + e] = x[e];
    }
    if constexpr (TIER && I8 && D == 256) {
      {
        // host record: 16 lanes per 64-dim group; lane l packs elements 4l..4l+3
        float gm = 0.0f;
#pragma unroll
        for (int e = 0; e < PL; ++e) gm = fmaxf(gm, fabsf(x[e]));
#pragma unroll
        for (int o = 1; o < 16; o <<= 1) gm = fmaxf(gm, __shfl_xor(gm, o));
        const __half g16 = __float2half_rn(quot_rn(gm, 7.0f));
        const float g = __half2float(g16);
        uint32_t nib = 0;
#pragma unroll
        for (int e = 0; e < PL; ++e) {
          const float c = g > 0.0f ? fminf(fmaxf(rintf(quot_rn(x[e], g)), -7.0f), 7.0f) : 0.0f;
          nib |= ((uint32_t)(int)c & 0xFu) << (4 * e);
        }
        uint8_t* hr = tg.host + (((size_t)b * tg.host_ctx + t) * Hkv + h) * (2 * HROW) + (isv ? HROW : 0);
        *reinterpret_cast<uint16_t*>(hr + 2 * lane) = (uint16_t)nib;
        if ((lane & 15) == 0) *reinterpret_cast<uint16_t*>(hr + D / 2 + 2 * (lane >> 4)) = __half_as_ushort(g16);
      }
    }
    if (TIER && crow < 0) continue;   // a tier without a tail keeps no int8 row
    const size_t rr = ((size_t)b * rows + crow) * Hkv + h;   // cache row of (b, t, h)
    if constexpr (I8) {
      float am = 0.0f;
#pragma unroll
      for (int e = 0; e < PL; ++e) am = fmaxf(am, fabsf(x[e]));
      am = __uint_as_float(wave_max(__float_as_uint(am)));   // non-negative: bit order = value order
      const __half s16 = __float2half_rn(quot_rn(am, 127.0f));
      const float s = __half2float(s16);
      uint32_t packed = 0;
#pragma unroll
      for (int e = 0; e < PL; ++e) {
        const float q = s > 0.0f ? fminf(fmaxf(rintf(quot_rn(x[e], s)), -127.0f), 127.0f) : 0.0f;
        packed |= (uint32_t)(uint8_t)(int8_t)(int)q << (8 * e);
      }
      uint8_t* dst = (isv ? vc : kc) + rr * D + lane * PL;
      if constexpr (PL == 4) *reinterpret_cast<uint32_t*>(dst) = packed;
      else *reinterpret_cast<uint16_t*>(dst) = (uint16_t)packed;
      if (lane == 0) (isv ? vsc : ksc)[rr] = __half_as_ushort(s16);
    } else {
      __half* dst = reinterpret_cast<__half*>(isv ? vc : kc) + rr * D + lane * PL;
#pragma unroll
      for (int e = 0; e < PL; ++e) dst[e] = src[e];
    }
  }
  __syncthreads();
  // ---- key sketch: thread i computes value i = h*R + r ----
  const int n = Hkv * R;
  const int i = threadIdx.x;
  float v = 0.0f;
  if (i < n) {
    const int h = i / R, r = i % R;
    const float* bp = basis + (size_t)h * D * R + r;
    const float* kp = s_k + h * D;
    for (int d0 = 0; d0 < D; d0 += 16) {
      float bv[16];
#pragma unroll
      for (int u = 0; u < 16; ++u) bv[u] = bp[(size_t)(d0 + u) * R];
#pragma unroll
      for (int u = 0; u < 16; ++u) v = v + kp[d0 + u] * bv[u];
    }
  }
  uint32_t am = i < n ? __float_as_uint(fabsf(v)) : 0u;
  am = wave_max(am);
  if (lane == 0) s_red[wave] = am;
  __syncthreads();
  const float amax = __uint_as_float(lds_max16(s_red, nw));
  const __half s16 = __float2half_rn(quot_rn(amax, 7.0f));
  const float s = __half2float(s16);
  if (i < n) s_c[i] = (int8_t)(int)(s > 0.0f ? fminf(fmaxf(rintf(quot_rn(v, s)), -7.0f), 7.0f) : 0.0f);
  __syncthreads();
  if (i < n / 2) {
    const uint32_t lo = (uint32_t)s_c[2 * i] & 0xFu, hi = (uint32_t)s_c[2 * i + 1] & 0xFu;
    codes[((size_t)b * max_ctx + t) * (n / 2) + i] = (uint8_t)(lo | (hi << 4));
  }
  if (threadIdx.x == 0) {
    sk_scale[(size_t)b * max_ctx + t] = __half_as_ushort(s16);
    ctx_len[b] = t + 1;   // every thread read t before the barriers above
    if (TIER) tg.tier_ctx[b] = t + 1;
  }
}

// Block mode (page "3.14M Context on 3x 3090 ...", sections "Why" and "What
// Needs to Stay in VRAM": the indexer key of a 4-token block is the mean of its
// tokens' raw keys, bf16): bf16 K/V rows are stored as they are; the raw key
// goes to staging row t % 4, and at t % 4 == 3 the pooled key of block t / 4 is
// the exact mean of the four (fp64 sum of four bf16 values is exact; / 4 is
// exact), rounded to nearest-even bf16, 0 below 2^-8 in magnitude, clamped to
// +-255.  One workgroup of 256 threads per sequence.
// nearest-even bf16 of a double, rounded once: the fp64 significand is
// rounded to 8 bits on the bit pattern; the result converts to fp32 exactly
__device__ __forceinline__ uint16_t bf16_rn_bits(double x) {
  unsigned long long u = (unsigned long long)__double_as_longlong(x);
  u = ((u + ((1ull << 44) - 1ull) + ((u >> 45) & 1ull)) >> 45) << 45;
  return (uint16_t)(__float_as_uint((float)__longlong_as_double((long long)u)) >> 16);
}

template <int D>
__global__ __launch_bounds__(256) void append_block_kernel(
    int32_t* __restrict__ ctx_len, const uint16_t* __restrict__ k_new,
    const uint16_t* __restrict__ v_new, const uint16_t* __restrict__ raw_new,
    uint16_t* __restrict__ stage, uint16_t* __restrict__ kc, uint16_t* __restrict__ vc,
    int64_t rows, uint16_t* __restrict__ kp, int Hkv, int ID, int max_ctx,
    uint32_t* __restrict__ flags) {
  const int b = blockIdx.x;
  const int t = ctx_len[b];
  if (t < 0 || t >= max_ctx) {
    if (threadIdx.x == 0) raise_flag(flags, SKV_FLAG_CTX_RANGE);
    return;
  }
  const size_t rr = ((size_t)b * rows + t) * Hkv;
  for (int i = threadIdx.x; i < Hkv * D; i += blockDim.x) {
    kc[rr * D + i] = k_new[(size_t)b * Hkv * D + i];
    vc[rr * D + i] = v_new[(size_t)b * Hkv * D + i];
  }
  uint16_t* st = stage + (size_t)b * 4 * ID;
  const uint16_t* raw = raw_new + (size_t)b * ID;
  const int slot = t & 3;
  for (int i = threadIdx.x; i < ID; i += blockDim.x) {
    const uint16_t x = raw[i];
    st[slot * ID + i] = x;
    if (slot == 3) {
      double sum = 0.0;
#pragma unroll
      for (int j = 0; j < 3; ++j) sum += (double)bf16_bits_to_float(st[j * ID + i]);
      sum += (double)bf16_bits_to_float(x);
      float y = bf16_bits_to_float(bf16_rn_bits(sum * 0.25));   // the exact mean, rounded once
      y = fabsf(y) < 0.00390625f ? 0.0f : fminf(fmaxf(y, -255.0f), 255.0f);
      kp[((size_t)b * (max_ctx / 4) + (t >> 2)) * ID + i] = (uint16_t)(__float_as_uint(y) >> 16);
    }
  }
  __syncthreads();
  if (threadIdx.x == 0) ctx_len[b] = t + 1;   // every thread read t before the barrier
}

}  // namespace

hipError_t launch_append_block(const skv_layer_desc& d, int32_t* ctx_len, const void* k_new,
                               const void* v_new, const void* raw_new, void* stage,
                               const skv_kv_view& kv, void* index_keys, void* ws, const WsLayout& L,
                               hipStream_t st) {
  uint32_t* flags = ws_ptr<uint32_t>(ws, L.flags);
#define SKV_APB(DD)                                                                              \
  hipLaunchKernelGGL((append_block_kernel<DD>), dim3(d.batch), dim3(256), 0, st, ctx_len,        \
                     (const uint16_t*)k_new, (const uint16_t*)v_new, (const uint16_t*)raw_new,   \
                     (uint16_t*)stage, (uint16_t*)kv.k, (uint16_t*)kv.v, kv.rows,                \
                     (uint16_t*)index_keys, d.n_kv_heads, d.index_dim, d.max_ctx, flags)
  if (d.head_dim == 256) SKV_APB(256);
  else if (d.head_dim == 128) SKV_APB(128);
  else return hipErrorInvalidValue;
#undef SKV_APB
  return hipGetLastError();
}

hipError_t launch_append(const skv_layer_desc& d, int32_t* ctx_len, const void* k_new,
                         const void* v_new, const float* basis, const skv_kv_view& kv,
                         void* index_keys, uint16_t* index_scale, void* ws, const WsLayout& L,
                         hipStream_t st) {
  uint32_t* flags = ws_ptr<uint32_t>(ws, L.flags);
  const bool i8 = d.kv_dtype == SKV_KV_I8_ROWSCALE;
  if (d.n_kv_heads > kAppMaxHkv || d.n_kv_heads * d.rank > kAppThreads) return hipErrorInvalidValue;
  const AppendTarget tg{nullptr, nullptr, 0, 0, -1, 0};   // a full cache: row = position
  hipEvent_t ev0 = nullptr, ev1 = nullptr;
  const bool timed = timer_next(kTimerStream, &ev0, &ev1);   // diagnostic timer (sparsekv_timer_enable)
#define SKV_AP(DD, I8)                                                                           \
  do {                                                                                           \
    if (timed)                                                                                   \
      hipExtLaunchKernelGGL((append_kernel<DD, I8, false>), dim3(d.batch), dim3(kAppThreads), 0, st,    \
                            ev0, ev1, 0, ctx_len, (const __half*)k_new, (const __half*)v_new,    \
                            basis, (uint8_t*)kv.k, (uint8_t*)kv.v, (uint16_t*)kv.k_scale,        \
                            (uint16_t*)kv.v_scale, kv.rows, (uint8_t*)index_keys, index_scale,   \
                            d.n_kv_heads, d.rank, d.max_ctx, flags, tg);                         \
    else                                                                                         \
      hipLaunchKernelGGL((append_kernel<DD, I8, false>), dim3(d.batch), dim3(kAppThreads), 0, st,       \
                         ctx_len, (const __half*)k_new, (const __half*)v_new, basis,             \
                         (uint8_t*)kv.k, (uint8_t*)kv.v, (uint16_t*)kv.k_scale,                  \
                         (uint16_t*)kv.v_scale, kv.rows, (uint8_t*)index_keys, index_scale,      \
                         d.n_kv_heads, d.rank, d.max_ctx, flags, tg);                            \
  } while (0)
  if (d.head_dim == 256 && i8) SKV_AP(256, true);
  else if (d.head_dim == 256) SKV_AP(256, false);
  else if (d.head_dim == 128 && i8) SKV_AP(128, true);
  else if (d.head_dim == 128) SKV_AP(128, false);
  else return hipErrorInvalidValue;
#undef SKV_AP
  return hipGetLastError();
}

hipError_t launch_tier_append(const skv_layer_desc& d, int32_t* ctx_len, const void* k_new,
                              const void* v_new, const float* basis, const skv_kv_view& resident,
                              void* index_keys, uint16_t* index_scale, uint32_t* flags,
                              const AppendTarget& tg, hipStream_t st) {
  if (d.head_dim != 256 || d.kv_dtype != SKV_KV_I8_ROWSCALE || d.n_kv_heads > kAppMaxHkv ||
      d.n_kv_heads * d.rank > kAppThreads || !tg.tier_ctx || !tg.host)
    return hipErrorInvalidValue;
  hipEvent_t ev0 = nullptr, ev1 = nullptr;
  const bool timed = timer_next(kTimerStream, &ev0, &ev1);   // diagnostic timer (sparsekv_timer_enable)
  if (timed)
    hipExtLaunchKernelGGL((append_kernel<256, true, true>), dim3(d.batch), dim3(kAppThreads), 0, st, ev0,
                          ev1, 0, ctx_len, (const __half*)k_new, (const __half*)v_new, basis,
                          (uint8_t*)resident.k, (uint8_t*)resident.v, (uint16_t*)resident.k_scale,
                          (uint16_t*)resident.v_scale, resident.rows, (uint8_t*)index_keys,
                          index_scale, d.n_kv_heads, d.rank, d.max_ctx, flags, tg);
  else
    hipLaunchKernelGGL((append_kernel<256, true, true>), dim3(d.batch), dim3(kAppThreads), 0, st, ctx_len,
                       (const __half*)k_new, (const __half*)v_new, basis, (uint8_t*)resident.k,
                       (uint8_t*)resident.v, (uint16_t*)resident.k_scale,
                       (uint16_t*)resident.v_scale, resident.rows, (uint8_t*)index_keys,
                       index_scale, d.n_kv_heads, d.rank, d.max_ctx, flags, tg);
  return hipGetLastError();
}

}  // namespace skv
