// Stage A2: exact ranking keys for every candidate of every sequence.
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
// Both kernels are pure HBM streams: the sketch (130 B/token at H_kv*R = 256)
// or the pooled keys (256 B/block) are read once, contiguously, with 16-byte
// loads spread over the lanes of a token so each wavefront load covers 1 KB
// of consecutive memory; several tokens per lane are in flight at once.
#include "skv_internal.h"

namespace skv {
namespace {

constexpr int kScoreThreads = 256;
constexpr int kScoreUnroll = 8;

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

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

// Sum over aligned groups of LPT lanes (LPT in {2,4,8,16}) with DPP moves:
// two quad permutes, then the half-row and row mirrors.  Every lane of the
// group ends with the group total.
template <int LPT>
__device__ __forceinline__ int group_sum_i32(int v) {
  v += __builtin_amdgcn_update_dpp(0, v, 0xB1, 0xF, 0xF, false);       // quad_perm [1,0,3,2]
  if (LPT >= 4) v += __builtin_amdgcn_update_dpp(0, v, 0x4E, 0xF, 0xF, false);   // [2,3,0,1]
  if (LPT >= 8) v += __builtin_amdgcn_update_dpp(0, v, 0x141, 0xF, 0xF, false);  // row_half_mirror
  if (LPT >= 16) v += __builtin_amdgcn_update_dpp(0, v, 0x140, 0xF, 0xF, false); // row_mirror
  return v;
}

template <int CTRL>
__device__ __forceinline__ double dpp_add_f64(double v) {
  const long long u = __double_as_longlong(v);
  const int lo = __builtin_amdgcn_update_dpp(0, (int)(u & 0xFFFFFFFF), CTRL, 0xF, 0xF, false);
  const int hi = __builtin_amdgcn_update_dpp(0, (int)(u >> 32), CTRL, 0xF, 0xF, false);
  return v + __longlong_as_double(((long long)hi << 32) | (unsigned)lo);
}

template <int LPB>
__device__ __forceinline__ double group_sum_f64(double x) {
  x = dpp_add_f64<0xB1>(x);
  if (LPB >= 4) x = dpp_add_f64<0x4E>(x);
  if (LPB >= 8) x = dpp_add_f64<0x141>(x);
  if (LPB >= 16) x = dpp_add_f64<0x140>(x);
  if (LPB >= 32) x += __shfl_xor(x, 16);
  return x;
}

template <int LPT>  // lanes per token; a token's sketch is 16*LPT bytes
__global__ __launch_bounds__(kScoreThreads) void score_sketch_kernel(
    const int8_t* __restrict__ qs, const uint8_t* __restrict__ codes,
    const uint16_t* __restrict__ scale, const int32_t* __restrict__ ctx_len,
    double* __restrict__ keys, uint32_t* __restrict__ flags, int max_ctx, int S, int L,
    int chunk) {
  constexpr int TB = 16 * LPT;
  constexpr int TPW = 64 / LPT;
  constexpr int STEP = (kScoreThreads / 64) * TPW;
  const int b = blockIdx.y;
  const int T = clamp_ctx(ctx_len, b, max_ctx, blockIdx.x == 0 ? flags : nullptr);
  const int lo = S;
  const int hi = T - L > S ? T - L : S;
  const int t0 = lo + blockIdx.x * chunk;
  if (t0 >= hi) return;
  const int t1 = min(hi, t0 + chunk);
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int sub = lane % LPT, tw = lane / LPT;

  // this lane's 32 query codes: even code positions of each 8-code word in
  // qe, odd ones in qo (matching the low / high nibbles of the code bytes)
  const uint8_t* qp = reinterpret_cast<const uint8_t*>(qs) + (size_t)b * (2 * TB) + 32 * sub;
  uint32_t qe[4], qo[4];
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

  const uint8_t* cbase = codes + (size_t)b * max_ctx * TB + 16 * sub;
  const uint16_t* sbase = scale + (size_t)b * max_ctx;
  double* kbase = keys + (size_t)b * max_ctx;
  for (int base = t0 + wave * TPW + tw; base < t1; base += STEP * kScoreUnroll) {
    u32x4 w[kScoreUnroll];
    uint16_t sc[kScoreUnroll];
    // all loads issued unconditionally (past the end they re-read the last
    // token; those results are dropped), so they are in flight together
#pragma unroll
    for (int u = 0; u < kScoreUnroll; ++u) {
      const int t = min(base + u * STEP, t1 - 1);
      w[u] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(cbase + (size_t)t * TB));
      sc[u] = sbase[t];   // the token's scale, fetched with its codes
    }
#pragma unroll
    for (int u = 0; u < kScoreUnroll; ++u) {
      const int t = base + u * STEP;
      const int acc = group_sum_i32<LPT>(dot32_i4(w[u], qe, qo, 0));
      if (sub == 0 && t < t1) {
        const double key = (double)(acc >> 4) * (double)half_bits_to_float(sc[u]) + 0.0;  // -0 -> +0
        kbase[t] = key;
      }
    }
  }
}

template <int LPB>  // lanes per pooled key; index_dim = 8*LPB bf16
__global__ __launch_bounds__(kScoreThreads) void score_pooled_kernel(
    const uint16_t* __restrict__ qi, const uint16_t* __restrict__ kp,
    const int32_t* __restrict__ ctx_len, double* __restrict__ keys, uint32_t* __restrict__ flags,
    int max_ctx, int chunk) {
  constexpr int ID = 8 * LPB;
  constexpr int BPW = 64 / LPB;
  constexpr int STEP = (kScoreThreads / 64) * BPW;
  const int b = blockIdx.y;
  const int T = clamp_ctx(ctx_len, b, max_ctx, blockIdx.x == 0 ? flags : nullptr);
  const int nb = T / 4;
  const int nbmax = max_ctx / 4;
  const int j0 = blockIdx.x * chunk;
  if (j0 >= nb) return;
  const int j1 = min(nb, j0 + chunk);
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int sub = lane % LPB, tw = lane / LPB;
  double qd[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) qd[e] = (double)bf16_bits_to_float(qi[(size_t)b * ID + 8 * sub + e]);
  const uint16_t* kb = kp + (size_t)b * nbmax * ID + 8 * sub;
  double* kout = keys + (size_t)b * nbmax;
  for (int base = j0 + wave * BPW + tw; base < j1; base += STEP * kScoreUnroll) {
    u32x4 w[kScoreUnroll];
#pragma unroll
    for (int u = 0; u < kScoreUnroll; ++u) {
      const int j = min(base + u * STEP, j1 - 1);
      w[u] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(kb + (size_t)j * ID));
    }
#pragma unroll
    for (int u = 0; u < kScoreUnroll; ++u) {
      const int j = base + u * STEP;
      const uint32_t ws[4] = {w[u].x, w[u].y, w[u].z, w[u].w};
      double acc = 0.0;
#pragma unroll
      for (int m = 0; m < 4; ++m) {
        acc = fma((double)__uint_as_float(ws[m] << 16), qd[2 * m], acc);
        acc = fma((double)__uint_as_float(ws[m] & 0xFFFF0000u), qd[2 * m + 1], acc);
      }
      acc = group_sum_f64<LPB>(acc);
      if (sub == 0 && j < j1) kout[j] = acc + 0.0;   // -0 -> +0
    }
  }
}

}  // namespace

hipError_t launch_score(const skv_layer_desc& d, const int32_t* ctx_len, const void* iq,
                        const void* ik, const uint16_t* isc, double* keys, uint32_t* flags,
                        hipStream_t st) {
  if (d.index_mode == SKV_INDEX_SKETCH_INT4) {
    const int tb = d.n_kv_heads * d.rank / 2;
    const int nchunk = (d.max_ctx + kScoreChunk - 1) / kScoreChunk;
    const dim3 grid(nchunk > 0 ? nchunk : 1, d.batch);
#define SKV_SK(LPT)                                                                        \
  hipLaunchKernelGGL(score_sketch_kernel<LPT>, grid, dim3(kScoreThreads), 0, st,           \
                     (const int8_t*)iq, (const uint8_t*)ik, isc, ctx_len, keys, flags,     \
                     d.max_ctx, d.n_sink, d.n_tail, kScoreChunk)
    switch (tb) {
      case 32: SKV_SK(2); break;
      case 64: SKV_SK(4); break;
      case 128: SKV_SK(8); break;
      case 256: SKV_SK(16); break;
      default: return hipErrorInvalidValue;
    }
#undef SKV_SK
  } else {
    const int nbmax = d.max_ctx / 4;
    const int nchunk = (nbmax + kPooledChunk - 1) / kPooledChunk;
    const dim3 grid(nchunk > 0 ? nchunk : 1, d.batch);
#define SKV_PK(LPB)                                                                         \
  hipLaunchKernelGGL(score_pooled_kernel<LPB>, grid, dim3(kScoreThreads), 0, st,            \
                     (const uint16_t*)iq, (const uint16_t*)ik, ctx_len, keys, flags,        \
                     d.max_ctx, kPooledChunk)
    switch (d.index_dim) {
      case 64: SKV_PK(8); break;
      case 128: SKV_PK(16); break;
      case 256: SKV_PK(32); break;
      default: return hipErrorInvalidValue;
    }
#undef SKV_PK
  }
  return hipGetLastError();
}

}  // namespace skv
