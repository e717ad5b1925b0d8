// Stage A1: the int8 query sketch of each sequence.
//
// Page "8 agents x 250K context on two 3090s: sparse KV decode with a rank-64
// key sketch and a host-RAM tier", section "The mechanism": tokens are scored
// through a rank-64 projection onto a frozen basis, and one pick per layer is
// shared by all KV heads.  Scoring is linear in the query, so the G query heads
// of a KV head are summed first; the summed query is projected onto that
// head's basis, and the H_kv*R sketch values of a sequence are quantized to
// int8 with one scale (max|s|/127, round half to even, clamp to +-127).
//
// The int8 codes are a decision taken on floating point values, so the
// evaluation order is fixed and every operation is a separately rounded fp32
// operation (no fused multiply-add): the codes are reproducible bit for bit.
// Plain operators are used under `fp contract(off)` (library helpers such as
// __fmul_rn can still be fused once inlined), and the two quotients are
// computed in fp64 and rounded once to fp32, which equals the correctly
// rounded fp32 quotient because 53 >= 2*24 + 2.
#include "skv_internal.h"

namespace skv {
namespace {

constexpr int kQsThreads = 1024;
constexpr int kQuarters = 4;     // d is split in 4 quarters, loaded at once, summed in order

// basis is [H_kv][D][R]: for each d the R basis values of a head are
// contiguous, so a wavefront (64 consecutive r) reads 256 contiguous bytes per
// d.  Thread (quarter q, pair p = (h, r)) loads and multiplies its D/4 values
// in one batch; the running sum then passes through the quarters in order, so
// the addition order is d = 0, 1, ..., D-1 exactly.
template <int DQ>   // D / 4
__global__ __launch_bounds__(kQsThreads) void qsketch_kernel(
    const __half* __restrict__ q, const float* __restrict__ basis, int8_t* __restrict__ qs,
    float* __restrict__ qs_scale, int Hq, int Hkv, int R) {
#pragma clang fp contract(off)
  constexpr int D = 4 * DQ;
  extern __shared__ float smem[];
  float* qbar = smem;              // [Hkv][D]
  float* sval = smem + Hkv * D;    // [Hkv*R] running sums, then final values
  __shared__ float red[kQsThreads / 64];
  const int b = blockIdx.x;
  const int G = Hq / Hkv;
  const int n = Hkv * R;           // <= 256

  // summed query per KV head, heads added in ascending order
  for (int i = threadIdx.x; i < Hkv * D; i += blockDim.x) {
    const int h = i / D, dd = i % D;
    const __half* qp = q + ((size_t)b * Hq + (size_t)h * G) * D + dd;
    float v[16];
#pragma unroll
    for (int j = 0; j < 16; ++j) v[j] = __half2float(qp[(size_t)min(j, G - 1) * D]);  // unconditional
    float acc = v[0];
#pragma unroll
    for (int j = 1; j < 16; ++j)
      if (j < G) acc = acc + v[j];
    qbar[i] = acc;
  }
  for (int i = threadIdx.x; i < n; i += blockDim.x) sval[i] = 0.0f;
  __syncthreads();

  const int p = threadIdx.x % n, qt = threadIdx.x / n;
  const bool active = threadIdx.x < kQuarters * n;
  float prod[DQ];
  if (active) {
    const int h = p / R, r = p % R;
    const float* bp = basis + ((size_t)h * D + (size_t)qt * DQ) * R + r;
    float bv[DQ];
#pragma unroll
    for (int j = 0; j < DQ; ++j) bv[j] = bp[(size_t)j * R];
    const float* qb = qbar + h * D + qt * DQ;
#pragma unroll
    for (int j = 0; j < DQ; ++j) prod[j] = qb[j] * bv[j];
  }
  for (int round = 0; round < kQuarters; ++round) {
    if (active && qt == round) {
      float s = sval[p];
#pragma unroll
      for (int j = 0; j < DQ; ++j) s = s + prod[j];
      sval[p] = s;
    }
    __syncthreads();
  }
  // max |s| over the sketch (exact, order-free)
  float amax = 0.0f;
  for (int i = threadIdx.x; i < n; i += blockDim.x) amax = fmaxf(amax, fabsf(sval[i]));
  for (int off = 32; off > 0; off >>= 1) amax = fmaxf(amax, __shfl_xor(amax, off));
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = amax;
  __syncthreads();
  amax = red[0];
  for (int w = 1; w < (int)(blockDim.x >> 6); ++w) amax = fmaxf(amax, red[w]);

  const float scale = amax == 0.0f ? 0.0f : (float)((double)amax / 127.0);
  for (int i = threadIdx.x; i < n; i += blockDim.x) {
    int code = 0;
    if (amax != 0.0f) {
      float r = rintf((float)((double)sval[i] / (double)scale));
      r = fminf(fmaxf(r, -127.0f), 127.0f);
      code = (int)r;
    }
    qs[(size_t)b * n + i] = (int8_t)code;
  }
  if (threadIdx.x == 0) qs_scale[b] = scale;
}

}  // namespace

hipError_t launch_qsketch(const skv_layer_desc& d, const void* q, const float* basis, int8_t* qs,
                          float* qs_scale, hipStream_t st) {
  const size_t lds = (size_t)(d.n_kv_heads * d.head_dim + d.n_kv_heads * d.rank) * sizeof(float);
  if (d.n_kv_heads * d.rank > 256 || d.n_q_heads / d.n_kv_heads > 16) return hipErrorInvalidValue;
  if (d.head_dim == 256)
    hipLaunchKernelGGL(qsketch_kernel<64>, dim3(d.batch), dim3(kQsThreads), lds, st,
                       (const __half*)q, basis, qs, qs_scale, d.n_q_heads, d.n_kv_heads, d.rank);
  else if (d.head_dim == 128)
    hipLaunchKernelGGL(qsketch_kernel<32>, dim3(d.batch), dim3(kQsThreads), lds, st,
                       (const __half*)q, basis, qs, qs_scale, d.n_q_heads, d.n_kv_heads, d.rank);
  else
    return hipErrorInvalidValue;
  return hipGetLastError();
}

}  // namespace skv
