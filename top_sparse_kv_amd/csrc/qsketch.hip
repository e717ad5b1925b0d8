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

constexpr int kQsThreads = 256;

__global__ __launch_bounds__(kQsThreads) void qsketch_kernel(
    const __half* __restrict__ q, const float* __restrict__ basis, int8_t* __restrict__ qs,
    float* __restrict__ qs_scale, int Hq, int Hkv, int D, int R) {
#pragma clang fp contract(off)
  extern __shared__ float smem[];
  float* qbar = smem;              // [Hkv][D]
  float* sval = smem + Hkv * D;    // [Hkv*R]
  __shared__ float red[kQsThreads / 64];
  const int b = blockIdx.x;
  const int G = Hq / Hkv;
  const int n = Hkv * R;

  // summed query per KV head, heads added in ascending order
  for (int i = threadIdx.x; i < Hkv * D; i += blockDim.x) {
    const int h = i / D, dd = i % D;
    const __half* qp = q + ((size_t)b * Hq + (size_t)h * G) * D + dd;
    float acc = __half2float(qp[0]);
    for (int j = 1; j < G; ++j) acc = acc + __half2float(qp[(size_t)j * D]);
    qbar[i] = acc;
  }
  __syncthreads();

  // projection, d ascending, separately rounded multiply and add
  float amax = 0.0f;
  for (int i = threadIdx.x; i < n; i += blockDim.x) {
    const int h = i / R, r = i % R;
    const float* bp = basis + (size_t)h * D * R + r;
    const float* qb = qbar + h * D;
    float s = 0.0f;
    for (int dd = 0; dd < D; ++dd) {
      const float p = qb[dd] * bp[(size_t)dd * R];
      s = s + p;
    }
    sval[i] = s;
    amax = fmaxf(amax, fabsf(s));
  }
  // max over the workgroup (exact, order-free)
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
  hipLaunchKernelGGL(qsketch_kernel, dim3(d.batch), dim3(kQsThreads), lds, st,
                     (const __half*)q, basis, qs, qs_scale, d.n_q_heads, d.n_kv_heads, d.head_dim,
                     d.rank);
  return hipGetLastError();
}

}  // namespace skv
