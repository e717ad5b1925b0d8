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
//
// One workgroup per (KV head, sequence) projects that head into an fp32
// sketch in the workspace.  The quantization needs the whole sequence, so it
// runs in the next kernel: a small quantize kernel (sparsekv_qsketch) or the
// sample kernel of the fused select (sparsekv_step), both with the same
// device function.
#include "keys_common.h"

namespace skv {
namespace {

constexpr int kQuarters = 4;     // d is split in 4 quarters, loaded at once, summed in order

// basis is [H_kv][D][R]: for each d the R basis values of a head are
// contiguous, so a wavefront (64 consecutive r) reads 256 contiguous bytes per
// d.  Thread (quarter qt, r) loads and multiplies its D/4 values in one batch;
// the running sum then passes through the quarters in order, so the addition
// order is d = 0, 1, ..., D-1 exactly.
template <int DQ>   // D / 4
__global__ __launch_bounds__(1024) void qsketch_proj_kernel(
    const __half* __restrict__ q, const float* __restrict__ basis, float* __restrict__ sproj,
    int Hq, int Hkv, int R) {
#pragma clang fp contract(off)
  constexpr int D = 4 * DQ;
  __shared__ float qbar[D];
  __shared__ float sval[256];
  const int h = blockIdx.x, b = blockIdx.y;
  const int G = Hq / Hkv;

  // summed query of head h, query heads added in ascending order
  for (int i = threadIdx.x; i < D; i += blockDim.x) {
    const __half* qp = q + ((size_t)b * Hq + (size_t)h * G) * D + i;
    float v[16];
#pragma unroll
    for (int j = 0; j < 16; ++j) v[j] = __half2float(qp[(size_t)min(j, G - 1) * D]);  // unconditional
    float acc = v[0];
#pragma unroll
    for (int j = 1; j < 16; ++j)
      if (j < G) acc = acc + v[j];
    qbar[i] = acc;
  }
  for (int i = threadIdx.x; i < R; i += blockDim.x) sval[i] = 0.0f;
  __syncthreads();

  const int r = threadIdx.x % R, qt = threadIdx.x / R;   // blockDim.x == 4 * R
  float prod[DQ];
  {
    const float* bp = basis + ((size_t)h * D + (size_t)qt * DQ) * R + r;
    float bv[DQ];
#pragma unroll
    for (int j = 0; j < DQ; ++j) bv[j] = bp[(size_t)j * R];
    const float* qb = qbar + qt * DQ;
#pragma unroll
    for (int j = 0; j < DQ; ++j) prod[j] = qb[j] * bv[j];
  }
  for (int round = 0; round < kQuarters; ++round) {
    if (qt == round) {
      float s = sval[r];
#pragma unroll
      for (int j = 0; j < DQ; ++j) s = s + prod[j];
      sval[r] = s;
    }
    __syncthreads();
  }
  for (int i = threadIdx.x; i < R; i += blockDim.x) sproj[((size_t)b * Hkv + h) * R + i] = sval[i];
}

// one workgroup per sequence: codes and scale from the fp32 sketch
__global__ __launch_bounds__(256) void qsketch_quant_kernel(const float* __restrict__ sproj,
                                                            int8_t* __restrict__ qs,
                                                            float* __restrict__ qs_scale, int n) {
  __shared__ int8_t q8[512];
  __shared__ uint32_t red[16];
  const int b = blockIdx.x;
  const float scale = quantize_sketch(sproj + (size_t)b * n, n, q8, red);
  for (int i = threadIdx.x; i < n; i += blockDim.x) qs[(size_t)b * n + i] = q8[i];
  if (threadIdx.x == 0) qs_scale[b] = scale;
}

}  // namespace

hipError_t launch_qsketch_proj(const skv_layer_desc& d, const void* q, const float* basis,
                               void* ws, const WsLayout& L, hipStream_t st) {
  // validated on the host: rank a multiple of 16 in [16, 256], H_kv*R <= 512
  if (d.rank < 16 || d.rank > 256 || d.rank % 16 || d.n_kv_heads * d.rank > 512 ||
      d.n_q_heads / d.n_kv_heads > 16)
    return hipErrorInvalidValue;
  float* sproj = ws_ptr<float>(ws, L.sproj);
  const dim3 grid(d.n_kv_heads, d.batch), block(4 * d.rank);
  if (d.head_dim == 256)
    hipLaunchKernelGGL(qsketch_proj_kernel<64>, grid, block, 0, st, (const __half*)q, basis, sproj,
                       d.n_q_heads, d.n_kv_heads, d.rank);
  else if (d.head_dim == 128)
    hipLaunchKernelGGL(qsketch_proj_kernel<32>, grid, block, 0, st, (const __half*)q, basis, sproj,
                       d.n_q_heads, d.n_kv_heads, d.rank);
  else
    return hipErrorInvalidValue;
  return hipGetLastError();
}

hipError_t launch_qsketch(const skv_layer_desc& d, const void* q, const float* basis, int8_t* qs,
                          float* qs_scale, void* ws, const WsLayout& L, hipStream_t st) {
  hipError_t e = launch_qsketch_proj(d, q, basis, ws, L, st);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(qsketch_quant_kernel, dim3(d.batch), dim3(256), 0, st,
                     ws_ptr<const float>(ws, L.sproj), qs, qs_scale, d.n_kv_heads * d.rank);
  return hipGetLastError();
}

}  // namespace skv
