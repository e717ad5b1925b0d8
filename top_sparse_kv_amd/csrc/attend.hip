// Stage A4: exact GQA attention over the selected K/V rows only.
//
// Page "8 agents x 250K context on two 3090s: sparse KV decode with a rank-64
// key sketch and a host-RAM tier", section "The mechanism": exact attention
// runs on the kept tokens only (int8 K/V there).  Page "3.14M Context on 3x
// 3090: The Power of an Architecture That Puts KV Cache in Host RAM", section
// "No Need to Rewrite the Kernel": the gather addresses row
// (token * n_kv_heads + kv_head) * head_dim, so K/V may live anywhere the
// GPU can address.
//
// Work split: one workgroup of W waves per (sequence, KV head, chunk of 32*W
// selected rows); each wave runs a softmax tile over 32 rows for the G query
// heads of that KV head.  W is the largest of 8, 4 that still gives about
// one workgroup per compute unit, else 2 (a 250K-token batch of 8 uses 8; a
// single 1M-token sequence uses 2, so its few thousand rows are gathered by
// many compute units rather than ten).  With 8 waves two workgroups share a
// compute unit, so one gathers while the other merges.  The waves merge in two LDS stages
// (wave w+W/2 into wave w, then the W/2 survivors), which bounds the LDS at
// (W/2)*G*(D+4) floats, and the workgroup writes one (max, sum, unnormalised
// output) partial; a second kernel merges the chunks of each query head in
// fixed order.
//
// Latency: a wave reads its row indices, n_sel and Q in one round trip, then
// issues every K, V and scale load of its tile in one batch (the per-row
// scales one per lane, handed to the lanes that need them by cross-lane
// reads), so the tile costs two dependent memory round trips.
//
// Inner step on the matrix cores (v_mfma_f32_16x16x32 f16 / bf16):
//   logits^T[32 tok x 16 heads] = K[32 x D] . Q^T[D x 16]   (2 M-tiles of 16)
//   O[16 heads x D]            += P[16 x 32 tok] . V[32 x D] (D/16 N-tiles)
// Only G of the 16 head columns are real (the rest multiply zeros).  The
// contraction index of an MFMA may be permuted freely as long as both operands
// agree, which is used twice:
//   * each lane reads one contiguous D/4 slice of a K row;
//   * the QK accumulator leaves, in every lane, the 8 token probabilities of
//     one head that the PV A-operand needs in that same lane (no shuffles);
//     V columns are gathered to match with byte permutes.
// int8 K/V are converted to fp16 exactly (offset-1152 trick: 0x64xx is 1024 +
// the biased byte).  Probabilities are split into a high and a low fp16 (or
// bf16) part and both are multiplied, so P keeps ~22 (or ~16) significant bits.
// All accumulation is fp32; the output is fp32.
#include "skv_internal.h"

#include <hip/hip_ext.h>

namespace skv {
namespace {

typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

enum { KV_I8 = 0, KV_F16 = 1, KV_BF16 = 2 };
constexpr float kLog2e = 1.4426950408889634f;

template <bool BF>
__device__ __forceinline__ f32x4 mfma(u32x4 a, u32x4 b, f32x4 c) {
  if constexpr (BF)
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                   __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
  else
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8, a),
                                                  __builtin_bit_cast(f16x8, b), c, 0, 0, 0);
}

// two int8 values (already xor 0x80 in their bytes) -> exact fp16 pair
__device__ __forceinline__ uint32_t i8pair_to_f16(uint32_t biased_dw, uint32_t sel) {
  const uint32_t r = __builtin_amdgcn_perm(0x64646464u, biased_dw, sel);
  f16x2 h = __builtin_bit_cast(f16x2, r);
  h = h - (f16x2){(_Float16)1152.0f, (_Float16)1152.0f};
  return __builtin_bit_cast(uint32_t, h);
}
// bytes 0..3 of a biased dword -> 4 fp16 (2 dwords)
__device__ __forceinline__ void i8x4_to_f16(uint32_t biased_dw, uint32_t& lo, uint32_t& hi) {
  lo = i8pair_to_f16(biased_dw, 0x04010400u);
  hi = i8pair_to_f16(biased_dw, 0x04030402u);
}

__device__ __forceinline__ uint16_t f32_to_bf16_rn(float x) {
  const uint32_t u = __float_as_uint(x);
  return (uint16_t)((u + 0x7FFFu + ((u >> 16) & 1u)) >> 16);
}

template <int KVT>
struct Esize {
  static constexpr int v = KVT == KV_I8 ? 1 : 2;
};

// ONE: the waves' partials merge in one stage (a slot per wave), else in two
// (half the slots); one stage when W slots of G rows fit the LDS budget
template <int KVT, int D, int WAVES, bool ONE>
__global__ __launch_bounds__(64 * WAVES) void attend_kernel(
    const void* __restrict__ qv, const uint8_t* __restrict__ kc, const uint8_t* __restrict__ vc,
    const uint16_t* __restrict__ ksc, const uint16_t* __restrict__ vsc, int64_t rows,
    const int32_t* __restrict__ idx, const int32_t* __restrict__ n_sel, int cap,
    float scale_log2, int Hq, int Hkv, float* __restrict__ part_ml, float* __restrict__ part_o,
    int n_chunks, uint32_t* __restrict__ flags, int mq, int n_keys) {
  constexpr bool BF = KVT == KV_BF16;
  constexpr int ES = Esize<KVT>::v;
  constexpr int KSTEPS = D / 32;          // MFMA k-steps over head_dim
  constexpr int NT = D / 16;              // PV N-tiles
  constexpr int KB = D / 4 * ES;          // bytes of one lane's K slice
  constexpr int VB = D / 16 * ES;         // bytes of one lane's V slice per token
  constexpr int KV4 = KB / 16;            // 16-byte loads per K slice
  constexpr int VV4 = VB / 16;            // 16-byte loads per V slice
  constexpr int NTH = 64 * WAVES;
  constexpr int HALF = WAVES / 2;
  constexpr int QP = D + 8;               // padded Q row (halves): conflict-free 16-byte reads
  constexpr int QPT = (16 * D / 2 + NTH - 1) / NTH;   // Q dwords per thread
  static_assert(kAttRowsPerWave == 32, "one 32-row tile per wave");
  __shared__ float s_m[WAVES][16];
  __shared__ float s_l[WAVES][16];
  __shared__ uint32_t s_q[16 * QP / 2];   // Q of the G heads, one row per head
  extern __shared__ float s_o[];          // [W or HALF][G][D + 4]

  // Workgroup -> (KV head h, chunk c, virtual sequence b).  Workgroups are
  // dealt to the 8 XCDs in turn (linear id mod 8), each XCD with its own L2.
  // One query per sequence: the H_kv heads of a (sequence, chunk) get ids
  // that land on one XCD.  Several: the mq queries of one (sequence, head,
  // chunk) do, so the rows they share (sinks, and the tail that moves by one
  // position per query) tend to be read from HBM once.
  int h, c, b;
  if (mq == 1) {
    // the H_kv heads of one (sequence, chunk) share an XCD: they read the same
    // row indices and the same row-scale sectors (scales of all heads of a
    // token are adjacent), which that XCD's L2 then serves once
    const int xcd = blockIdx.x & 7, s = blockIdx.x >> 3;
    const int key = (s / Hkv) * 8 + xcd;  // (sequence, chunk), chunk fastest
    if (key >= n_keys) return;            // padding of the last round; before any barrier
    h = s % Hkv;
    c = key % n_chunks;
    b = key / n_chunks;
  } else {
    const int xcd = blockIdx.x & 7, s = blockIdx.x >> 3;
    const int key = (s / mq) * 8 + xcd;   // (sequence, chunk, head), head fastest
    if (key >= n_keys) return;            // padding of the last round; before any barrier
    h = key % Hkv;
    c = (key / Hkv) % n_chunks;
    b = (key / Hkv / n_chunks) * mq + s % mq;
  }
  const int G = Hq / Hkv;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int i16 = lane & 15, g = lane >> 4;
  const int r0 = c * (kAttRowsPerWave * WAVES);
  const int rb = r0 + wave * kAttRowsPerWave;   // this wave's 32 selected rows
  const int32_t* ib = idx + (size_t)b * cap;
  // The row indices this lane uses are loaded together with n_sel and Q
  // (clamped into the array, masked by n below), saving dependent round trips:
  //   QK A operand: M-tile mt row i16 -> selected row rb + 16*mt + i16;
  //   P / V: e = 0..3 -> row rb + 4g + e, e = 4..7 -> row rb + 16 + 4g + e-4;
  //   scales: lane l loads the K (l < 32) or V (l >= 32) scale of row l % 32.
  int tk[2], tv[8];
#pragma unroll
  for (int mt = 0; mt < 2; ++mt) tk[mt] = ib[min(rb + 16 * mt + i16, cap - 1)];
#pragma unroll
  for (int e = 0; e < 8; ++e) tv[e] = ib[min(rb + (e < 4 ? 4 * g + e : 16 + 4 * g + (e - 4)), cap - 1)];
  const int ts = ib[min(rb + (lane & 31), cap - 1)];
  int n = n_sel[b];
  // the G query heads of this KV head pass through LDS (G*D/2 dwords)
  const int qdw = G * D / 2;
  uint32_t qd[QPT];
  {
    const uint32_t* qp = reinterpret_cast<const uint32_t*>(qv) + ((size_t)b * Hq + (size_t)h * G) * (D / 2);
#pragma unroll
    for (int u = 0; u < QPT; ++u) qd[u] = qp[min((int)threadIdx.x + u * NTH, qdw - 1)];
  }
  if (n < 0 || n > cap) {
    if (threadIdx.x == 0 && c == 0 && h == 0) raise_flag(flags, SKV_FLAG_INDEX_RANGE);
    n = n < 0 ? 0 : cap;
  }
  if (r0 >= n) return;
#pragma unroll
  for (int u = 0; u < QPT; ++u) {
    const int x = threadIdx.x + u * NTH;
    if (x < qdw) s_q[(x / (D / 2)) * (QP / 2) + x % (D / 2)] = qd[u];
  }
  __syncthreads();
  const size_t row_stride = (size_t)Hkv * D * ES;   // bytes between consecutive rows

  f32x4 o[NT];
  float m_run = -INFINITY;   // max of head i16 (log2 units), same in all 4 groups
  float l_run = 0.0f;

  // b is a virtual sequence (query b % mq of sequence b / mq): its rows are
  // those of sequence b / mq
  const size_t bk = (size_t)(b / mq);
  const uint8_t* kbase = kc + (bk * rows * Hkv + h) * D * ES;
  const uint8_t* vbase = vc + (bk * rows * Hkv + h) * D * ES;
  const uint16_t* ksb = ksc ? ksc + bk * rows * Hkv + h : nullptr;
  const uint16_t* vsb = vsc ? vsc + bk * rows * Hkv + h : nullptr;

  if (rb < n) {
    // out-of-range rows load row 0 and are masked through vok
    int ka[2];
#pragma unroll
    for (int mt = 0; mt < 2; ++mt) {
      const int ri = rb + 16 * mt + i16;
      const int tok = tk[mt];
      if (ri < n && (tok < 0 || (int64_t)tok >= rows)) raise_flag(flags, SKV_FLAG_INDEX_RANGE);
      ka[mt] = (ri < n && tok >= 0 && (int64_t)tok < rows) ? tok : 0;
    }
    int vt[8];
    bool vok[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const int ri = rb + (e < 4 ? 4 * g + e : 16 + 4 * g + (e - 4));
      const int tok = tv[e];
      const bool ok = ri < n && tok >= 0 && (int64_t)tok < rows;
      vt[e] = ok ? tok : 0;
      vok[e] = ok;
    }
    const int tsc = (rb + (lane & 31) < n && ts >= 0 && (int64_t)ts < rows) ? ts : 0;
    // ---- every load of the tile, issued back to back ----
    u32x4 kraw[2][KV4];
#pragma unroll
    for (int mt = 0; mt < 2; ++mt) {
      const u32x4* kp = reinterpret_cast<const u32x4*>(kbase + (size_t)ka[mt] * row_stride + g * KB);
#pragma unroll
      for (int x = 0; x < KV4; ++x) kraw[mt][x] = kp[x];
    }
    u32x4 vraw[8][VV4];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const u32x4* vp = reinterpret_cast<const u32x4*>(vbase + (size_t)vt[e] * row_stride + i16 * VB);
#pragma unroll
      for (int x = 0; x < VV4; ++x) vraw[e][x] = vp[x];
    }
    uint16_t sbits = 0;
    if constexpr (KVT == KV_I8) sbits = (lane < 32 ? ksb : vsb)[(size_t)tsc * Hkv];
    // 16-bit K/V do not fit in registers all at once: the compiler interleaves
    if constexpr (KVT == KV_I8) __builtin_amdgcn_sched_barrier(0);
    float kscale[8], vscale[8];
    if constexpr (KVT == KV_I8) {
      const float sc = half_bits_to_float(sbits);
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int row = e < 4 ? 4 * g + e : 16 + 4 * g + (e - 4);
        kscale[e] = __shfl(sc, row);
        vscale[e] = __shfl(sc, 32 + row);
      }
    } else {
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        kscale[e] = 1.0f;
        vscale[e] = 1.0f;
      }
    }

    // ---- logits (transposed): 2 M-tiles of 16 tokens x 16 heads ----
    // B operand: lane (head j = i16, group g), step s holds Q[j][g*D/4 + 8s .. +8]
    f32x4 sacc[2] = {(f32x4){0.f, 0.f, 0.f, 0.f}, (f32x4){0.f, 0.f, 0.f, 0.f}};
    const u32x4* qrow = reinterpret_cast<const u32x4*>(s_q + min(i16, G - 1) * (QP / 2) + g * (D / 8));
#pragma unroll
    for (int s = 0; s < KSTEPS; ++s) {
      const u32x4 bq = i16 < G ? qrow[s] : (u32x4){0u, 0u, 0u, 0u};
#pragma unroll
      for (int mt = 0; mt < 2; ++mt) {
        u32x4 a;
        if constexpr (KVT == KV_I8) {
          // step s uses bytes 8s..8s+7 of the lane's 64-byte slice
          const u32x4 w = kraw[mt][s >> 1];
          const uint32_t d0 = ((s & 1) ? w.z : w.x) ^ 0x80808080u;
          const uint32_t d1 = ((s & 1) ? w.w : w.y) ^ 0x80808080u;
          uint32_t a0, a1, a2, a3;
          i8x4_to_f16(d0, a0, a1);
          i8x4_to_f16(d1, a2, a3);
          a = (u32x4){a0, a1, a2, a3};
        } else {
          a = kraw[mt][s];
        }
        sacc[mt] = mfma<BF>(a, bq, sacc[mt]);
      }
    }
    // lane (head i16, group g) holds logits of rows 4g+e of each M-tile
    float lg[8];
    float tmax = -INFINITY;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const float sv = e < 4 ? sacc[0][e] : sacc[1][e - 4];
      lg[e] = vok[e] ? sv * kscale[e] * scale_log2 : -INFINITY;
      tmax = fmaxf(tmax, lg[e]);
    }
    tmax = fmaxf(tmax, __shfl_xor(tmax, 16));
    tmax = fmaxf(tmax, __shfl_xor(tmax, 32));
    float psum = 0.0f;
    float pv[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const float p = lg[e] == -INFINITY ? 0.0f : exp2f(lg[e] - tmax);
      psum += p;
      pv[e] = p * vscale[e];
    }
    psum += __shfl_xor(psum, 16);
    psum += __shfl_xor(psum, 32);
    l_run = psum;
    m_run = tmax;

    // P (A operand of PV): high and low parts
    u32x4 phi, plo;
    {
      uint32_t hw[4], lw[4];
#pragma unroll
      for (int pp = 0; pp < 4; ++pp) {
        const float x0 = pv[2 * pp], x1 = pv[2 * pp + 1];
        if constexpr (BF) {
          const uint16_t h0 = f32_to_bf16_rn(x0), h1 = f32_to_bf16_rn(x1);
          const float r0f = x0 - __uint_as_float((uint32_t)h0 << 16);
          const float r1f = x1 - __uint_as_float((uint32_t)h1 << 16);
          hw[pp] = (uint32_t)h0 | ((uint32_t)h1 << 16);
          lw[pp] = (uint32_t)f32_to_bf16_rn(r0f) | ((uint32_t)f32_to_bf16_rn(r1f) << 16);
        } else {
          const _Float16 h0 = (_Float16)x0, h1 = (_Float16)x1;
          const _Float16 l0 = (_Float16)(x0 - (float)h0), l1 = (_Float16)(x1 - (float)h1);
          hw[pp] = __builtin_bit_cast(uint32_t, (f16x2){h0, h1});
          lw[pp] = __builtin_bit_cast(uint32_t, (f16x2){l0, l1});
        }
      }
      phi = (u32x4){hw[0], hw[1], hw[2], hw[3]};
      plo = (u32x4){lw[0], lw[1], lw[2], lw[3]};
    }
    // ---- PV: N-tile t holds column d = i16*(D/16) + t ----
#pragma unroll
    for (int t = 0; t < NT; ++t) {
      uint32_t bw[4];
      if constexpr (KVT == KV_I8) {
        const int dw = t >> 2, by = t & 3;
        const uint32_t sel = (uint32_t)by | (0x0Cu << 8) | ((uint32_t)(4 + by) << 16) | (0x0Cu << 24);
#pragma unroll
        for (int pp = 0; pp < 4; ++pp) {
          const uint32_t x = __builtin_amdgcn_perm(vraw[2 * pp + 1][0][dw], vraw[2 * pp][0][dw], sel) ^ 0x64806480u;
          f16x2 hv = __builtin_bit_cast(f16x2, x);
          hv = hv - (f16x2){(_Float16)1152.0f, (_Float16)1152.0f};
          bw[pp] = __builtin_bit_cast(uint32_t, hv);
        }
      } else {
        // 16-bit elements: element t is half (t&1) of dword t>>1 of the slice
        const int dw = t >> 1;
        const uint32_t sel = (t & 1) ? 0x07060302u : 0x05040100u;
#pragma unroll
        for (int pp = 0; pp < 4; ++pp)
          bw[pp] = __builtin_amdgcn_perm(vraw[2 * pp + 1][dw >> 2][dw & 3], vraw[2 * pp][dw >> 2][dw & 3], sel);
      }
      const u32x4 bv = (u32x4){bw[0], bw[1], bw[2], bw[3]};
      o[t] = mfma<BF>(phi, bv, (f32x4){0.f, 0.f, 0.f, 0.f});
      o[t] = mfma<BF>(plo, bv, o[t]);
    }
  } else {
#pragma unroll
    for (int t = 0; t < NT; ++t) o[t] = (f32x4){0.f, 0.f, 0.f, 0.f};
  }

  // ---- merge the W waves of the workgroup in LDS ----
  // One stage (ONE), or two: wave w + HALF goes into wave w, then the HALF
  // survivors are combined.  A
  // slot holds G rows of D + 4 floats; lane (i16, g) owns columns
  // i16*(D/16) .. +D/16 of heads 4g .. 4g+3, stored as float4 runs.
  // Inside its run, lane i16 stores float4 u at position (u + i16/4) mod
  // (D/64): the 16 lanes of one store then hit 16 different 16-byte bank
  // groups instead of a handful (runs are 64 bytes apart).
  constexpr int DP = D + 4;
  constexpr int CPL = D / 16;   // columns per lane
  constexpr int NU = CPL / 4;   // float4 per lane and row (a power of two)
  static_assert((NU & (NU - 1)) == 0, "swizzle");
  auto slot_at = [&](int slot, int j, int u) -> f32x4* {
    return reinterpret_cast<f32x4*>(s_o + ((size_t)slot * G + j) * DP + i16 * CPL) + ((u + (i16 >> 2)) & (NU - 1));
  };
  // LDS offset (floats, inside a row) of column d under that swizzle
  auto col_of = [](int d) -> int {
    const int gi = d / CPL, w = d % CPL;
    return gi * CPL + 4 * (((w >> 2) + (gi >> 2)) & (NU - 1)) + (w & 3);
  };
  if constexpr (ONE) {
    if (g == 0) {
      s_m[wave][i16] = m_run;
      s_l[wave][i16] = l_run;
    }
    __syncthreads();
    // every wave rescales its accumulators to the workgroup's max of each
    // head and writes them to its own slot; the slots are summed in wave order
    float Mw = -INFINITY;
#pragma unroll
    for (int w = 0; w < WAVES; ++w) Mw = fmaxf(Mw, s_m[w][i16]);
    const float fw = m_run == -INFINITY ? 0.0f : exp2f(m_run - Mw);
    float f_row[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) f_row[e] = __shfl(fw, 4 * g + e);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int j = 4 * g + e;
      if (j < G) {
#pragma unroll
        for (int u = 0; u < NU; ++u)
          *slot_at(wave, j, u) = (f32x4){o[4 * u][e] * f_row[e], o[4 * u + 1][e] * f_row[e],
                                         o[4 * u + 2][e] * f_row[e], o[4 * u + 3][e] * f_row[e]};
      }
    }
    const size_t pbase = ((size_t)b * Hkv + h) * n_chunks + c;
    if (threadIdx.x < 16) {
      const int j = threadIdx.x;
      float M = -INFINITY;
#pragma unroll
      for (int w = 0; w < WAVES; ++w) M = fmaxf(M, s_m[w][j]);
      float Ls = 0.0f;
#pragma unroll
      for (int w = 0; w < WAVES; ++w)
        Ls += s_m[w][j] == -INFINITY ? 0.0f : s_l[w][j] * exp2f(s_m[w][j] - M);
      if (j < G) {
        part_ml[(pbase * 16 + j) * 2 + 0] = M;
        part_ml[(pbase * 16 + j) * 2 + 1] = Ls;
      }
    }
    __syncthreads();
    for (int x = threadIdx.x; x < G * D; x += blockDim.x) {
      const int j = x / D, d = x % D;
      float acc = 0.0f;
#pragma unroll
      for (int w = 0; w < WAVES; ++w) acc += s_o[((size_t)w * G + j) * DP + col_of(d)];
      part_o[(pbase * G + j) * D + d] = acc;
    }
    return;
  }
  if (g == 0) {
    s_m[wave][i16] = m_run;
    s_l[wave][i16] = l_run;
  }
  if (wave >= HALF) {
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int j = 4 * g + e;
      if (j < G) {
#pragma unroll
        for (int u = 0; u < NU; ++u)
          *slot_at(wave - HALF, j, u) = (f32x4){o[4 * u][e], o[4 * u + 1][e], o[4 * u + 2][e], o[4 * u + 3][e]};
      }
    }
  }
  __syncthreads();
  if (wave < HALF) {
    // wave w absorbs wave w + HALF: both rescaled to the larger max
    const float mp = s_m[wave + HALF][i16], lp = s_l[wave + HALF][i16];
    const float M = fmaxf(m_run, mp);
    const float aw = m_run == -INFINITY ? 0.0f : exp2f(m_run - M);
    const float ap = mp == -INFINITY ? 0.0f : exp2f(mp - M);
    float aw_row[4], ap_row[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      aw_row[e] = __shfl(aw, 4 * g + e);
      ap_row[e] = __shfl(ap, 4 * g + e);
    }
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int j = 4 * g + e;
      if (j < G) {
#pragma unroll
        for (int u = 0; u < NU; ++u) {
          const f32x4 x = *slot_at(wave, j, u);
#pragma unroll
          for (int q = 0; q < 4; ++q) o[4 * u + q][e] = o[4 * u + q][e] * aw_row[e] + x[q] * ap_row[e];
        }
      }
    }
    m_run = M;
    l_run = l_run * aw + lp * ap;
  }
  __syncthreads();
  if (wave < HALF) {
    if (g == 0) {
      s_m[wave][i16] = m_run;
      s_l[wave][i16] = l_run;
    }
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int j = 4 * g + e;
      if (j < G) {
#pragma unroll
        for (int u = 0; u < NU; ++u)
          *slot_at(wave, j, u) = (f32x4){o[4 * u][e], o[4 * u + 1][e], o[4 * u + 2][e], o[4 * u + 3][e]};
      }
    }
  }
  __syncthreads();
  // per query head: the workgroup's max and sum, and each slot's factor
  const size_t pbase = ((size_t)b * Hkv + h) * n_chunks + c;
  if (threadIdx.x < 16) {
    const int j = threadIdx.x;
    float M = -INFINITY;
#pragma unroll
    for (int w = 0; w < HALF; ++w) M = fmaxf(M, s_m[w][j]);
    float Ls = 0.0f;
#pragma unroll
    for (int w = 0; w < HALF; ++w) {
      const float f = s_m[w][j] == -INFINITY ? 0.0f : exp2f(s_m[w][j] - M);
      s_l[HALF + w][j] = f;   // rows HALF.. of s_l are free now
      Ls += s_l[w][j] * f;
    }
    if (j < G) {
      part_ml[(pbase * 16 + j) * 2 + 0] = M;
      part_ml[(pbase * 16 + j) * 2 + 1] = Ls;
    }
  }
  __syncthreads();
  for (int x = threadIdx.x; x < G * D; x += blockDim.x) {
    const int j = x / D, d = x % D;
    float acc = 0.0f;
#pragma unroll
    for (int w = 0; w < HALF; ++w) acc += s_o[((size_t)w * G + j) * DP + col_of(d)] * s_l[HALF + w][j];
    part_o[(pbase * G + j) * D + d] = acc;
  }
}

// ---- the same attention on the vector ALUs (a measurement aid) ------------
// Same workgroups, rows and partials as attend_kernel<KV_I8, D, 8, ·> with one
// query per sequence, but both contractions are fp32 dot products on the
// vector ALUs: for the logits lane l holds row l%32 of its wave's 32 and the
// query heads [h0, h0 + ceil(G/2)) of half l/32, reading its K row 16 bytes at
// a time against Q in LDS; for P.V lane l owns D/64 columns and reads them
// from the 32 V rows (one row = 64 lanes x D/64 bytes, contiguous), with the
// row-scaled probabilities from LDS.  The waves merge in LDS as in the
// one-stage path.  Exists to measure what the matrix cores bring.
constexpr int kValuWaves = 8;
template <int D>
__global__ __launch_bounds__(64 * kValuWaves) void attend_valu_kernel(
    const __half* __restrict__ qv, const int8_t* __restrict__ kc, const int8_t* __restrict__ vc,
    const uint16_t* __restrict__ ksc, const uint16_t* __restrict__ vsc, int64_t rows,
    const int32_t* __restrict__ idx, const int32_t* __restrict__ n_sel, int cap, float scale_log2,
    int Hq, int Hkv, float* __restrict__ part_ml, float* __restrict__ part_o, int n_chunks,
    uint32_t* __restrict__ flags, int n_keys) {
  constexpr int W = kValuWaves;
  constexpr int GM = 16;          // query heads per KV head, at most
  constexpr int GH = GM / 2;      // heads per half-wave in the logits
  constexpr int CPL = D / 64;     // P.V columns per lane
  // LDS (dynamic, sized by the launch): the waves' output slots [W][G][D] (Q
  // [G][D] in their first part until the logits are done), the row-scaled
  // probabilities [W][G][32], and each wave's max, sum and merge factor [W][G]
  extern __shared__ float s_o[];
  // workgroup -> (KV head h, chunk c, sequence b), as attend_kernel with one query
  const int xcd = blockIdx.x & 7, sg = blockIdx.x >> 3;
  const int key = (sg / Hkv) * 8 + xcd;
  if (key >= n_keys) return;   // before any barrier
  const int h = sg % Hkv, c = key % n_chunks, b = key / n_chunks;
  const int G = Hq / Hkv;
  float* s_p = s_o + W * G * D;
  float* s_m = s_p + W * G * 32;
  float* s_l = s_m + W * G;
  float* s_f = s_l + W * G;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  int n = n_sel[b];
  if (n < 0 || n > cap) {
    if (threadIdx.x == 0 && c == 0 && h == 0) raise_flag(flags, SKV_FLAG_INDEX_RANGE);
    n = n < 0 ? 0 : cap;
  }
  const int r0 = c * 32 * W;
  if (r0 >= n) return;
  float* s_q = s_o;
  for (int x = threadIdx.x; x < G * D; x += blockDim.x)
    s_q[x] = __half2float(qv[((size_t)b * Hq + (size_t)h * G) * D + x]);
  __syncthreads();
  // ---- logits of this lane's row for its half of the heads ----
  const int r = lane & 31, hh = lane >> 5;
  const int ri = r0 + wave * 32 + r;
  const int tok = ri < n ? idx[(size_t)b * cap + ri] : -1;
  const bool ok = ri < n && tok >= 0 && (int64_t)tok < rows;
  if (ri < n && !ok) raise_flag(flags, SKV_FLAG_INDEX_RANGE);
  const int t = ok ? tok : 0;
  const size_t kb = ((size_t)b * rows + t) * Hkv + h;
  const int j0 = hh * ((G + 1) / 2), j1 = min(G, j0 + (G + 1) / 2);
  float acc[GH];
#pragma unroll
  for (int jj = 0; jj < GH; ++jj) acc[jj] = 0.0f;
  const int8_t* krow = kc + kb * D;
  for (int d0 = 0; d0 < D; d0 += 16) {
    const int4 w = *reinterpret_cast<const int4*>(krow + d0);
    const int wd[4] = {w.x, w.y, w.z, w.w};
    float kf[16];
#pragma unroll
    for (int e = 0; e < 16; ++e) kf[e] = (float)(int8_t)((wd[e >> 2] >> (8 * (e & 3))) & 0xFF);
#pragma unroll
    for (int jj = 0; jj < GH; ++jj) {
      const int j = j0 + jj;
      if (j < j1) {
        const float* qp = s_q + j * D + d0;
#pragma unroll
        for (int e = 0; e < 16; ++e) acc[jj] += qp[e] * kf[e];
      }
    }
  }
  const float ks = half_bits_to_float(ksc[kb]);
  const float vs = half_bits_to_float(vsc[kb]);
#pragma unroll
  for (int jj = 0; jj < GH; ++jj) {
    const int j = j0 + jj;
    const float lg = ok ? acc[jj] * ks * scale_log2 : -INFINITY;
    float m = lg;
    for (int o = 16; o > 0; o >>= 1) m = fmaxf(m, __shfl_xor(m, o));   // over the 32 rows
    const float p = lg == -INFINITY ? 0.0f : exp2f(lg - m);
    float sum = p;
    for (int o = 16; o > 0; o >>= 1) sum += __shfl_xor(sum, o);
    if (j < j1) {
      s_p[(wave * G + j) * 32 + r] = p * vs;
      if (r == 0) {
        s_m[wave * G + j] = m;
        s_l[wave * G + j] = sum;
      }
    }
  }
  __syncthreads();   // s_p complete; Q no longer read (s_o reused below)
  // ---- P.V: lane owns columns lane*CPL .. +CPL ----
  float o[GM][CPL];
#pragma unroll
  for (int j = 0; j < GM; ++j)
#pragma unroll
    for (int e = 0; e < CPL; ++e) o[j][e] = 0.0f;
  uint32_t vw[32];
#pragma unroll
  for (int rr = 0; rr < 32; ++rr) {
    const int tr = __shfl(t, rr);   // lanes 0..31 hold the rows' tokens
    const int8_t* vp = vc + (((size_t)b * rows + tr) * Hkv + h) * D + lane * CPL;
    vw[rr] = CPL == 4 ? *reinterpret_cast<const uint32_t*>(vp) : (uint32_t)*reinterpret_cast<const uint16_t*>(vp);
  }
#pragma unroll
  for (int rr = 0; rr < 32; ++rr) {
    float vf[CPL];
#pragma unroll
    for (int e = 0; e < CPL; ++e) vf[e] = (float)(int8_t)((vw[rr] >> (8 * e)) & 0xFF);
#pragma unroll
    for (int j = 0; j < GM; ++j) {
      if (j < G) {
        const float pj = s_p[(wave * G + j) * 32 + rr];
#pragma unroll
        for (int e = 0; e < CPL; ++e) o[j][e] += pj * vf[e];
      }
    }
  }
  // ---- merge the waves: each wave's slot, then the sum in wave order ----
#pragma unroll
  for (int j = 0; j < GM; ++j)
    if (j < G)
#pragma unroll
      for (int e = 0; e < CPL; ++e) s_o[((size_t)wave * G + j) * D + lane * CPL + e] = o[j][e];
  __syncthreads();
  const size_t pbase = ((size_t)b * Hkv + h) * n_chunks + c;
  if ((int)threadIdx.x < G) {
    const int j = threadIdx.x;
    float M = -INFINITY;
#pragma unroll
    for (int w = 0; w < W; ++w) M = fmaxf(M, s_m[w * G + j]);
    float Ls = 0.0f;
#pragma unroll
    for (int w = 0; w < W; ++w) {
      const float f = s_m[w * G + j] == -INFINITY ? 0.0f : exp2f(s_m[w * G + j] - M);
      s_f[w * G + j] = f;
      Ls += s_l[w * G + j] * f;
    }
    part_ml[(pbase * 16 + j) * 2 + 0] = M;
    part_ml[(pbase * 16 + j) * 2 + 1] = Ls;
  }
  __syncthreads();
  for (int x = threadIdx.x; x < G * D; x += blockDim.x) {
    const int j = x / D, d = x % D;
    float a = 0.0f;
#pragma unroll
    for (int w = 0; w < W; ++w) a += s_o[((size_t)w * G + j) * D + d] * s_f[w * G + j];
    part_o[(pbase * G + j) * D + d] = a;
  }
}

// merge the chunks of each (sequence, query head) in ascending chunk order
constexpr int kMaxChunks = kMaxAttChunks;   // one thread per chunk

// Thread d owns output column d (D <= 256); the partials of the first MB
// chunks are loaded together with the (max, sum) pairs, before the factors
// are known, so a merge of up to MB chunks costs one round trip plus the
// reductions (MB = 16, or 32 past 16 chunks: one sequence's 2,051 rows in
// 2-wave chunks make 33).  Chunks at or past the selection's end are not
// written in this call: they are skipped by a select, not multiplied by a
// zero factor.
template <int MB>
__global__ __launch_bounds__(256) void attend_merge_kernel(
    const float* __restrict__ part_ml, const float* __restrict__ part_o,
    const int32_t* __restrict__ n_sel, int cap, int Hq, int Hkv, int D, int n_chunks,
    int rows_per_chunk, float* __restrict__ out) {
  __shared__ float s_f[kMaxChunks + MB];
  __shared__ float s_red[2][4];
  const int jq = blockIdx.x, b = blockIdx.y;
  const int G = Hq / Hkv;
  const int h = jq / G, j = jq % G;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  int n = n_sel[b];
  n = n < 0 ? 0 : (n > cap ? cap : n);
  const int nc = min((n + rows_per_chunk - 1) / rows_per_chunk, n_chunks);
  const size_t pb = ((size_t)b * Hkv + h) * n_chunks;
  const int d = min((int)threadIdx.x, D - 1);
  const float* po = part_o + (pb * G + j) * D + d;   // chunk cc at po[cc * G * D]
  const size_t cstride = (size_t)G * D;
  float v[MB];
#pragma unroll
  for (int u = 0; u < MB; ++u) v[u] = po[(size_t)min(u, n_chunks - 1) * cstride];   // unconditional
  const int c = threadIdx.x;   // one chunk per thread (n_chunks <= kMaxChunks)
  const float m = part_ml[((pb + min(c, n_chunks - 1)) * 16 + j) * 2];
  const float l = part_ml[((pb + min(c, n_chunks - 1)) * 16 + j) * 2 + 1];
  const bool live = c < nc && m != -INFINITY;
  float M = live ? m : -INFINITY;
  for (int off = 32; off > 0; off >>= 1) M = fmaxf(M, __shfl_xor(M, off));
  if (lane == 0) s_red[0][wave] = M;
  __syncthreads();
  M = fmaxf(fmaxf(s_red[0][0], s_red[0][1]), fmaxf(s_red[0][2], s_red[0][3]));
  const float f = live ? exp2f(m - M) : 0.0f;
  float Ls = live ? l * f : 0.0f;
  for (int off = 32; off > 0; off >>= 1) Ls += __shfl_xor(Ls, off);
  if (lane == 0) s_red[1][wave] = Ls;
  s_f[c] = f;
  __syncthreads();
  Ls = (s_red[1][0] + s_red[1][1]) + (s_red[1][2] + s_red[1][3]);
  const float inv = Ls > 0.0f ? 1.0f / Ls : 0.0f;
  // chunks in ascending order
  float acc = 0.0f;
#pragma unroll
  for (int u = 0; u < MB; ++u) acc += u < nc ? v[u] * s_f[u] : 0.0f;
  for (int cc = MB; cc < nc; cc += MB) {
#pragma unroll
    for (int u = 0; u < MB; ++u) v[u] = po[(size_t)min(cc + u, nc - 1) * cstride];
#pragma unroll
    for (int u = 0; u < MB; ++u) acc += cc + u < nc ? v[u] * s_f[cc + u] : 0.0f;
  }
  if ((int)threadIdx.x < D) out[((size_t)b * Hq + jq) * D + threadIdx.x] = acc * inv;
}

}  // namespace

int g_contract_path = SKV_PATH_MFMA;

hipError_t launch_attend(const skv_layer_desc& d, const void* q, const skv_kv_view& kv,
                         const int32_t* idx, const int32_t* n_sel, float sm_scale, float* out,
                         void* ws, const WsLayout& Lw, hipStream_t st, int mq) {
  uint32_t* flags = ws_ptr<uint32_t>(ws, Lw.flags);
  float* part_ml = ws_ptr<float>(ws, Lw.att_ml);
  float* part_o = ws_ptr<float>(ws, Lw.att_o);
  const int cap = select_capacity(d);
  const int G = d.n_q_heads / d.n_kv_heads;
  if (Lw.n_att_chunks > kMaxChunks) return hipErrorInvalidValue;
  // one workgroup per (sequence, chunk, head) and query, a 1-D grid padded to
  // whole rounds of 8 keys: one query, keys (sequence, chunk) with the H_kv
  // heads of a key on one XCD; several queries, keys (sequence, chunk, head)
  // with the mq queries of a key on one XCD
  const int n_keys = mq == 1 ? d.batch * Lw.n_att_chunks
                             : d.batch / mq * Lw.n_att_chunks * d.n_kv_heads;
  const dim3 grid = mq == 1 ? dim3((unsigned)(((n_keys + 7) / 8) * 8 * d.n_kv_heads))
                            : dim3((unsigned)(((n_keys + 7) / 8) * 8 * mq));
  const int waves = att_waves(d);
  // one-stage merge when a slot per wave stays within 52 KB of LDS (two
  // workgroups per compute unit with the static arrays)
  const size_t lds1 = (size_t)waves * G * (d.head_dim + 4) * sizeof(float);
  const bool one = lds1 <= 52 * 1024;
  const size_t lds = one ? lds1 : lds1 / 2;
  const float sl = sm_scale * kLog2e;
  hipEvent_t ev0 = nullptr, ev1 = nullptr;
  const bool timed = timer_next(kTimerAttend, &ev0, &ev1);   // diagnostic timer
#define SKV_AT_ARGS                                                                                \
  q, (const uint8_t*)kv.k, (const uint8_t*)kv.v, kv.k_scale, kv.v_scale, kv.rows, idx, n_sel, cap,  \
      sl, d.n_q_heads, d.n_kv_heads, part_ml, part_o, Lw.n_att_chunks, flags, mq, n_keys
#define SKV_AT_O(KVT, DD, WV, ON)                                                                   \
  do {                                                                                             \
    if (timed)                                                                                     \
      hipExtLaunchKernelGGL((attend_kernel<KVT, DD, WV, ON>), grid, dim3(64 * WV), lds, st, ev0,   \
                            ev1, 0, SKV_AT_ARGS);                                                  \
    else                                                                                           \
      hipLaunchKernelGGL((attend_kernel<KVT, DD, WV, ON>), grid, dim3(64 * WV), lds, st,           \
                         SKV_AT_ARGS);                                                             \
  } while (0)
#define SKV_AT(KVT, DD, WV)                                                                        \
  do {                                                                                             \
    if (one) SKV_AT_O(KVT, DD, WV, true);                                                          \
    else SKV_AT_O(KVT, DD, WV, false);                                                             \
  } while (0)
#define SKV_AT_W(KVT, DD)                                                                          \
  do {                                                                                             \
    if (waves == 16) SKV_AT(KVT, DD, 16);                                                          \
    else if (waves == 8) SKV_AT(KVT, DD, 8);                                                       \
    else if (waves == 4) SKV_AT(KVT, DD, 4);                                                       \
    else SKV_AT(KVT, DD, 2);                                                                       \
  } while (0)
  const int kvt = d.kv_dtype == SKV_KV_I8_ROWSCALE ? KV_I8 : (d.kv_dtype == SKV_KV_F16 ? KV_F16 : KV_BF16);
  // LDS of the vector-ALU kernel: output slots, probabilities, max / sum / factor
  const size_t lv = (size_t)kValuWaves * G * (d.head_dim + 32 + 3) * sizeof(float);
  const bool valu = g_contract_path == SKV_PATH_VALU && kvt == KV_I8 && mq == 1 && waves == kValuWaves &&
                    (d.head_dim == 256 || d.head_dim == 128) && lv <= 64 * 1024;
  if (valu) {
    // the vector-ALU kernel (measurement aid): same grid, partials and merge
#define SKV_AV(DD)                                                                                 \
  do {                                                                                             \
    if (timed)                                                                                     \
      hipExtLaunchKernelGGL((attend_valu_kernel<DD>), grid, dim3(64 * kValuWaves), lv, st, ev0, ev1, 0, \
                            (const __half*)q, (const int8_t*)kv.k, (const int8_t*)kv.v, kv.k_scale,  \
                            kv.v_scale, kv.rows, idx, n_sel, cap, sl, d.n_q_heads, d.n_kv_heads,     \
                            part_ml, part_o, Lw.n_att_chunks, flags, n_keys);                        \
    else                                                                                           \
      hipLaunchKernelGGL((attend_valu_kernel<DD>), grid, dim3(64 * kValuWaves), lv, st,            \
                         (const __half*)q, (const int8_t*)kv.k, (const int8_t*)kv.v, kv.k_scale,     \
                         kv.v_scale, kv.rows, idx, n_sel, cap, sl, d.n_q_heads, d.n_kv_heads,        \
                         part_ml, part_o, Lw.n_att_chunks, flags, n_keys);                           \
  } while (0)
    if (d.head_dim == 256) SKV_AV(256);
    else SKV_AV(128);
#undef SKV_AV
  } else if (kvt == KV_I8 && d.head_dim == 256) SKV_AT_W(KV_I8, 256);
  else if (kvt == KV_I8 && d.head_dim == 128) SKV_AT_W(KV_I8, 128);
  else if (kvt == KV_F16 && d.head_dim == 256) SKV_AT_W(KV_F16, 256);
  else if (kvt == KV_F16 && d.head_dim == 128) SKV_AT_W(KV_F16, 128);
  else if (kvt == KV_BF16 && d.head_dim == 256) SKV_AT_W(KV_BF16, 256);
  else if (kvt == KV_BF16 && d.head_dim == 128) SKV_AT_W(KV_BF16, 128);
  else return hipErrorInvalidValue;
#undef SKV_AT_W
#undef SKV_AT
#undef SKV_AT_O
#undef SKV_AT_ARGS
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  if (Lw.n_att_chunks <= 16)
    hipLaunchKernelGGL(attend_merge_kernel<16>, dim3(d.n_q_heads, d.batch), dim3(256), 0, st, part_ml,
                       part_o, n_sel, cap, d.n_q_heads, d.n_kv_heads, d.head_dim, Lw.n_att_chunks,
                       att_rows_per_wg(d), out);
  else
    hipLaunchKernelGGL(attend_merge_kernel<32>, dim3(d.n_q_heads, d.batch), dim3(256), 0, st, part_ml,
                       part_o, n_sel, cap, d.n_q_heads, d.n_kv_heads, d.head_dim, Lw.n_att_chunks,
                       att_rows_per_wg(d), out);
  return hipGetLastError();
}

}  // namespace skv
