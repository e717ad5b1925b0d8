// Internal declarations of the gfx950 sparse-KV library: workspace layout,
// small device helpers and the kernel launchers used by api.hip.
#pragma once

#include <hip/hip_runtime.h>
#include <hip/hip_fp16.h>
#include <stdint.h>
#include <stddef.h>

#include "../../include/sparsekv.h"

namespace skv {

// ---------------------------------------------------------------------------
// constants
// ---------------------------------------------------------------------------
constexpr int kHistBits = 12;                 // coarse-key histogram digit (1/8 octave)
constexpr int kHistBins = 1 << kHistBits;     // 4096 bins
constexpr int kListCap = 8192;                // candidates the select kernel holds in LDS
constexpr int kMaxTopk = 4096;                // largest budget
constexpr int kMaxSeg = 8192;                 // candidate segments per sequence
constexpr int kSegTok = 256;                  // candidates per segment, token mode (32 KB of sketch per wave)
constexpr int kSegBlk = 128;                  // candidates per segment, block mode (32 KB of keys per wave)
constexpr int kAttRowsPerWave = 32;           // selected rows per attention wave
constexpr int kMaxAttChunks = 256;            // attention partials per (sequence, KV head)
constexpr int kMaxQueries = 16;               // query tokens per sequence in one step (MFMA tile width)

// per-sequence select state written by the sample stage (u32 words)
struct TopkState {
  uint32_t beta;       // threshold bucket: candidates with digit >= beta are collected
  uint32_t pad[15];
};

// ---------------------------------------------------------------------------
// workspace layout (host and device agree through this struct)
// ---------------------------------------------------------------------------
struct WsLayout {
  size_t flags;        // uint32 flag word (+ padding)
  size_t state;        // [B] TopkState (sparsekv_topk path)
  size_t sproj;        // [B][H_kv*R] f32 unquantized query sketch
  size_t sdig;         // [B][sdig_stride] u16 sampled key digits
  size_t segcnt;       // [B][n_seg] u32 candidates found in each segment
  size_t cand;         // [B][n_seg*seg_items] Cand; also the fallback key buffer
  int n_seg;           // segments per sequence
  int seg_items;       // candidates per segment
  int n_samp;          // largest number of sampled lines per sequence
  int sdig_stride;     // u16 per sequence in sdig: room for every front workgroup's whole sample
  size_t att_ml;       // [B][H_kv][n_chunks][16][2] f32  (m, l) per head row
  size_t att_o;        // [B][H_kv][n_chunks][G][D] f32
  size_t total;
  int n_att_chunks;
};

inline size_t align_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

inline int select_capacity(const skv_layer_desc& d) {
  return d.index_mode == SKV_INDEX_SKETCH_INT4 ? d.n_sink + d.topk + d.n_tail : 4 * d.topk + 3;
}

// Waves per attention workgroup (one 32-row tile each): the largest of 8 and
// 4 that still gives at least 200 workgroups (about one per compute unit),
// else 2, so a small batch is spread over the GPU instead of a few CUs; more
// waves (up to 16) only where the capacity would need more than
// kMaxAttChunks chunks.  Two 8-wave workgroups per compute unit let one
// gather while the other merges, which 16-wave workgroups (one per compute
// unit) cannot.
inline int att_waves(const skv_layer_desc& d) {
  const int cap = select_capacity(d);
  auto chunks = [cap](int w) { return (cap + kAttRowsPerWave * w - 1) / (kAttRowsPerWave * w); };
  int w = 8;
  while (w > 2 && (int64_t)d.batch * d.n_kv_heads * chunks(w) < 200) w >>= 1;
  while (w < 16 && chunks(w) > kMaxAttChunks) w <<= 1;
  return w;
}
inline int att_rows_per_wg(const skv_layer_desc& d) { return kAttRowsPerWave * att_waves(d); }

inline int max_candidates(const skv_layer_desc& d) {
  return d.index_mode == SKV_INDEX_SKETCH_INT4 ? d.max_ctx : d.max_ctx / 4;
}

// Sample lines of a sequence, at most: every line when short, never more than
// 1024 lines (16K candidates).
inline int max_sample_lines(int nmax) {
  const int lines = (nmax + 15) / 16;
  return lines < 1024 ? (lines > 0 ? lines : 1) : 1024;
}

inline WsLayout ws_layout(const skv_layer_desc& d) {
  WsLayout w{};
  size_t off = 0;
  const size_t B = (size_t)d.batch;
  w.flags = off;  off = align_up(off + 256, 256);
  const int max_cand = max_candidates(d);
  w.seg_items = d.index_mode == SKV_INDEX_SKETCH_INT4 ? kSegTok : kSegBlk;
  w.n_seg = (max_cand + w.seg_items - 1) / w.seg_items;
  if (w.n_seg < 1) w.n_seg = 1;
  w.n_samp = max_sample_lines(max_cand);
  w.state = off;   off = align_up(off + B * sizeof(TopkState), 256);
  w.sproj = off;   off = align_up(off + B * (size_t)(d.n_kv_heads * (d.rank > 0 ? d.rank : 1)) * 4, 256);
  w.sdig_stride = (w.n_samp + 256) * 16;   // >= front workgroups x sample slots of each (<= 32 lines)
  w.sdig = off;    off = align_up(off + B * (size_t)w.sdig_stride * 2, 256);
  w.segcnt = off;  off = align_up(off + B * w.n_seg * 4, 256);
  w.cand = off;    off = align_up(off + B * (size_t)w.n_seg * w.seg_items * 16, 256);
  const int cap = select_capacity(d);
  w.n_att_chunks = (cap + att_rows_per_wg(d) - 1) / att_rows_per_wg(d);
  const int G = d.n_q_heads / d.n_kv_heads;
  w.att_ml = off; off = align_up(off + B * d.n_kv_heads * w.n_att_chunks * 16 * 2 * 4, 256);
  w.att_o = off;  off = align_up(off + B * d.n_kv_heads * w.n_att_chunks * (size_t)G * d.head_dim * 4, 256);
  w.total = off;
  return w;
}

template <typename T>
inline T* ws_ptr(void* ws, size_t off) { return reinterpret_cast<T*>(reinterpret_cast<char*>(ws) + off); }

// ---------------------------------------------------------------------------
// device helpers
// ---------------------------------------------------------------------------
__device__ __forceinline__ void raise_flag(uint32_t* flags, uint32_t bit) {
  atomicOr(flags, bit);
}

// Clamp a device-side context length into [0, max_ctx], flagging bad values.
__device__ __forceinline__ int clamp_ctx(const int32_t* ctx_len, int b, int max_ctx, uint32_t* flags) {
  int T = ctx_len[b];
  if (T < 0 || T > max_ctx) {
    if (flags) raise_flag(flags, SKV_FLAG_CTX_RANGE);
    T = T < 0 ? 0 : max_ctx;
  }
  return T;
}

// Order-preserving maps of floating point keys onto unsigned integers
// (larger key -> larger integer).  -0 must already be canonicalised to +0.
__device__ __forceinline__ uint64_t ordered_u64(double x) {
  uint64_t u = (uint64_t)__double_as_longlong(x);
  return (u & 0x8000000000000000ull) ? ~u : (u | 0x8000000000000000ull);
}
__device__ __forceinline__ uint32_t ordered_u32(float x) {
  uint32_t u = __float_as_uint(x);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}
// Histogram digit of an exact key: top kHistBits of the order-preserving image
// of the key rounded to fp32 (rounding is monotone, so digits are ordered).
__device__ __forceinline__ uint32_t key_digit(double x) {
  return ordered_u32(__double2float_rn(x)) >> (32 - kHistBits);
}

__device__ __forceinline__ float half_bits_to_float(uint16_t h) {
  return __half2float(__ushort_as_half(h));
}
__device__ __forceinline__ float bf16_bits_to_float(uint16_t h) {
  return __uint_as_float(((uint32_t)h) << 16);
}

// ---------------------------------------------------------------------------
// diagnostic kernel timer (sparsekv_timer_*): when it is enabled for the
// given kind, the kernel is launched with a start/stop event pair recorded by
// the dispatch itself (hipExtLaunchKernelGGL); otherwise both stay null
// ---------------------------------------------------------------------------
constexpr int kTimerStream = SKV_TIMER_STREAM;   // the call's streaming kernel
constexpr int kTimerAttend = SKV_TIMER_ATTEND;   // the attention kernel
bool timer_next(int kind, hipEvent_t* start, hipEvent_t* stop);
// units of the dense contractions (attention, multi-query score): SKV_PATH_MFMA
// or SKV_PATH_VALU (a measurement aid)
extern int g_contract_path;

// ---------------------------------------------------------------------------
// launchers (each returns hipSuccess or the launch error)
// ---------------------------------------------------------------------------
// query sketch, unquantized: sproj [B][H_kv*R] f32 in the workspace
hipError_t launch_qsketch_proj(const skv_layer_desc& d, const void* q, const float* basis,
                               void* ws, const WsLayout& L, hipStream_t st);
// query sketch: projection + quantization into qs int8 / qs_scale
hipError_t launch_qsketch(const skv_layer_desc& d, const void* q, const float* basis, int8_t* qs,
                          float* qs_scale, void* ws, const WsLayout& L, hipStream_t st);
// keys only
hipError_t launch_score(const skv_layer_desc& d, const int32_t* ctx_len, const void* iq,
                        const void* ik, const uint16_t* isc, double* keys, uint32_t* flags,
                        hipStream_t st);
// select from materialized keys: sample + collect + final
hipError_t launch_topk(const skv_layer_desc& d, const int32_t* ctx_len, const double* keys,
                       int32_t* idx, int32_t* n_sel, void* ws, const WsLayout& L, hipStream_t st);
// score and select without materializing keys: sample (from the index) +
// score/collect + final (which recomputes keys itself in the rare case the
// candidates are too few)
// sample + score/collect (score.hip); the final select is launched by launch_score_select.
// Token mode with qs_out != NULL: the query sketch is quantized from sproj in
// the workspace and written to qs_out / qscale_out; otherwise iq is the index
// query (int8 sketch or bf16 indexer query).
// Token mode with qs_out != NULL: the query sketch is computed from q and
// basis (written to qs_out / qscale_out) inside the front kernel.
hipError_t launch_sample_collect(const skv_layer_desc& d, const int32_t* ctx_len, const void* iq,
                                 const void* q, const float* basis, int8_t* qs_out, float* qscale_out,
                                 const void* ik, const uint16_t* isc, void* ws, const WsLayout& L,
                                 hipStream_t st);
hipError_t launch_score_select(const skv_layer_desc& d, const int32_t* ctx_len, const void* iq,
                               const void* q, const float* basis, int8_t* qs_out, float* qscale_out,
                               const void* ik, const uint16_t* isc, int32_t* idx, int32_t* n_sel,
                               void* ws, const WsLayout& L, hipStream_t st);
// d.batch counts virtual sequences: mq query tokens per sequence, whose K/V
// rows are those of sequence b / mq (mq = 1: the ordinary step)
hipError_t launch_attend(const skv_layer_desc& d, const void* q, const skv_kv_view& kv,
                         const int32_t* idx, const int32_t* n_sel, float sm_scale, float* out,
                         void* ws, const WsLayout& L, hipStream_t st, int mq = 1);
// multi-query step (token sketch): dv.batch = batch * mq virtual sequences.
// Sample + threshold + score/collect with all mq queries of a sequence per
// pass over its sketch (score.hip), then the per-query final select (topk.hip).
hipError_t launch_sample_collect_multi(const skv_layer_desc& dv, int mq, const int32_t* ctx_len,
                                       int8_t* qs_out, float* qscale_out, const void* ik,
                                       const uint16_t* isc, void* ws, const WsLayout& L,
                                       hipStream_t st);
// threshold digits of the dv.batch virtual sequences from the sampled digits
hipError_t launch_beta(const skv_layer_desc& dv, int mq, const int32_t* ctx_len, void* ws,
                       const WsLayout& L, hipStream_t st);
hipError_t launch_final_multi(const skv_layer_desc& dv, int mq, const int32_t* ctx_len,
                              const int8_t* qs, const void* ik, const uint16_t* isc, int32_t* idx,
                              int32_t* n_sel, void* ws, const WsLayout& L, hipStream_t st);
hipError_t launch_append_block(const skv_layer_desc& d, int32_t* ctx_len, const void* k_new,
                               const void* v_new, const void* raw_new, void* stage,
                               const skv_kv_view& kv, void* index_keys, void* ws, const WsLayout& L,
                               hipStream_t st);
// Where an append writes besides the key sketch: a full cache (ring_len < 0:
// row = position) or a host tier's resident tail ring and host records.
struct AppendTarget {
  int32_t* tier_ctx;   // per-sequence context of the tier (nullptr: no tier)
  uint8_t* host;       // device address of the host records (nullptr: none)
  int64_t host_ctx;    // positions per sequence in the host records
  int ring_base;       // first tail row
  int ring_len;        // tail rows (< 0: no ring; 0: no tail)
  int ring_anchor;     // position held by row ring_base (positions congruent mod ring_len)
};
hipError_t launch_tier_append(const skv_layer_desc& d, int32_t* ctx_len, const void* k_new,
                              const void* v_new, const float* basis, const skv_kv_view& resident,
                              void* index_keys, uint16_t* index_scale, uint32_t* flags,
                              const AppendTarget& tg, hipStream_t st);
hipError_t launch_append(const skv_layer_desc& d, int32_t* ctx_len, const void* k_new,
                         const void* v_new, const float* basis, const skv_kv_view& kv,
                         void* index_keys, uint16_t* index_scale, void* ws, const WsLayout& L,
                         hipStream_t st);

// sparse prefill attention over host-resident K/V (prefill.hip): workspace
// = flag word + per query head (max, sum) + accumulator; chunk tokens that a
// working buffer of chunk_bytes holds (K and V rows of fp16 / bf16)
size_t prefill_workspace_bytes(const skv_layer_desc& d, int n_query);
size_t prefill_chunk_tokens(const skv_layer_desc& d, size_t chunk_bytes);
hipError_t launch_prefill(const skv_layer_desc& d, int n_query, const void* q, const int32_t* idx,
                          const int32_t* n_sel, int cap, const void* host_k, const void* host_v,
                          int64_t n_tokens, void* chunk_buf, size_t chunk_bytes, float sm_scale,
                          float* out, void* ws, hipStream_t st);

}  // namespace skv
