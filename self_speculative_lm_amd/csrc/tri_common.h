// Internal declarations shared by the gfx950 kernels and the runtime of
// libtrimode.so.  Not part of the public C-ABI (see include/trimode.h).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "trimode.h"

namespace tri {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint16_t bf16_t;  // raw bfloat16 storage

__device__ __forceinline__ float bf16_to_f32(bf16_t b) {
  return __uint_as_float(static_cast<uint32_t>(b) << 16);
}

// Round-to-nearest-even float32 -> bfloat16 (NaN kept quiet).
__device__ __forceinline__ bf16_t f32_to_bf16(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return static_cast<bf16_t>((u >> 16) | 0x40u);
  u += 0x7fffu + ((u >> 16) & 1u);
  return static_cast<bf16_t>(u >> 16);
}

// Element access for the two storage types.  store4 writes four consecutive
// elements (i % 4 == 0) with one vector store.
template <typename T> struct Elem;
template <> struct Elem<float> {
  __device__ static float load(const float* p, size_t i) { return p[i]; }
  __device__ static void store(float* p, size_t i, float v) { p[i] = v; }
  __device__ static void store4(float* p, size_t i, f32x4 v) { *reinterpret_cast<f32x4*>(p + i) = v; }
};
template <> struct Elem<bf16_t> {
  __device__ static float load(const bf16_t* p, size_t i) { return bf16_to_f32(p[i]); }
  __device__ static void store(bf16_t* p, size_t i, float v) { p[i] = f32_to_bf16(v); }
  __device__ static void store4(bf16_t* p, size_t i, f32x4 v) {
    const uint32_t lo = (uint32_t)f32_to_bf16(v[0]) | ((uint32_t)f32_to_bf16(v[1]) << 16);
    const uint32_t hi = (uint32_t)f32_to_bf16(v[2]) | ((uint32_t)f32_to_bf16(v[3]) << 16);
    *reinterpret_cast<uint2*>(p + i) = make_uint2(lo, hi);
  }
};

// Wave-wide all-reduce without an LDS round trip: DPP inside 16-lane rows
// (lane ^ 1, lane ^ 2, then the half-row and row mirrors), then
// v_permlane16_swap and v_permlane32_swap, which exchange the odd 16-lane rows
// (the upper 32 lanes) of one register with the even rows (the lower 32
// lanes) of another; fed the same value twice, the two results of lane l are
// x[l] and x[l ^ 16] (x[l ^ 32]).  Every step combines a lane with a partner
// holding the same operands, so all 64 lanes end with the same bits, in an
// order fixed by the lane layout.
template <typename Op>
__device__ __forceinline__ uint32_t wave_allreduce_u32(uint32_t x, Op op) {
  x = op(x, (uint32_t)__builtin_amdgcn_update_dpp((int)x, (int)x, 0xB1, 0xF, 0xF, false));   // quad_perm [1,0,3,2]
  x = op(x, (uint32_t)__builtin_amdgcn_update_dpp((int)x, (int)x, 0x4E, 0xF, 0xF, false));   // quad_perm [2,3,0,1]
  x = op(x, (uint32_t)__builtin_amdgcn_update_dpp((int)x, (int)x, 0x141, 0xF, 0xF, false));  // row_half_mirror
  x = op(x, (uint32_t)__builtin_amdgcn_update_dpp((int)x, (int)x, 0x140, 0xF, 0xF, false));  // row_mirror
  auto r = __builtin_amdgcn_permlane16_swap(x, x, false, false);
  x = op(r[0], r[1]);
  r = __builtin_amdgcn_permlane32_swap(x, x, false, false);
  return op(r[0], r[1]);
}
__device__ __forceinline__ int wave_max_i32(int x) {
  return (int)wave_allreduce_u32((uint32_t)x, [](uint32_t a, uint32_t b) { return (uint32_t)max((int)a, (int)b); });
}
__device__ __forceinline__ int wave_min_i32(int x) {
  return (int)wave_allreduce_u32((uint32_t)x, [](uint32_t a, uint32_t b) { return (uint32_t)min((int)a, (int)b); });
}
__device__ __forceinline__ float wave_sum_f32(float x) {
  return __uint_as_float(wave_allreduce_u32(__float_as_uint(x), [](uint32_t a, uint32_t b) {
    return __float_as_uint(__uint_as_float(a) + __uint_as_float(b));
  }));
}

// V element as the bf16 attention multiplies it: rounded to bf16 (the cache's
// storage precision), then converted to fp16 with saturation at +-65504.  A
// V cache kept in this form spares every attention workgroup that reads a
// tile the conversion, with the same bits.  `sat` is set when the bf16 value
// lies outside the fp16 range (the saturation changed it).
__device__ __forceinline__ bf16_t v_cache_f16(float v, bool& sat) {
  const float b = bf16_to_f32(f32_to_bf16(v));
  sat = sat || fabsf(b) > 65504.f;
  const _Float16 h = (_Float16)fminf(fmaxf(b, -65504.f), 65504.f);
  return __builtin_bit_cast(bf16_t, h);
}

// RMSNorm statistic in one fixed order.  The row is cut into chunks of 16
// columns: a chunk's sum of squares is ((q0 + q1) + (q2 + q3)) over its four
// groups of four consecutive columns, each group fmaf(v3, v3, fmaf(v2, v2,
// fmaf(v1, v1, v0 * v0))).  The row total is then reduced by one wave: lane
// i adds chunks i, i + 64, ..., i + 448 in that order (zero past the row's
// chunks, so at most 512 chunks: d <= 8192), and the lanes are summed by
// wave_sum_f32.
constexpr int ROW_CHUNK_STRIDES = 8;
__device__ __forceinline__ float sumsq4(f32x4 v) {
  return fmaf(v[3], v[3], fmaf(v[2], v[2], fmaf(v[1], v[1], v[0] * v[0])));
}
__device__ __forceinline__ float row_total(const float* part, int nch) {
  const int lane = threadIdx.x & 63;
  float acc = 0.f;
#pragma unroll
  for (int j = 0; j < ROW_CHUNK_STRIDES; ++j) {
    const int i = lane + 64 * j;
    const float v = i < nch ? part[i] : 0.f;
    acc = j == 0 ? v : acc + v;
  }
  return wave_sum_f32(acc);
}
__device__ __forceinline__ float rms_inv(float total, int d, float eps) {
  return 1.0f / sqrtf(total / (float)d + eps);
}

// ---------------------------------------------------------------- launchers
// Each returns hipSuccess or the launch error.  All are asynchronous.

// Y partial slots: P[s][m][n] (float32), s < S, for Y = X W^T where the rows of
// W are the concatenation of up to three segments (each [rows][K]).
struct WSeg {
  const void* ptr;
  int rows;
};
struct GemmPlan {
  int S;          // K splits (partial slots)
  int Ks;         // K per split (bf16: a multiple of the 256-wide stage; K padded to S*Ks)
  int nch = 1;    // bf16: stages per straight-line pass (divides Ks / 256)
  int depth = 4;  // bf16: W fragments in flight per wave
};
// unsplit: one K split whatever the shape (the lm_head writes logits directly).
GemmPlan gemm_plan(int N, int K, int dtype, bool unsplit = false);
// Bytes of a packed weight matrix for a plan (bf16: step-major MFMA fragments,
// rows padded to 128, K padded to S*Ks; float32: row-major) and the packing
// launch (segments concatenated by rows).
size_t gemm_packed_bytes(const GemmPlan& p, int N, int K, int dtype);
// Packed row order: PACK_PLAIN keeps the segments' rows; PACK_GATEUP
// interleaves two equal segments in groups of 16 rows (gate/up pairs).
enum { PACK_PLAIN = 0, PACK_GATEUP = 1 };
hipError_t launch_pack(int dtype, const WSeg* segs, int nseg, int N, int K, const GemmPlan& p, void* dst,
                       int order, hipStream_t st);
// Y = X W^T with W packed by launch_pack.
// Output slots a launch_gemm of M rows writes (the consumer adds them in slot
// order): the plan's S on the decode kernel, fewer on the large-M kernel
// unless `invariant`.  With `invariant` every row's outputs are bit-identical
// whatever M is (one slot per K split on both kernels).
int gemm_out_slots(int dtype, const GemmPlan& p, int M, int N, int K, bool invariant);
// Whether the gate/up projection of M rows can apply SwiGLU in its epilogue
// (large-M kernel, one slot): launch_gemm(..., swiglu_out = h) then writes
// h = bf16(silu(gate) * up) [M][N/2] instead of float32 slots, bit-identical
// to the slots followed by the SwiGLU kernel.
bool gemm_swiglu_fused(int dtype, const GemmPlan& p, int M, int N, int K, bool invariant);
// One past the highest packed W element launch_gemm's kernel reads (host
// evaluation of the kernels' address arithmetic over the launch grid).
size_t gemm_w_reach(int dtype, const GemmPlan& p, int M, int N, int K, bool invariant);
hipError_t launch_gemm(int dtype, const void* X, int M, int K, const void* W, int N, const GemmPlan& plan,
                       float* P, size_t slot_stride, bool invariant, hipStream_t st, void* swiglu_out = nullptr);

struct AttnLaunch {
  const void* q;
  const void* kc;
  const void* vc;
  const int32_t* seq_start;
  const int32_t* slot_seq;  // cache sequence of each slot (NULL = identity)
  const int32_t* row_hi;
  int n_seq, rows, max_rows_per_seq, max_hi;
  int hq, hkv, hd, ctx;
  float scale;
  int kv_split;
  void* out;
  float* part;  // split partials
  bool v_f16 = false;  // bf16: the V cache holds the fp16 form written by launch_rope_kv(v_f16)
  // Quadratic-speculation blocks: a row with row_blk[r] >= 0 also attends to
  // the blk_len keys of rows [row_blk[r], row_blk[r] + blk_len) of the row
  // scratch (k_scr, v_scr [rows][hkv][hd], written by launch_rope_kv), after
  // the cache keys [0, row_hi[r]).  NULL: no block rows.
  const int32_t* row_blk = nullptr;
  const void* k_scr = nullptr;
  const void* v_scr = nullptr;
  int blk_len = 0;
  // Compacted grid from attn_work_table (NULL: the regular grid).
  const int32_t* work = nullptr;
  int nwork = 0;
};
int attn_pick_split(int max_ctx, int n_seq, int hq, int hkv);
int attn_pick_split_launch(int max_hi, int n_seq, int rows_per_seq, int hq, int hkv);
size_t attn_ws_bytes(int rows, int hq, int hd, int max_hi, int kv_split);
// Entries of the compacted attention grid of a forward whose slots start at
// seq_start[0..n_slots] (host); 0 = launch the regular grid.
int attn_work_table(const int32_t* seq_start, int n_slots, int hq, int hkv, int max_hi, int32_t* out, int cap);
// Query vectors per query group of an attention launch (launch_attn's shape).
int attn_group_vectors(int max_rows_per_seq, int G, int max_hi);
hipError_t launch_attn(int dtype, const AttnLaunch& a, hipStream_t st);

// Misc kernels.
hipError_t launch_embed(int dtype, const int32_t* tok, int rows, const void* E, int n_emb, int d,
                        float* x, hipStream_t st);
hipError_t launch_resid_norm(int dtype, float* x, const float* P, int nslots, size_t slot_stride,
                             int rows, int d, const float* g, float eps, void* y, hipStream_t st);
// vsat: set to 1 when a V value saturates its fp16 form (v_f16).  row_blk
// (optional, device int32 [rows]): rows with row_blk[r] >= 0 belong to a
// quadratic-speculation block and write k, v to kscr / vscr [rows][hkv][hd]
// (model storage type) instead of the cache.
hipError_t launch_rope_kv(int dtype, const float* P, int nslots, size_t slot_stride, int rows,
                          int hq, int hkv, int hd, const int32_t* row_seq, const int32_t* row_pos,
                          const float* rope, void* qout, void* kc, void* vc, int ctx,
                          size_t cache_seq_stride, hipStream_t st, bool v_f16 = false, int32_t* vsat = nullptr,
                          const int32_t* row_blk = nullptr, void* kscr = nullptr, void* vscr = nullptr);
hipError_t launch_swiglu(int dtype, const float* P, int nslots, size_t slot_stride, int rows,
                         int ffn, void* h, hipStream_t st);
hipError_t launch_lora_mid(int dtype, const float* P, int nslots, size_t slot_stride, int rows,
                           int r, const int32_t* row_lora, void* mid, hipStream_t st);
hipError_t launch_zero_f32(float* p, size_t n, hipStream_t st);
size_t vocab_ws_bytes(int rows, int vocab);
hipError_t launch_scatter_gather(const int32_t* src, const int32_t* sidx, const int32_t* didx, int n,
                                 int32_t* dst, hipStream_t st);
hipError_t launch_sample_commit(const float* logits, int rows, int vocab, const int32_t* row_kind,
                                const int32_t* block_start, int n_blocks, float threshold,
                                int32_t* out_tok, float* out_conf, int32_t* out_commit,
                                int32_t* out_status, void* ws, hipStream_t st);
hipError_t launch_verify_accept(const int32_t* draft, const int32_t* ar_tok, int batch, int k,
                                int32_t* accept_len, int32_t* committed, int32_t* kv_len,
                                hipStream_t st);

}  // namespace tri
