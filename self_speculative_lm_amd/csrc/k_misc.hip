// Row-wise kernels of the decode forward and the sampling/acceptance kernels.
//
// Every row-wise reduction here runs in a fixed order that depends only on the
// row's own data and the shape, so a row's result does not depend on which
// other rows share the launch.
#include <math.h>

#include <algorithm>
#include <type_traits>

#include "tri_common.h"

namespace tri {
namespace {

constexpr int MAX_SLOTS = 17;  // split-K partial slots a consumer adds (<= 16 GEMM splits + a LoRA slot)

// Sum of the partial slots at offset `off` (slot order).  All slot loads are
// issued before the first add so their latencies overlap.
__device__ __forceinline__ float slot_sum(const float* P, int nslots, size_t stride, size_t off) {
  float v[MAX_SLOTS];
#pragma unroll
  for (int s = 0; s < MAX_SLOTS; ++s) v[s] = s < nslots ? P[s * stride + off] : 0.f;
  float acc = v[0];
#pragma unroll
  for (int s = 1; s < MAX_SLOTS; ++s)
    if (s < nslots) acc += v[s];
  return acc;
}

// Four consecutive columns (off % 4 == 0, stride % 4 == 0) with the slot
// count known at compile time: every load is issued
// unconditionally before the first add, so the sum costs one memory round
// trip.  (A runtime count compiles to one branch per slot, and the join
// after each branch made the compiler wait for the loads already issued:
// two round trips instead of one.)  Same additions in the same order as
// slot_sum.
template <int NS>
__device__ __forceinline__ f32x4 slot_sum4n(const float* P, size_t stride, size_t off) {
  static_assert(NS >= 1 && NS <= MAX_SLOTS, "slot count");
  f32x4 v[NS];
#pragma unroll
  for (int s = 0; s < NS; ++s) v[s] = *reinterpret_cast<const f32x4*>(P + s * stride + off);
  f32x4 acc = v[0];
#pragma unroll
  for (int s = 1; s < NS; ++s) acc += v[s];
  return acc;
}

// x[r] = E[tok[r]]; an id outside [0, n_emb) (e.g. the -1 the sampler writes
// for a row with non-finite logits) gives a zero row instead of a stray read.
// Four columns per thread (d % 4 == 0), all of a row's loads issued at once.
template <typename T>
__global__ __launch_bounds__(1024) void embed_kernel(const int32_t* tok, const T* E, int n_emb, int d, float* x) {
  const int r = blockIdx.x;
  const int t = tok[r];
  const bool ok = t >= 0 && t < n_emb;
  const T* src = E + (size_t)(ok ? t : 0) * d;
  for (int c = 4 * (int)threadIdx.x; c < d; c += 4 * (int)blockDim.x) {
    f32x4 v = {0.f, 0.f, 0.f, 0.f};
    if (ok) {
      if constexpr (sizeof(T) == 2) {
        const uint2 u = *reinterpret_cast<const uint2*>(src + c);
        v = f32x4{bf16_to_f32((bf16_t)(u.x & 0xffff)), bf16_to_f32((bf16_t)(u.x >> 16)),
                  bf16_to_f32((bf16_t)(u.y & 0xffff)), bf16_to_f32((bf16_t)(u.y >> 16))};
      } else {
        v = *reinterpret_cast<const f32x4*>(src + c);
      }
    }
    *reinterpret_cast<f32x4*>(x + (size_t)r * d + c) = v;
  }
}

// x[r] += sum of slots; y[r] = x[r] / sqrt(mean(x[r]^2) + eps) * g   (RMSNorm).
// One workgroup per row, VPT groups of four columns per thread (the
// launcher sizes the workgroup so that every group lies in the row, except
// for the last workgroup rounding).  Every load of the row (x, g, the NS
// slots of each group) is issued before the first use, at a clamped address
// for a group past the row, and x is written back with y at the end, so the
// kernel makes one memory round trip.  The mean square is taken in a fixed
// order (16-column chunks, then one wave over the chunks: sumsq4 / row_total).
constexpr int NORM_CHUNKS = 512;  // 16-column chunks: d <= 8192
template <typename T, int NS, int VPT>
__global__ __launch_bounds__(VPT == 1 ? 1024 : (VPT == 2 ? 640 : 512)) void resid_norm_kernel(
    float* __restrict__ x, const float* __restrict__ P, size_t stride, int d, const float* __restrict__ g,
    float eps, T* __restrict__ y) {
  __shared__ float chunk[NORM_CHUNKS];
  __shared__ float tot_s;
  const int r = blockIdx.x, tid = threadIdx.x, nt = blockDim.x;
  float* xr = x + (size_t)r * d;
  f32x4 v[VPT], gv[VPT];
#pragma unroll
  for (int i = 0; i < VPT; ++i) {
    const int c = min((tid + i * nt) * 4, d - 4);
    gv[i] = *reinterpret_cast<const f32x4*>(g + c);
    v[i] = *reinterpret_cast<const f32x4*>(xr + c);
    if constexpr (NS > 0) v[i] += slot_sum4n<NS>(P, stride, (size_t)r * d + c);
  }
#pragma unroll
  for (int i = 0; i < VPT; ++i) {
    const int c = (tid + i * nt) * 4;
    if (c >= d) v[i] = f32x4{0.f, 0.f, 0.f, 0.f};
    float q = sumsq4(v[i]);
    q += __shfl_xor(q, 1);
    q += __shfl_xor(q, 2);
    if ((tid & 3) == 0 && c < d) chunk[c / 16] = q;
  }
  __syncthreads();
  if (tid < 64) {
    const float t = row_total(chunk, d / 16);
    if (tid == 0) tot_s = t;
  }
  __syncthreads();
  const float inv = rms_inv(tot_s, d, eps);
#pragma unroll
  for (int i = 0; i < VPT; ++i) {
    const int c = (tid + i * nt) * 4;
    if (c < d) {
      Elem<T>::store4(y, (size_t)r * d + c, v[i] * inv * gv[i]);
      if constexpr (NS > 0) *reinterpret_cast<f32x4*>(xr + c) = v[i];
    }
  }
}

// Sum the QKV slots, rotate q and k (rotate-half pairs (i, i + hd/2) by
// pos * base^(-2i/hd), cos/sin table precomputed), store q and write k, v
// into the cache slot of the row's position (V transposed).
// Grid (rows, heads / 4), one wave per (row, head) of the hq + 2*hkv heads:
// q and k heads rotate pairs (c, c + hd/2), v heads are copied to the
// transposed V cache.  A row of a quadratic-speculation block (blk[r] >= 0)
// writes its k and v to the forward's row scratch instead, [r][hkv][hd]
// each (its keys are seen by its own block only, never through the cache).
struct BlockScratch {
  const int32_t* blk;  // per row: first row of its block, or -1 (NULL: no block rows)
  void* k;             // [rows][hkv][hd], the model's storage type
  void* v;             // [rows][hkv][hd]
};
constexpr int ROPE_HEADS = 4;  // waves (heads) per workgroup
template <typename T>
__global__ __launch_bounds__(64 * ROPE_HEADS) void rope_kv_kernel(const float* __restrict__ P, int nslots,
                                                                  size_t stride, int hq, int hkv, int hd,
                                                                  const int32_t* row_seq,
                                                                  const int32_t* row_pos,
                                                                  const float* __restrict__ rope,
                                                                  T* __restrict__ qout, T* __restrict__ kc,
                                                                  T* __restrict__ vc, int ctx, size_t css,
                                                                  BlockScratch bs) {
  const int r = blockIdx.x, h = blockIdx.y * ROPE_HEADS + (int)(threadIdx.x >> 6);
  if (h >= hq + 2 * hkv) return;
  const int pos = row_pos[r], seq = row_seq[r];
  const bool scr = bs.blk && bs.blk[r] >= 0;
  const int half = hd / 2;
  const size_t rb = (size_t)r * (hq + 2 * hkv) * hd + (size_t)h * hd;
  if (h < hq + hkv) {
    for (int c = threadIdx.x & 63; c < half; c += 64) {
      const float xa = slot_sum(P, nslots, stride, rb + c);
      const float xb = slot_sum(P, nslots, stride, rb + c + half);
      const float cs = rope[((size_t)pos * half + c) * 2];
      const float sn = rope[((size_t)pos * half + c) * 2 + 1];
      const float ra = fmaf(xa, cs, -(xb * sn));
      const float rbv = fmaf(xb, cs, xa * sn);
      if (h < hq) {
        const size_t o = ((size_t)r * hq + h) * hd + c;
        Elem<T>::store(qout, o, ra);
        Elem<T>::store(qout, o + half, rbv);
      } else {
        T* kd = scr ? static_cast<T*>(bs.k) : kc;
        const size_t o = scr ? ((size_t)r * hkv + (h - hq)) * hd + c
                             : (size_t)seq * css + ((size_t)(h - hq) * ctx + pos) * hd + c;
        Elem<T>::store(kd, o, ra);
        Elem<T>::store(kd, o + half, rbv);
      }
    }
  } else {
    const int kh = h - hq - hkv;
    for (int dd = threadIdx.x & 63; dd < hd; dd += 64) {
      const float val = slot_sum(P, nslots, stride, rb + dd);
      if (scr)
        Elem<T>::store(static_cast<T*>(bs.v), ((size_t)r * hkv + kh) * hd + dd, val);
      else
        Elem<T>::store(vc, (size_t)seq * css + ((size_t)kh * hd + dd) * ctx + pos, val);
    }
  }
}

// The same for head_dim 128 with vector accesses: 16 lanes per head, each
// lane four consecutive columns of both halves (float4 slot and table loads),
// four heads per wave.  Same arithmetic per element as rope_kv_kernel.  VF16
// (bf16 models): V is written in the attention's fp16 form, and *vsat is set
// when a value saturates it.  Block rows write k and v (bf16, not the fp16
// form) to the row scratch as rope_kv_kernel does.
constexpr int ROPE128_HPW = 4;                    // heads per wave
constexpr int ROPE128_HEADS = 4 * ROPE128_HPW;    // heads per 256-thread workgroup
template <typename T, bool VF16, int NS>
__global__ __launch_bounds__(256) void rope_kv128_kernel(const float* __restrict__ P, size_t stride,
                                                         int hq, int hkv, const int32_t* row_seq,
                                                         const int32_t* row_pos, const float* __restrict__ rope,
                                                         T* __restrict__ qout, T* __restrict__ kc,
                                                         T* __restrict__ vc, int ctx, size_t css, int32_t* vsat,
                                                         BlockScratch bs) {
  constexpr int hd = 128, half = 64;
  const int r = blockIdx.x;
  const int h = blockIdx.y * ROPE128_HEADS + (int)(threadIdx.x >> 4);
  if (h >= hq + 2 * hkv) return;
  const int c = 4 * (threadIdx.x & 15);
  const int pos = row_pos[r], seq = row_seq[r];
  const size_t rb = (size_t)r * (hq + 2 * hkv) * hd + (size_t)h * hd;
  const f32x4 xa = slot_sum4n<NS>(P, stride, rb + c);
  const f32x4 xb = slot_sum4n<NS>(P, stride, rb + c + half);
  const bool scr = bs.blk && bs.blk[r] >= 0;
  if (h < hq + hkv) {
    const f32x4 t0 = *reinterpret_cast<const f32x4*>(rope + ((size_t)pos * half + c) * 2);
    const f32x4 t1 = *reinterpret_cast<const f32x4*>(rope + ((size_t)pos * half + c) * 2 + 4);
    const float cs[4] = {t0[0], t0[2], t1[0], t1[2]}, sn[4] = {t0[1], t0[3], t1[1], t1[3]};
    f32x4 ra, rbv;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      ra[e] = fmaf(xa[e], cs[e], -(xb[e] * sn[e]));
      rbv[e] = fmaf(xb[e], cs[e], xa[e] * sn[e]);
    }
    if (h < hq) {
      const size_t o = ((size_t)r * hq + h) * hd + c;
      Elem<T>::store4(qout, o, ra);
      Elem<T>::store4(qout, o + half, rbv);
    } else if (scr) {
      const size_t o = ((size_t)r * hkv + (h - hq)) * hd + c;
      Elem<T>::store4(static_cast<T*>(bs.k), o, ra);
      Elem<T>::store4(static_cast<T*>(bs.k), o + half, rbv);
    } else {
      const size_t o = (size_t)seq * css + ((size_t)(h - hq) * ctx + pos) * hd + c;
      Elem<T>::store4(kc, o, ra);
      Elem<T>::store4(kc, o + half, rbv);
    }
  } else if (scr) {
    const int kh = h - hq - hkv;
    const size_t o = ((size_t)r * hkv + kh) * hd + c;
    Elem<T>::store4(static_cast<T*>(bs.v), o, xa);
    Elem<T>::store4(static_cast<T*>(bs.v), o + half, xb);
  } else {
    const int kh = h - hq - hkv;
    const size_t o = (size_t)seq * css + (size_t)kh * hd * ctx + pos;
    bool sat = false;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      if constexpr (VF16) {
        vc[o + (size_t)(c + e) * ctx] = v_cache_f16(xa[e], sat);
        vc[o + (size_t)(c + half + e) * ctx] = v_cache_f16(xb[e], sat);
      } else {
        Elem<T>::store(vc, o + (size_t)(c + e) * ctx, xa[e]);
        Elem<T>::store(vc, o + (size_t)(c + half + e) * ctx, xb[e]);
      }
    }
    if (VF16 && sat && vsat) atomicOr(vsat, 1);
  }
}

// h = silu(gate) * up.  The gate/up projection's columns interleave in groups
// of 16 (the weight packing's order): columns [32j, 32j+16) are gate
// features [16j, 16j+16) and [32j+16, 32j+32) the matching up features.
// One thread per four consecutive columns of h in one row.
template <typename T, int NS>
__global__ __launch_bounds__(256) void swiglu_kernel(const float* __restrict__ P, size_t stride, int rows, int ffn,
                                                     T* __restrict__ h) {
  const int q4 = ffn / 4;
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= rows * q4) return;
  const int r = i / q4, c = (i - r * q4) * 4;
  const size_t rb = (size_t)r * 2 * ffn + (size_t)(c >> 4) * 32 + (c & 15);
  const f32x4 gt = slot_sum4n<NS>(P, stride, rb);
  const f32x4 up = slot_sum4n<NS>(P, stride, rb + 16);
  f32x4 o;
#pragma unroll
  for (int e = 0; e < 4; ++e) o[e] = gt[e] / (1.0f + expf(-gt[e])) * up[e];
  Elem<T>::store4(h, (size_t)r * ffn + c, o);
}

// LoRA middle activation A o, kept only on flagged rows (zero elsewhere);
// NS slots, all loaded before the first add (slot_sum's order).
template <typename T, int NS>
__global__ void lora_mid_kernel(const float* P, size_t stride, int rk, const int32_t* row_lora, T* mid) {
  const int r = blockIdx.x;
  const bool on = row_lora[r] != 0;
  for (int c = threadIdx.x; c < rk; c += blockDim.x) {
    const size_t off = (size_t)r * rk + c;
    float v[NS];
#pragma unroll
    for (int s = 0; s < NS; ++s) v[s] = P[s * stride + off];
    float acc = v[0];
#pragma unroll
    for (int s = 1; s < NS; ++s) acc += v[s];
    Elem<T>::store(mid, off, on ? acc : 0.f);
  }
}

__global__ void zero_kernel(float* p, size_t n) {
  for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += (size_t)gridDim.x * blockDim.x)
    p[i] = 0.f;
}

// ------------------------------------------------------------ vocab reduction
// Running (max, lowest argmax, sum exp(l - max)) of a stream of logits.
struct Red {
  float m;
  float s;
  int idx;
};

__device__ __forceinline__ Red red_merge(Red a, Red b) {
  if (b.s == 0.f) return a;
  if (a.s == 0.f) return b;
  const bool bw = (b.m > a.m) || (b.m == a.m && b.idx < a.idx);
  const Red w = bw ? b : a, o = bw ? a : b;
  Red out;
  out.m = w.m;
  out.idx = w.idx;
  out.s = w.s + o.s * expf(o.m - w.m);
  return out;
}

constexpr int VCHUNK = 4096;

// (m, s, idx) of lane ^ off, for the fixed-order wave merges below.
__device__ __forceinline__ Red red_shfl(const Red& a, int off) {
  Red o;
  o.m = __shfl_xor(a.m, off);
  o.s = __shfl_xor(a.s, off);
  o.idx = __shfl_xor(a.idx, off);
  return o;
}
// Merge over the 64 lanes (xor butterfly: every lane ends with the same
// result; ties keep the lowest index, so the argmax does not depend on the
// order).
__device__ __forceinline__ Red wave_red(Red a) {
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) a = red_merge(a, red_shfl(a, off));
  return a;
}

// Stage 1: grid (chunks, rows); per chunk partial (m, s, idx).  Each thread
// reads 16 logits (four float4 when the row allows it), takes their maximum
// first and then one sum of exp(x - m); the four waves merge through LDS.
__global__ __launch_bounds__(256) void vocab_stage1_kernel(const float* __restrict__ logits, int vocab,
                                                           const int32_t* row_kind, Red* part,
                                                           int nchunk, int32_t* status) {
  __shared__ Red sh[4];
  const int c = blockIdx.x, r = blockIdx.y, tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  if (c == 0 && r == 0 && tid == 0) *status = 0;
  if (row_kind[r] == 0) return;
  const float* lr = logits + (size_t)r * vocab;
  const int beg = c * VCHUNK, end = min(vocab, beg + VCHUNK);
  float v[16];
  int i0[4];
  const bool vec = ((vocab & 3) == 0);
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    i0[u] = beg + (u * 256 + tid) * 4;
    if (vec && i0[u] + 4 <= end) {
      const f32x4 q = *reinterpret_cast<const f32x4*>(lr + i0[u]);
#pragma unroll
      for (int e = 0; e < 4; ++e) v[u * 4 + e] = q[e];
    } else {
#pragma unroll
      for (int e = 0; e < 4; ++e) v[u * 4 + e] = i0[u] + e < end ? lr[i0[u] + e] : -INFINITY;
    }
  }
  Red acc{-INFINITY, 0.f, 0x7fffffff};
#pragma unroll
  for (int t = 0; t < 16; ++t)
    if (v[t] > acc.m) {  // increasing index order: the first maximum wins
      acc.m = v[t];
      acc.idx = i0[t >> 2] + (t & 3);
    }
  if (acc.idx != 0x7fffffff) {
#pragma unroll
    for (int t = 0; t < 16; ++t)
      if (v[t] != -INFINITY) acc.s += expf(v[t] - acc.m);
  } else {
    // no value above -inf: a NaN still poisons the sum (the row is flagged)
#pragma unroll
    for (int t = 0; t < 16; ++t)
      if (v[t] != v[t]) acc.s = v[t];
  }
  acc = wave_red(acc);
  if (lane == 0) sh[wave] = acc;
  __syncthreads();
  if (tid == 0) {
    Red t = sh[0];
    for (int w = 1; w < 4; ++w) t = red_merge(t, sh[w]);
    part[(size_t)r * nchunk + c] = t;
  }
}

// Stage 2: one wave per row merges its chunks (lane-strided loads, then the
// fixed wave merge).
__global__ __launch_bounds__(64) void vocab_stage2_kernel(const Red* part, int rows, int nchunk,
                                                          const int32_t* row_kind, int32_t* out_tok,
                                                          float* out_conf, int32_t* out_commit,
                                                          int32_t* status) {
  const int r = blockIdx.x, lane = threadIdx.x;
  const int kind = row_kind[r];
  if (kind == 0) {
    if (lane == 0) out_commit[r] = 0;
    return;
  }
  Red acc{-INFINITY, 0.f, 0x7fffffff};
  for (int c = lane; c < nchunk; c += 64) acc = red_merge(acc, part[(size_t)r * nchunk + c]);
  acc = wave_red(acc);
  if (lane != 0) return;
  const float conf = 1.0f / acc.s;
  const bool finite = isfinite(conf) && isfinite(acc.m) && acc.idx != 0x7fffffff;
  out_tok[r] = finite ? acc.idx : -1;
  out_conf[r] = finite ? conf : NAN;
  out_commit[r] = (kind == 1 && finite) ? 1 : 0;
  if (!finite) atomicAdd(status, 1);
}

// Stage 3: one wave per block: threshold commit, at least one.
__global__ __launch_bounds__(64) void commit_kernel(const int32_t* row_kind, const int32_t* block_start,
                                                    float threshold, const float* conf,
                                                    int32_t* out_commit) {
  const int b = blockIdx.x, lane = threadIdx.x;
  const int beg = block_start[b], end = block_start[b + 1];
  bool any = false;
  float best = -1.f;
  int bestr = 0x7fffffff;
  for (int r0 = beg; r0 < end; r0 += 64) {
    const int r = r0 + lane;
    bool pass = false;
    if (r < end && row_kind[r] == 2) {
      const float c = conf[r];
      if (isfinite(c)) {
        pass = c > threshold;
        if (c > best || (c == best && r < bestr)) {
          best = c;
          bestr = r;
        }
      }
      out_commit[r] = pass ? 1 : 0;
    } else if (r < end && row_kind[r] == 3) {
      out_commit[r] = 0;
    }
    any = any || pass;
  }
  any = __any(any);
  if (any) return;
  for (int off = 32; off > 0; off >>= 1) {
    const float ob = __shfl_xor(best, off);
    const int orr = __shfl_xor(bestr, off);
    if (ob > best || (ob == best && orr < bestr)) {
      best = ob;
      bestr = orr;
    }
  }
  if (lane == 0 && bestr != 0x7fffffff) out_commit[bestr] = 1;
}

// One wave per sequence: a = first mismatch (or k).
__global__ __launch_bounds__(64) void verify_accept_kernel(const int32_t* draft, const int32_t* ar,
                                                           int k, int32_t* accept_len,
                                                           int32_t* committed, int32_t* kv_len) {
  const int b = blockIdx.x, lane = threadIdx.x;
  int a = k;
  for (int i0 = 0; i0 < k; i0 += 64) {
    const int i = i0 + lane;
    const bool mis = i < k && draft[(size_t)b * k + i] != ar[(size_t)b * (k + 1) + i];
    const unsigned long long bal = __ballot(mis);
    if (bal) {
      a = i0 + __ffsll((long long)bal) - 1;
      break;
    }
  }
  for (int i = lane; i <= k; i += 64)
    committed[(size_t)b * (k + 1) + i] = (i <= a) ? ar[(size_t)b * (k + 1) + i] : -1;
  if (lane == 0) {
    accept_len[b] = a;
    if (kv_len) kv_len[b] += a;
  }
}

__global__ void scatter_gather_kernel(const int32_t* src, const int32_t* sidx, const int32_t* didx, int n,
                                      int32_t* dst) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) dst[didx[i]] = src[sidx[i]];
}

}  // namespace

#define TRI_DISPATCH(dtype, F32CALL, BF16CALL) \
  do {                                         \
    if ((dtype) == TRI_F32) {                  \
      F32CALL;                                 \
    } else {                                   \
      BF16CALL;                                \
    }                                          \
  } while (0)

hipError_t launch_embed(int dtype, const int32_t* tok, int rows, const void* E, int n_emb, int d, float* x,
                        hipStream_t st) {
  if (rows <= 0) return hipSuccess;
  if (d % 4) return hipErrorInvalidValue;
  const int threads = std::min(1024, (d / 4 + 63) / 64 * 64);
  TRI_DISPATCH(dtype,
               hipLaunchKernelGGL(embed_kernel<float>, dim3(rows), dim3(threads), 0, st, tok,
                                  static_cast<const float*>(E), n_emb, d, x),
               hipLaunchKernelGGL(embed_kernel<bf16_t>, dim3(rows), dim3(threads), 0, st, tok,
                                  static_cast<const bf16_t*>(E), n_emb, d, x));
  return hipGetLastError();
}

// Calls fn(std::integral_constant<int, n>) for a slot count n in [K, MAX_SLOTS].
template <int K, typename Fn>
hipError_t with_slots(int n, Fn& fn) {
  if constexpr (K > MAX_SLOTS) {
    return hipErrorInvalidValue;
  } else {
    return n == K ? fn(std::integral_constant<int, K>{}) : with_slots<K + 1>(n, fn);
  }
}

// Four columns per thread in one pass up to 4096 columns (1024 threads), two
// passes up to 5120 (640 threads), four up to 8192 (512 threads).
hipError_t launch_resid_norm(int dtype, float* x, const float* P, int nslots, size_t stride, int rows,
                             int d, const float* g, float eps, void* y, hipStream_t st) {
  if (rows <= 0) return hipSuccess;
  if (d > NORM_CHUNKS * 16 || d % 16 || nslots < 0 || nslots > MAX_SLOTS) return hipErrorInvalidValue;
  const int vpt = d <= 4096 ? 1 : (d <= 5120 ? 2 : 4);
  const int threads = ((d / 4 + vpt - 1) / vpt + 63) / 64 * 64;
  auto launch = [&](auto ns) -> hipError_t {
    constexpr int NS = decltype(ns)::value;
    auto go = [&](auto vp) {
      constexpr int V = decltype(vp)::value;
      TRI_DISPATCH(dtype,
                   hipLaunchKernelGGL((resid_norm_kernel<float, NS, V>), dim3(rows), dim3(threads), 0, st, x, P,
                                      stride, d, g, eps, static_cast<float*>(y)),
                   hipLaunchKernelGGL((resid_norm_kernel<bf16_t, NS, V>), dim3(rows), dim3(threads), 0, st, x, P,
                                      stride, d, g, eps, static_cast<bf16_t*>(y)));
    };
    if (vpt == 1)
      go(std::integral_constant<int, 1>{});
    else if (vpt == 2)
      go(std::integral_constant<int, 2>{});
    else
      go(std::integral_constant<int, 4>{});
    return hipGetLastError();
  };
  return with_slots<0>(nslots, launch);
}

hipError_t launch_rope_kv(int dtype, const float* P, int nslots, size_t stride, int rows, int hq, int hkv,
                          int hd, const int32_t* row_seq, const int32_t* row_pos, const float* rope,
                          void* qout, void* kc, void* vc, int ctx, size_t css, hipStream_t st, bool v_f16,
                          int32_t* vsat, const int32_t* row_blk, void* kscr, void* vscr) {
  if (rows <= 0) return hipSuccess;
  if (nslots < 1 || nslots > MAX_SLOTS || (v_f16 && (dtype != TRI_BF16 || hd != 128))) return hipErrorInvalidValue;
  if (row_blk && (!kscr || !vscr)) return hipErrorInvalidValue;
  const BlockScratch bs{row_blk, kscr, vscr};
  if (hd == 128) {
    const dim3 grid128(rows, (hq + 2 * hkv + ROPE128_HEADS - 1) / ROPE128_HEADS);
    auto launch = [&](auto ns) -> hipError_t {
      constexpr int NS = decltype(ns)::value;
      if (v_f16)
        hipLaunchKernelGGL((rope_kv128_kernel<bf16_t, true, NS>), grid128, dim3(256), 0, st, P, stride, hq, hkv,
                           row_seq, row_pos, rope, static_cast<bf16_t*>(qout), static_cast<bf16_t*>(kc),
                           static_cast<bf16_t*>(vc), ctx, css, vsat, bs);
      else
        TRI_DISPATCH(dtype,
                     hipLaunchKernelGGL((rope_kv128_kernel<float, false, NS>), grid128, dim3(256), 0, st, P, stride,
                                        hq, hkv, row_seq, row_pos, rope, static_cast<float*>(qout),
                                        static_cast<float*>(kc), static_cast<float*>(vc), ctx, css, vsat, bs),
                     hipLaunchKernelGGL((rope_kv128_kernel<bf16_t, false, NS>), grid128, dim3(256), 0, st, P,
                                        stride, hq, hkv, row_seq, row_pos, rope, static_cast<bf16_t*>(qout),
                                        static_cast<bf16_t*>(kc), static_cast<bf16_t*>(vc), ctx, css, vsat, bs));
      return hipGetLastError();
    };
    return with_slots<1>(nslots, launch);
  }
  const dim3 grid(rows, (hq + 2 * hkv + ROPE_HEADS - 1) / ROPE_HEADS);
  TRI_DISPATCH(dtype,
               hipLaunchKernelGGL(rope_kv_kernel<float>, grid, dim3(64 * ROPE_HEADS), 0, st, P, nslots, stride,
                                  hq, hkv, hd, row_seq, row_pos, rope, static_cast<float*>(qout),
                                  static_cast<float*>(kc), static_cast<float*>(vc), ctx, css, bs),
               hipLaunchKernelGGL(rope_kv_kernel<bf16_t>, grid, dim3(64 * ROPE_HEADS), 0, st, P, nslots,
                                  stride, hq, hkv, hd, row_seq, row_pos, rope,
                                  static_cast<bf16_t*>(qout), static_cast<bf16_t*>(kc),
                                  static_cast<bf16_t*>(vc), ctx, css, bs));
  return hipGetLastError();
}

hipError_t launch_swiglu(int dtype, const float* P, int nslots, size_t stride, int rows, int ffn, void* h,
                         hipStream_t st) {
  if (rows <= 0) return hipSuccess;
  if (ffn % 16 || nslots < 1 || nslots > MAX_SLOTS) return hipErrorInvalidValue;
  const dim3 grid((unsigned)(((size_t)rows * (ffn / 4) + 255) / 256));
  auto launch = [&](auto ns) -> hipError_t {
    constexpr int NS = decltype(ns)::value;
    TRI_DISPATCH(dtype,
                 hipLaunchKernelGGL((swiglu_kernel<float, NS>), grid, dim3(256), 0, st, P, stride, rows, ffn,
                                    static_cast<float*>(h)),
                 hipLaunchKernelGGL((swiglu_kernel<bf16_t, NS>), grid, dim3(256), 0, st, P, stride, rows, ffn,
                                    static_cast<bf16_t*>(h)));
    return hipGetLastError();
  };
  return with_slots<1>(nslots, launch);
}

hipError_t launch_lora_mid(int dtype, const float* P, int nslots, size_t stride, int rows, int rk,
                           const int32_t* row_lora, void* mid, hipStream_t st) {
  if (rows <= 0) return hipSuccess;
  if (nslots < 1 || nslots > MAX_SLOTS) return hipErrorInvalidValue;
  auto launch = [&](auto ns) -> hipError_t {
    constexpr int NS = decltype(ns)::value;
    TRI_DISPATCH(dtype,
                 hipLaunchKernelGGL((lora_mid_kernel<float, NS>), dim3(rows), dim3(128), 0, st, P, stride, rk,
                                    row_lora, static_cast<float*>(mid)),
                 hipLaunchKernelGGL((lora_mid_kernel<bf16_t, NS>), dim3(rows), dim3(128), 0, st, P, stride, rk,
                                    row_lora, static_cast<bf16_t*>(mid)));
    return hipGetLastError();
  };
  return with_slots<1>(nslots, launch);
}

hipError_t launch_zero_f32(float* p, size_t n, hipStream_t st) {
  if (n == 0) return hipSuccess;
  const size_t blocks = (n + 255) / 256;
  hipLaunchKernelGGL(zero_kernel, dim3(blocks > 4096 ? 4096 : (unsigned)blocks), dim3(256), 0, st, p, n);
  return hipGetLastError();
}

size_t vocab_ws_bytes(int rows, int vocab) {
  const int nchunk = (vocab + VCHUNK - 1) / VCHUNK;
  return (size_t)rows * nchunk * sizeof(Red) + 256;
}

hipError_t launch_sample_commit(const float* logits, int rows, int vocab, const int32_t* row_kind,
                                const int32_t* block_start, int n_blocks, float threshold,
                                int32_t* out_tok, float* out_conf, int32_t* out_commit,
                                int32_t* out_status, void* ws, hipStream_t st) {
  if (rows <= 0) return hipSuccess;
  const int nchunk = (vocab + VCHUNK - 1) / VCHUNK;
  Red* part = static_cast<Red*>(ws);
  hipLaunchKernelGGL(vocab_stage1_kernel, dim3(nchunk, rows), dim3(256), 0, st, logits, vocab, row_kind,
                     part, nchunk, out_status);
  hipLaunchKernelGGL(vocab_stage2_kernel, dim3(rows), dim3(64), 0, st, part, rows, nchunk,
                     row_kind, out_tok, out_conf, out_commit, out_status);
  if (n_blocks > 0)
    hipLaunchKernelGGL(commit_kernel, dim3(n_blocks), dim3(64), 0, st, row_kind, block_start, threshold,
                       out_conf, out_commit);
  return hipGetLastError();
}

hipError_t launch_verify_accept(const int32_t* draft, const int32_t* ar_tok, int batch, int k,
                                int32_t* accept_len, int32_t* committed, int32_t* kv_len,
                                hipStream_t st) {
  if (batch <= 0) return hipSuccess;
  hipLaunchKernelGGL(verify_accept_kernel, dim3(batch), dim3(64), 0, st, draft, ar_tok, k, accept_len,
                     committed, kv_len);
  return hipGetLastError();
}

hipError_t launch_scatter_gather(const int32_t* src, const int32_t* sidx, const int32_t* didx, int n,
                                 int32_t* dst, hipStream_t st) {
  if (n <= 0) return hipSuccess;
  hipLaunchKernelGGL(scatter_gather_kernel, dim3((n + 255) / 256), dim3(256), 0, st, src, sidx, didx, n, dst);
  return hipGetLastError();
}

}  // namespace tri
