// Block-causal grouped-query attention over the KV cache.
//
// Every query row r attends to keys [0, hi[r]) of its sequence: a clean row at
// position p has hi = p + 1 (causal), a row of the noisy block [L, L + B) has
// hi = L + B (bidirectional inside the block, causal over the prefix)
// [Notes §3.2; Digest, Method].  Query head h reads kv head h / (hq / hkv).
//
// bf16 kernel (gfx950 MFMA): one workgroup per (split of kv_split keys,
// group of up to 16*WAVES*QT query vectors, sequence x kv head).  All query
// heads of a kv head share the K/V tiles, so K [64 keys][128] and V^T
// [128][64 keys] tiles are staged in LDS (V is cached transposed, so both
// tiles are contiguous 16-byte loads) and read by every wave.  The tiles are
// double-buffered: the loads of tile t+1 are in flight while tile t runs, and
// they are unconditional (a tile never crosses the cache capacity, and the
// cache holds finite values everywhere, so keys past a row's limit are masked
// through their scores alone).  Each wave owns QT tiles of 16 query vectors
// and computes S^T = K Q^T with v_mfma_f32_16x16x32_bf16, reading every K and
// V fragment from LDS once for its QT query tiles.  The K rows fed to the
// MFMA are permuted so that a lane ends up holding 8 scores of one query for 8
// consecutive keys: the softmax row statistics then need only two cross-lane
// steps, and the same registers, rounded to fp16, are directly the B operand
// of O^T = V^T P^T (no LDS round trip for P).  P.V runs in fp16 (V converted
// from bf16 when staged, exact inside the fp16 range and saturated at
// +-65504): P in [0, 1] keeps 11 significant bits instead of bf16's 8, which
// measurably moved the logits of 4096-wide models.  Online softmax in float32
// (exp2 with the scale folded in).  Splits write unnormalised partials
// (O, m, l) that a combine kernel merges in split order; a launch with a
// single split normalises in place.  A row's result depends only on its own
// q, its keys and kv_split, not on the other rows of the launch.
#include <math.h>

#include "tri_common.h"

namespace tri {
namespace {

typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));

constexpr int HD = 128;
constexpr int KT = 64;
constexpr int KPAD = HD + 8;  // LDS row stride (elements) of the K tile
constexpr int VPAD = KT + 8;  // LDS row stride (elements) of the V^T tile

struct AttnArgs {
  const bf16_t* q;
  const bf16_t* kc;
  const bf16_t* vc;
  const int32_t* seq_start;
  const int32_t* slot_seq;
  const int32_t* row_hi;
  int rows, hq, hkv, ctx, kv_split, nsplit;
  float scale_log2;
  bf16_t* out;
  float* part_o;   // [nsplit][rows][hq][HD]
  float* part_ml;  // [nsplit][rows][hq][2]
};

__device__ __forceinline__ bf16x8 ld16(const bf16_t* p) {
  return *reinterpret_cast<const bf16x8*>(p);
}

// NT_ALL > 0: a split holds at most NT_ALL tiles and all of them are loaded at
// once, together with the queries, before anything else (one memory round
// trip per split, the rest is compute); NT_ALL == 0: any number of tiles,
// double-buffered.
template <int WAVES, int QT, int NT_ALL>
__global__ __launch_bounds__(WAVES * 64) void attn_bf16_kernel(AttnArgs a) {
  constexpr int NT = WAVES * 64;
  constexpr int PIECES = KT * HD / 8;  // 16-byte pieces of one K (or V^T) tile
  constexpr int PPT = PIECES / NT;     // per thread
  constexpr int NREG = NT_ALL > 0 ? NT_ALL : 1;
  static_assert(PIECES % NT == 0, "every thread stages the same number of pieces");
  __shared__ __attribute__((aligned(16))) bf16_t ks[2][KT * KPAD];
  __shared__ __attribute__((aligned(16))) _Float16 vs[2][HD * VPAD];  // V^T tile in fp16
  __shared__ int s_maxhi;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int seq = blockIdx.z / a.hkv, kvh = blockIdx.z - seq * a.hkv;
  const int G = a.hq / a.hkv;
  const int r0 = a.seq_start[seq];
  const int nq = (a.seq_start[seq + 1] - r0) * G;
  const int qbase = blockIdx.y * (WAVES * 16 * QT);
  if (qbase >= nq) return;
  const int kbeg = blockIdx.x * a.kv_split;
  const int cseq = a.slot_seq ? a.slot_seq[seq] : seq;
  const bf16_t* kbase = a.kc + (size_t)(cseq * a.hkv + kvh) * a.ctx * HD;
  const bf16_t* vbase = a.vc + (size_t)(cseq * a.hkv + kvh) * HD * a.ctx;

  // Tile staging: registers <- global (whole 64-key tiles, clamped inside the
  // cache capacity), then LDS.
  auto load_tile = [&](int t0, bf16x8* kr, bf16x8* vr) {
    t0 = min(t0, a.ctx - KT);
#pragma unroll
    for (int u = 0; u < PPT; ++u) {
      const int i = tid + u * NT;
      kr[u] = ld16(kbase + (size_t)(t0 + (i >> 4)) * HD + (i & 15) * 8);
      vr[u] = ld16(vbase + (size_t)(i >> 3) * a.ctx + t0 + (i & 7) * 8);
    }
  };
  // V is converted to fp16 here (exact inside the fp16 range, saturated
  // outside it).  vlim < 64: keys of the tile at or past vlim may hold
  // anything (a caller's cache is not cleared); their scores are masked and
  // their V values are zeroed here, by the thread that stages them, so that
  // 0 * V is never NaN.
  auto store_tile = [&](int b, const bf16x8* kr, const bf16x8* vr, int vlim) {
#pragma unroll
    for (int u = 0; u < PPT; ++u) {
      const int i = tid + u * NT;
      *reinterpret_cast<bf16x8*>(&ks[b][(i >> 4) * KPAD + (i & 15) * 8]) = kr[u];
      f16x8 vv;
#pragma unroll
      for (int e = 0; e < 8; ++e) vv[e] = (_Float16)fminf(fmaxf((float)vr[u][e], -65504.f), 65504.f);
      if (vlim < KT) {
#pragma unroll
        for (int e = 0; e < 8; ++e)
          if ((i & 7) * 8 + e >= vlim) vv[e] = (_Float16)0.0f;
      }
      *reinterpret_cast<f16x8*>(&vs[b][(i >> 3) * VPAD + (i & 7) * 8]) = vv;
    }
  };

  // 1. Issue the tile loads of the split (all of them, or the first) and the
  //    query loads; they need nothing but the launch geometry.
  bf16x8 kr[NREG][PPT], vr[NREG][PPT];
#pragma unroll
  for (int t = 0; t < NREG; ++t) load_tile(kbeg + t * KT, kr[t], vr[t]);
  const int j = lane & 15, g = lane >> 4;
  bool valid[QT];
  int row[QT], head[QT], rhi[QT];
  bf16x8 qf[QT][4];
#pragma unroll
  for (int q = 0; q < QT; ++q) {
    const int v = qbase + (wave * QT + q) * 16 + j;
    valid[q] = v < nq;
    row[q] = r0 + (valid[q] ? v / G : 0);
    head[q] = kvh * G + (valid[q] ? v % G : 0);
    rhi[q] = a.row_hi[row[q]];
    const bf16_t* qp = a.q + ((size_t)row[q] * a.hq + head[q]) * HD + g * 8;
#pragma unroll
    for (int ds = 0; ds < 4; ++ds) qf[q][ds] = ld16(qp + ds * 32);
  }

  // 2. Key range of this workgroup: up to the largest limit of its rows.
  if (tid == 0) s_maxhi = 0;
  __syncthreads();
  {
    int myhi = 0;
    const int qend = min(nq, qbase + WAVES * 16 * QT);
    for (int v = qbase + tid; v < qend; v += NT) myhi = max(myhi, a.row_hi[r0 + v / G]);
    atomicMax(&s_maxhi, myhi);
  }
  __syncthreads();
  const int wg_hi = s_maxhi;
  if (kbeg >= wg_hi) return;
  const int kend = min(kbeg + a.kv_split, wg_hi);
  const int ntiles = (kend - kbeg + KT - 1) / KT;
  const int tail = kend - (kbeg + (ntiles - 1) * KT);  // valid keys in the last tile, 1..64
  int lim[QT];
#pragma unroll
  for (int q = 0; q < QT; ++q) lim[q] = valid[q] ? min(rhi[q], kend) : 0;

  f32x4 oacc[QT][8];
  float m_run[QT], l_run[QT];
#pragma unroll
  for (int q = 0; q < QT; ++q) {
#pragma unroll
    for (int dt = 0; dt < 8; ++dt) oacc[q][dt] = f32x4{0.f, 0.f, 0.f, 0.f};
    m_run[q] = -1e30f;
    l_run[q] = 0.f;
  }

  // One 64-key tile from LDS buffer b starting at key t0.
  auto compute = [&](int b, int t0) {
    // S^T tile t of key group m: MFMA row i loads key 32m + 8(i/4) + 4t + i%4,
    // so output lane (j, g) gets keys 32m + 8g + (4t + r) of query j.
    float p[QT][2][8];
    float tmax[QT];
#pragma unroll
    for (int q = 0; q < QT; ++q) tmax[q] = -INFINITY;
#pragma unroll
    for (int m = 0; m < 2; ++m) {
#pragma unroll
      for (int t = 0; t < 2; ++t) {
        f32x4 s[QT];
#pragma unroll
        for (int q = 0; q < QT; ++q) s[q] = f32x4{0.f, 0.f, 0.f, 0.f};
        const int krow = 32 * m + 8 * (j >> 2) + 4 * t + (j & 3);
#pragma unroll
        for (int ds = 0; ds < 4; ++ds) {
          const bf16x8 kf = *reinterpret_cast<const bf16x8*>(&ks[b][krow * KPAD + ds * 32 + g * 8]);
#pragma unroll
          for (int q = 0; q < QT; ++q) s[q] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kf, qf[q][ds], s[q], 0, 0, 0);
        }
#pragma unroll
        for (int q = 0; q < QT; ++q) {
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const int key = t0 + 32 * m + 8 * g + 4 * t + r;
            const float sv = (key < lim[q]) ? s[q][r] * a.scale_log2 : -INFINITY;
            p[q][m][4 * t + r] = sv;
            tmax[q] = fmaxf(tmax[q], sv);
          }
        }
      }
    }
    f16x8 pb[QT][2];
#pragma unroll
    for (int q = 0; q < QT; ++q) {
      float tm = tmax[q];
      tm = fmaxf(tm, __shfl_xor(tm, 16));
      tm = fmaxf(tm, __shfl_xor(tm, 32));
      const float m_new = fmaxf(m_run[q], tm);
      const float alpha = exp2f(m_run[q] - m_new);
      m_run[q] = m_new;
      float psum = 0.f;
#pragma unroll
      for (int m = 0; m < 2; ++m) {
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const float pv = exp2f(p[q][m][e] - m_new);
          psum += pv;
          pb[q][m][e] = (_Float16)pv;
        }
      }
      l_run[q] = l_run[q] * alpha + psum;
#pragma unroll
      for (int dt = 0; dt < 8; ++dt) oacc[q][dt] *= alpha;
    }
#pragma unroll
    for (int dt = 0; dt < 8; ++dt) {
#pragma unroll
      for (int m = 0; m < 2; ++m) {
        const f16x8 vf = *reinterpret_cast<const f16x8*>(&vs[b][(16 * dt + j) * VPAD + 32 * m + 8 * g]);
#pragma unroll
        for (int q = 0; q < QT; ++q)
          oacc[q][dt] = __builtin_amdgcn_mfma_f32_16x16x32_f16(vf, pb[q][m], oacc[q][dt], 0, 0, 0);
      }
    }
  };

  // 3. Tiles: stage, then multiply.
  if constexpr (NT_ALL > 0) {
    // every tile of the split is already in flight (tiles past the split's
    // end re-read a clamped tile and are never used)
#pragma unroll
    for (int t = 0; t < NT_ALL; ++t) {
      if (t >= ntiles) break;
      // buffer t&1 was last read by compute(t-2), which ended before the barrier of step t-1
      store_tile(t & 1, kr[t], vr[t], t + 1 == ntiles ? tail : KT);
      __syncthreads();
      compute(t & 1, kbeg + t * KT);
    }
  } else {
    // The last tile is peeled so that every prefetch in the loop is unconditional.
    store_tile(0, kr[0], vr[0], ntiles == 1 ? tail : KT);
    __syncthreads();
    int b = 0;
    for (int t = 0; t + 1 < ntiles; ++t) {
      load_tile(kbeg + (t + 1) * KT, kr[0], vr[0]);
      __builtin_amdgcn_sched_barrier(0);  // keep the prefetch ahead of the MFMAs
      compute(b, kbeg + t * KT);
      store_tile(b ^ 1, kr[0], vr[0], t + 2 == ntiles ? tail : KT);
      __syncthreads();
      b ^= 1;
    }
    compute(b, kbeg + (ntiles - 1) * KT);
  }

#pragma unroll
  for (int q = 0; q < QT; ++q) {
    float l = l_run[q];
    l += __shfl_xor(l, 16);
    l += __shfl_xor(l, 32);
    if (!valid[q]) continue;
    // lane (j, g) holds O^T[16dt + 4g + r][query j]
    if (a.nsplit == 1) {
      bf16_t* op = a.out + ((size_t)row[q] * a.hq + head[q]) * HD + 4 * g;
#pragma unroll
      for (int dt = 0; dt < 8; ++dt) {
        uint32_t lo = (uint32_t)f32_to_bf16(oacc[q][dt][0] / l) | ((uint32_t)f32_to_bf16(oacc[q][dt][1] / l) << 16);
        uint32_t hi = (uint32_t)f32_to_bf16(oacc[q][dt][2] / l) | ((uint32_t)f32_to_bf16(oacc[q][dt][3] / l) << 16);
        *reinterpret_cast<uint2*>(op + 16 * dt) = make_uint2(lo, hi);
      }
    } else {
      const size_t base = ((size_t)blockIdx.x * a.rows + row[q]) * a.hq + head[q];
      float* po = a.part_o + base * HD + 4 * g;
#pragma unroll
      for (int dt = 0; dt < 8; ++dt) *reinterpret_cast<f32x4*>(po + 16 * dt) = oacc[q][dt];
      if (g == 0) {
        a.part_ml[base * 2] = m_run[q];
        a.part_ml[base * 2 + 1] = l;
      }
    }
  }
}

// Merge the split partials of one (row, head) in split order, as one online
// pass; the partials of up to 16 splits are loaded at once.
template <typename T>
__global__ void attn_combine_kernel(const float* part_o, const float* part_ml, const int32_t* row_hi,
                                    int rows, int hq, int hd, int kv_split, T* out) {
  constexpr int B = 16;
  const int row = blockIdx.x, head = blockIdx.y, d = threadIdx.x;
  const int ns = (row_hi[row] + kv_split - 1) / kv_split;
  float M = -1e30f, L = 0.f, O = 0.f;
  for (int c0 = 0; c0 < ns; c0 += B) {
    float m[B], l[B], o[B];
#pragma unroll
    for (int i = 0; i < B; ++i) {
      const size_t base = ((size_t)min(c0 + i, ns - 1) * rows + row) * hq + head;
      m[i] = part_ml[base * 2];
      l[i] = part_ml[base * 2 + 1];
      o[i] = d < hd ? part_o[base * hd + d] : 0.f;
    }
#pragma unroll
    for (int i = 0; i < B; ++i) {
      if (c0 + i >= ns) break;
      const float Mn = fmaxf(M, m[i]);
      const float wa = exp2f(M - Mn), wb = exp2f(m[i] - Mn);
      L = L * wa + l[i] * wb;
      O = O * wa + o[i] * wb;
      M = Mn;
    }
  }
  if (d < hd) Elem<T>::store(out, ((size_t)row * hq + head) * hd + d, O / L);
}

// float32 path: one wave per (row, head), keys 64 at a time, one pass.
__global__ __launch_bounds__(64) void attn_f32_kernel(const float* q, const float* kc, const float* vc,
                                                       const int32_t* seq_start, const int32_t* slot_seq,
                                                       int n_seq, const int32_t* row_hi, int hq, int hkv, int hd,
                                                       int ctx, float scale, float* out) {
  __shared__ float qs[HD];
  const int row = blockIdx.x, head = blockIdx.y, lane = threadIdx.x;
  int seq = 0;
  while (seq + 1 < n_seq && seq_start[seq + 1] <= row) ++seq;
  if (slot_seq) seq = slot_seq[seq];
  const int kvh = head / (hq / hkv);
  const int hi = row_hi[row];
  for (int d = lane; d < hd; d += 64) qs[d] = q[((size_t)row * hq + head) * hd + d];
  __syncthreads();
  const float* kb = kc + (size_t)(seq * hkv + kvh) * ctx * hd;
  const float* vb = vc + (size_t)(seq * hkv + kvh) * hd * ctx;
  float m = -1e30f, l = 0.f, o0 = 0.f, o1 = 0.f;
  for (int j0 = 0; j0 < hi; j0 += 64) {
    const int key = j0 + lane;
    float s = -INFINITY;
    if (key < hi) {
      float acc = 0.f;
      for (int d = 0; d < hd; ++d) acc = fmaf(qs[d], kb[(size_t)key * hd + d], acc);
      s = acc * scale;
    }
    float cmax = s;
    for (int off = 32; off > 0; off >>= 1) cmax = fmaxf(cmax, __shfl_xor(cmax, off));
    const float m_new = fmaxf(m, cmax);
    const float alpha = expf(m - m_new);
    const float p = (key < hi) ? expf(s - m_new) : 0.f;
    float ps = p;
    for (int off = 32; off > 0; off >>= 1) ps += __shfl_xor(ps, off);
    l = l * alpha + ps;
    o0 *= alpha;
    o1 *= alpha;
    const int nk = min(64, hi - j0);
    for (int jj = 0; jj < nk; ++jj) {
      const float pj = __shfl(p, jj);
      if (lane < hd) o0 = fmaf(pj, vb[(size_t)lane * ctx + j0 + jj], o0);
      if (lane + 64 < hd) o1 = fmaf(pj, vb[(size_t)(lane + 64) * ctx + j0 + jj], o1);
    }
    m = m_new;
  }
  float* op = out + ((size_t)row * hq + head) * hd;
  if (lane < hd) op[lane] = o0 / l;
  if (lane + 64 < hd) op[lane + 64] = o1 / l;
}

}  // namespace

int attn_pick_split(int max_ctx) {
  // keys per split for a session of max_ctx keys: the largest power of two at
  // most max_ctx / 32, within [128, 1024].  Measured on MI355X for 33-row
  // decode forwards (attention + combine): 600 keys 15 us with 128-key
  // splits, 8K keys 31 us with 512, 32K keys 64 us with 1024.  A session
  // keeps one split size, so a row's result never depends on the launch.
  int s = 128;
  while (s < 1024 && 2 * s <= max_ctx / 32) s *= 2;
  return s;
}

size_t attn_ws_bytes(int rows, int hq, int hd, int max_hi, int kv_split) {
  if (kv_split <= 0) kv_split = attn_pick_split(max_hi);
  const size_t ns = (size_t)((max_hi + kv_split - 1) / kv_split);
  if (ns <= 1) return 256;
  return ns * (size_t)rows * hq * (hd + 2) * sizeof(float) + 256;
}

hipError_t launch_attn(int dtype, const AttnLaunch& L, hipStream_t st) {
  if (L.rows <= 0) return hipSuccess;
  if (dtype == TRI_F32) {
    hipLaunchKernelGGL(attn_f32_kernel, dim3(L.rows, L.hq), dim3(64), 0, st, static_cast<const float*>(L.q),
                       static_cast<const float*>(L.kc), static_cast<const float*>(L.vc), L.seq_start, L.slot_seq,
                       L.n_seq, L.row_hi, L.hq, L.hkv, L.hd, L.ctx, L.scale, static_cast<float*>(L.out));
    return hipGetLastError();
  }
  AttnArgs a;
  a.q = static_cast<const bf16_t*>(L.q);
  a.kc = static_cast<const bf16_t*>(L.kc);
  a.vc = static_cast<const bf16_t*>(L.vc);
  a.seq_start = L.seq_start;
  a.slot_seq = L.slot_seq;
  a.row_hi = L.row_hi;
  a.rows = L.rows;
  a.hq = L.hq;
  a.hkv = L.hkv;
  a.ctx = L.ctx;
  a.kv_split = L.kv_split;
  a.nsplit = (L.max_hi + L.kv_split - 1) / L.kv_split;
  a.scale_log2 = L.scale * 1.4426950408889634f;
  a.out = static_cast<bf16_t*>(L.out);
  const size_t np = (size_t)a.nsplit * L.rows * L.hq;
  a.part_o = L.part;
  a.part_ml = L.part + np * HD;
  const int G = L.hq / L.hkv;
  const int qtiles = (L.max_rows_per_seq * G + 15) / 16;
  // Short prefixes: 4 waves of one query tile, several query groups (more
  // workgroups, each latency-bound); long prefixes: 8 waves of two query tiles,
  // one group (every K/V tile read once per kv head).
  const bool wide = qtiles > 4 && L.max_hi > 8192;
  const int waves = wide ? 8 : 4, qt = wide ? 2 : 1;
  const int qgroups = (qtiles + waves * qt - 1) / (waves * qt);
  // Splits of up to 4 tiles load all their tiles at once.
  const int nt = (L.kv_split == KT || L.kv_split == 2 * KT || L.kv_split == 4 * KT) ? L.kv_split / KT : 0;
  dim3 grid(a.nsplit, qgroups, L.n_seq * L.hkv);
#define TRI_ATTN(W_, Q_, N_)                                                                    \
  if (waves == W_ && qt == Q_ && nt == N_) {                                                    \
    hipLaunchKernelGGL((attn_bf16_kernel<W_, Q_, N_>), grid, dim3(W_ * 64), 0, st, a);          \
  }
  TRI_ATTN(4, 1, 1) TRI_ATTN(4, 1, 2) TRI_ATTN(4, 1, 4) TRI_ATTN(4, 1, 0)
  TRI_ATTN(8, 2, 1) TRI_ATTN(8, 2, 2) TRI_ATTN(8, 2, 4) TRI_ATTN(8, 2, 0)
#undef TRI_ATTN
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || a.nsplit == 1) return e;
  hipLaunchKernelGGL(attn_combine_kernel<bf16_t>, dim3(L.rows, L.hq), dim3(HD), 0, st, a.part_o, a.part_ml,
                     L.row_hi, L.rows, L.hq, HD, L.kv_split, a.out);
  return hipGetLastError();
}

}  // namespace tri
