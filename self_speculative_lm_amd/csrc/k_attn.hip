// Block-causal grouped-query attention over the KV cache.
//
// Every query row r attends to keys [0, hi[r]) of its sequence: a clean row at
// position p has hi = p + 1 (causal), a row of the noisy block [L, L + B) has
// hi = L + B (bidirectional inside the block, causal over the prefix)
// [Notes §3.2; Digest, Method].  Query head h reads kv head h / (hq / hkv).
//
// bf16 kernel (gfx950 MFMA): one workgroup per (split of kv_split keys,
// group of up to 16*WAVES query vectors, sequence x kv head).  All query heads
// of a kv head share the K/V tiles, so K [64 keys][128] and V^T [128][64 keys]
// tiles are staged in LDS (V is cached transposed, so both tiles are
// contiguous 16-byte loads) and read by every wave.  The tiles are
// double-buffered: the loads of tile t+1 are in flight while tile t runs.
// Each wave owns 16 query vectors and computes S^T = K Q^T with
// v_mfma_f32_16x16x32_bf16.  The K rows fed to the MFMA are permuted so that a
// lane ends up holding 8 scores of one query for 8 consecutive keys: the
// softmax row statistics then need only two cross-lane steps, and the same
// registers, rounded to bf16, are directly the B operand of O^T = V^T P^T (no
// LDS round trip for P).  Online softmax in float32 (exp2 with the scale
// folded in).  Splits write unnormalised partials (O, m, l) that a combine
// kernel merges in split order; a launch with a single split normalises in
// place.  A row's result depends only on its own q, its keys and kv_split,
// not on the other rows of the launch.
#include <math.h>

#include "tri_common.h"

namespace tri {
namespace {

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

template <int WAVES>
__global__ __launch_bounds__(WAVES * 64) void attn_bf16_kernel(AttnArgs a) {
  constexpr int NT = WAVES * 64;
  constexpr int PIECES = KT * HD / 8;  // 16-byte pieces of one K (or V^T) tile
  constexpr int PPT = PIECES / NT;     // per thread
  __shared__ __attribute__((aligned(16))) bf16_t ks[2][KT * KPAD];
  __shared__ __attribute__((aligned(16))) bf16_t vs[2][HD * VPAD];
  __shared__ int s_maxhi;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int seq = blockIdx.z / a.hkv, kvh = blockIdx.z - seq * a.hkv;
  const int G = a.hq / a.hkv;
  const int r0 = a.seq_start[seq];
  const int nq = (a.seq_start[seq + 1] - r0) * G;
  const int qbase = blockIdx.y * (WAVES * 16);
  if (qbase >= nq) return;

  if (tid == 0) s_maxhi = 0;
  __syncthreads();
  {
    int myhi = 0;
    const int qend = min(nq, qbase + WAVES * 16);
    for (int v = qbase + tid; v < qend; v += NT) myhi = max(myhi, a.row_hi[r0 + v / G]);
    atomicMax(&s_maxhi, myhi);
  }
  __syncthreads();
  const int wg_hi = s_maxhi;
  const int kbeg = blockIdx.x * a.kv_split;
  if (kbeg >= wg_hi) return;
  const int kend = min(kbeg + a.kv_split, wg_hi);

  const int j = lane & 15, g = lane >> 4;
  const int v = qbase + wave * 16 + j;
  const bool valid = v < nq;
  const int row = r0 + (valid ? v / G : 0);
  const int head = kvh * G + (valid ? v % G : 0);
  const int lim = valid ? min(a.row_hi[row], kend) : 0;

  const bf16x8 zero = {};
  bf16x8 qf[4];
  {
    const bf16_t* qp = a.q + ((size_t)row * a.hq + head) * HD + g * 8;
#pragma unroll
    for (int ds = 0; ds < 4; ++ds) qf[ds] = valid ? ld16(qp + ds * 32) : zero;
  }
  const int cseq = a.slot_seq ? a.slot_seq[seq] : seq;
  const bf16_t* kbase = a.kc + (size_t)(cseq * a.hkv + kvh) * a.ctx * HD;
  const bf16_t* vbase = a.vc + (size_t)(cseq * a.hkv + kvh) * HD * a.ctx;

  // Tile staging: registers <- global (keys >= kend read as zero), then LDS.
  auto load_tile = [&](int t0, bf16x8* kr, bf16x8* vr) {
#pragma unroll
    for (int u = 0; u < PPT; ++u) {
      const int i = tid + u * NT;
      const int key = i >> 4, c = i & 15;
      kr[u] = (t0 + key < kend) ? ld16(kbase + (size_t)(t0 + key) * HD + c * 8) : zero;
      const int d = i >> 3, c8 = i & 7;
      const int key0 = t0 + c8 * 8;
      bf16x8 val = zero;
      if (key0 < kend) {
        val = ld16(vbase + (size_t)d * a.ctx + key0);
        if (key0 + 8 > kend) {
#pragma unroll
          for (int e = 0; e < 8; ++e)
            if (key0 + e >= kend) val[e] = (__bf16)0.0f;
        }
      }
      vr[u] = val;
    }
  };
  auto store_tile = [&](int b, const bf16x8* kr, const bf16x8* vr) {
#pragma unroll
    for (int u = 0; u < PPT; ++u) {
      const int i = tid + u * NT;
      *reinterpret_cast<bf16x8*>(&ks[b][(i >> 4) * KPAD + (i & 15) * 8]) = kr[u];
      *reinterpret_cast<bf16x8*>(&vs[b][(i >> 3) * VPAD + (i & 7) * 8]) = vr[u];
    }
  };

  f32x4 oacc[8];
#pragma unroll
  for (int dt = 0; dt < 8; ++dt) oacc[dt] = f32x4{0.f, 0.f, 0.f, 0.f};
  float m_run = -1e30f, l_run = 0.f;

  // One 64-key tile from LDS buffer b starting at key t0.
  auto compute = [&](int b, int t0) {
    // S^T tile t of key group m: MFMA row i loads key 32m + 8(i/4) + 4t + i%4,
    // so output lane (j, g) gets keys 32m + 8g + (4t + r) of query j.
    float p[2][8];
    float tmax = -INFINITY;
#pragma unroll
    for (int m = 0; m < 2; ++m) {
#pragma unroll
      for (int t = 0; t < 2; ++t) {
        f32x4 s = {0.f, 0.f, 0.f, 0.f};
        const int krow = 32 * m + 8 * (j >> 2) + 4 * t + (j & 3);
#pragma unroll
        for (int ds = 0; ds < 4; ++ds) {
          const bf16x8 kf = *reinterpret_cast<const bf16x8*>(&ks[b][krow * KPAD + ds * 32 + g * 8]);
          s = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kf, qf[ds], s, 0, 0, 0);
        }
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int key = t0 + 32 * m + 8 * g + 4 * t + r;
          const float sv = (key < lim) ? s[r] * a.scale_log2 : -INFINITY;
          p[m][4 * t + r] = sv;
          tmax = fmaxf(tmax, sv);
        }
      }
    }
    tmax = fmaxf(tmax, __shfl_xor(tmax, 16));
    tmax = fmaxf(tmax, __shfl_xor(tmax, 32));
    const float m_new = fmaxf(m_run, tmax);
    const float alpha = exp2f(m_run - m_new);
    m_run = m_new;
    float psum = 0.f;
    bf16x8 pb[2];
#pragma unroll
    for (int m = 0; m < 2; ++m) {
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float pv = exp2f(p[m][e] - m_new);
        psum += pv;
        pb[m][e] = (__bf16)pv;
      }
    }
    l_run = l_run * alpha + psum;
#pragma unroll
    for (int dt = 0; dt < 8; ++dt) oacc[dt] *= alpha;
#pragma unroll
    for (int dt = 0; dt < 8; ++dt) {
#pragma unroll
      for (int m = 0; m < 2; ++m) {
        const bf16x8 vf = *reinterpret_cast<const bf16x8*>(&vs[b][(16 * dt + j) * VPAD + 32 * m + 8 * g]);
        oacc[dt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vf, pb[m], oacc[dt], 0, 0, 0);
      }
    }
  };

  bf16x8 kr[PPT], vr[PPT];
  load_tile(kbeg, kr, vr);
  store_tile(0, kr, vr);
  __syncthreads();
  int b = 0;
  for (int t0 = kbeg; t0 < kend; t0 += KT) {
    const bool more = t0 + KT < kend;
    if (more) load_tile(t0 + KT, kr, vr);
    compute(b, t0);
    if (more) store_tile(b ^ 1, kr, vr);
    __syncthreads();
    b ^= 1;
  }
  l_run += __shfl_xor(l_run, 16);
  l_run += __shfl_xor(l_run, 32);
  if (!valid) return;
  // lane (j, g) holds O^T[16dt + 4g + r][query j]
  if (a.nsplit == 1) {
    bf16_t* op = a.out + ((size_t)row * a.hq + head) * HD + 4 * g;
#pragma unroll
    for (int dt = 0; dt < 8; ++dt) {
      uint32_t lo = (uint32_t)f32_to_bf16(oacc[dt][0] / l_run) |
                    ((uint32_t)f32_to_bf16(oacc[dt][1] / l_run) << 16);
      uint32_t hi = (uint32_t)f32_to_bf16(oacc[dt][2] / l_run) |
                    ((uint32_t)f32_to_bf16(oacc[dt][3] / l_run) << 16);
      *reinterpret_cast<uint2*>(op + 16 * dt) = make_uint2(lo, hi);
    }
  } else {
    const size_t base = ((size_t)blockIdx.x * a.rows + row) * a.hq + head;
    float* po = a.part_o + base * HD + 4 * g;
#pragma unroll
    for (int dt = 0; dt < 8; ++dt) *reinterpret_cast<f32x4*>(po + 16 * dt) = oacc[dt];
    if (g == 0) {
      a.part_ml[base * 2] = m_run;
      a.part_ml[base * 2 + 1] = l_run;
    }
  }
}

// Merge the split partials of one (row, head) in split order.
template <typename T>
__global__ void attn_combine_kernel(const float* part_o, const float* part_ml, const int32_t* row_hi,
                                    int rows, int hq, int hd, int kv_split, T* out) {
  const int row = blockIdx.x, head = blockIdx.y;
  const int ns = (row_hi[row] + kv_split - 1) / kv_split;
  float M = -1e30f;
  for (int c = 0; c < ns; ++c) M = fmaxf(M, part_ml[(((size_t)c * rows + row) * hq + head) * 2]);
  for (int d = threadIdx.x; d < hd; d += blockDim.x) {
    float L = 0.f, O = 0.f;
    for (int c = 0; c < ns; ++c) {
      const size_t base = ((size_t)c * rows + row) * hq + head;
      const float w = exp2f(part_ml[base * 2] - M);
      L += part_ml[base * 2 + 1] * w;
      O += part_o[base * hd + d] * w;
    }
    Elem<T>::store(out, ((size_t)row * hq + head) * hd + d, O / L);
  }
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

int attn_pick_split(int max_hi) {
  // keys per split: enough splits to spread a long prefix over the chip
  int s = 256;
  while (s < 4096 && (max_hi + s - 1) / s > 32) s *= 2;
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
  const int waves = qtiles > 4 ? 8 : 4;  // >= 4 waves: staging is spread over >= 256 threads
  const int qgroups = (qtiles + waves - 1) / waves;
  dim3 grid(a.nsplit, qgroups, L.n_seq * L.hkv);
  if (waves == 4)
    hipLaunchKernelGGL(attn_bf16_kernel<4>, grid, dim3(256), 0, st, a);
  else
    hipLaunchKernelGGL(attn_bf16_kernel<8>, grid, dim3(512), 0, st, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || a.nsplit == 1) return e;
  hipLaunchKernelGGL(attn_combine_kernel<bf16_t>, dim3(L.rows, L.hq), dim3(HD), 0, st, a.part_o, a.part_ml,
                     L.row_hi, L.rows, L.hq, HD, L.kv_split, a.out);
  return hipGetLastError();
}

}  // namespace tri
