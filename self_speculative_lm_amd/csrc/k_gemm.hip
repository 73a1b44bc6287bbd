// Projection GEMMs of the decode forward: Y = X W^T with X [M][K] (the rows of
// one forward) and W [N][K] (a weight matrix, streamed once per forward).
//
// At decode shapes M is 1..64 rows per 64-row tile while N*K is the whole
// weight matrix, so the kernel is bound by streaming W from HBM (every weight
// is loaded once per forward: [Blog], the paragraph on why AR decoding is
// memory bound).  The bf16 path still runs the dot products on the matrix
// cores (v_mfma_f32_16x16x32_bf16): a 16-feature x 16-row tile per MFMA, W as
// the A operand read straight from global memory into registers (16 rows x 64
// contiguous bytes per load instruction), the rows of X staged in LDS in
// MFMA-fragment order (conflict-free 1 KiB reads) and shared by the waves of
// the workgroup.  Both are double-buffered over 256-wide K chunks: the loads
// of chunk c+1 are in flight while chunk c runs on the matrix cores.
// Split-K across workgroups keeps enough workgroups in flight for the N = d
// projections; every split writes its own float32 partial slot and the
// consumer kernel (norm, RoPE, SwiGLU) adds the slots in slot order, so results
// are deterministic and independent of M (a row's value never depends on which
// other rows share the launch).
#include "tri_common.h"

namespace tri {
namespace {

constexpr int KC = 256;          // K per stage
constexpr int KSTEPS = KC / 32;  // MFMA k-steps per stage
constexpr int MAX_S = 16;        // split-K slots (a LoRA slot may be added by the caller)

struct GemmArgs {
  const bf16_t* X;
  int M, K;
  const bf16_t* w0;
  const bf16_t* w1;
  const bf16_t* w2;
  int r0, r1, r2;  // rows of the segments (0 = absent)
  int N, Ks;
  float* P;
  size_t slot_stride;
};

__device__ __forceinline__ bf16x8 ld16(const bf16_t* p) {
  return *reinterpret_cast<const bf16x8*>(p);
}

// Grid: x = feature blocks of 16*WAVES, y = K splits, z = 16*MT-row tiles of X.
// Wave w of a workgroup owns features [16*WAVES*x + 16*w, +16).
template <int MT, int WAVES>
__global__ __launch_bounds__(WAVES * 64) void gemm_bf16_kernel(GemmArgs a) {
  constexpr int NT = WAVES * 64;
  constexpr int XPIECES = MT * 16 * (KC / 8);     // 16-byte pieces of one X chunk
  constexpr int XPT = (XPIECES + NT - 1) / NT;    // pieces per thread
  __shared__ bf16x8 xs[2][KSTEPS][MT][64];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int n0 = blockIdx.x * (16 * WAVES) + wave * 16;
  const int m0 = blockIdx.z * (MT * 16);
  const int kbeg = blockIdx.y * a.Ks;
  const int kend = min(a.K, kbeg + a.Ks);
  const int nch = (kend - kbeg + KC - 1) / KC;

  // Segment of this wave's features (segment boundaries are multiples of 64;
  // rows past the end of the last segment are clamped and never stored).
  const bf16_t* wb = a.w0;
  int nl = n0, sr = a.r0;
  if (nl >= a.r0 && a.r1 > 0) {
    nl -= a.r0;
    wb = a.w1;
    sr = a.r1;
    if (nl >= a.r1 && a.r2 > 0) {
      nl -= a.r1;
      wb = a.w2;
      sr = a.r2;
    }
  }
  const int wr = min(nl + (lane & 15), sr - 1);
  // A operand: lane l supplies W[n0 + l%16][k + 8*(l/16) .. +8]
  const bf16_t* wrow = wb + (size_t)wr * a.K + (lane >> 4) * 8;
  const bf16x8 zero = {};

  auto load_w = [&](int kc, bf16x8* wf) {
#pragma unroll
    for (int s = 0; s < KSTEPS; ++s) {
      const int k = kc + s * 32;
      wf[s] = (k < kend) ? ld16(wrow + k) : zero;
    }
  };
  // B operand staging: xs[b][s][t][g*16 + j] = X[m0 + 16t + j][kc + 32s + 8g .. +8]
  auto load_x = [&](int kc, bf16x8* xr) {
#pragma unroll
    for (int it = 0; it < XPT; ++it) {
      const int i = tid + it * NT;
      const int g = i & 3, r = (i >> 2) % (MT * 16), s = (i >> 2) / (MT * 16);
      const int k = kc + s * 32 + g * 8, m = m0 + r;
      xr[it] = (i < XPIECES && m < a.M && k < kend) ? ld16(a.X + (size_t)m * a.K + k) : zero;
    }
  };
  auto store_x = [&](int b, const bf16x8* xr) {
#pragma unroll
    for (int it = 0; it < XPT; ++it) {
      const int i = tid + it * NT;
      if (i < XPIECES) {
        const int g = i & 3, r = (i >> 2) % (MT * 16), s = (i >> 2) / (MT * 16);
        xs[b][s][r >> 4][g * 16 + (r & 15)] = xr[it];
      }
    }
  };

  f32x4 acc[MT];
#pragma unroll
  for (int t = 0; t < MT; ++t) acc[t] = f32x4{0.f, 0.f, 0.f, 0.f};
  auto compute = [&](int b, const bf16x8* wf) {
#pragma unroll
    for (int s = 0; s < KSTEPS; ++s) {
#pragma unroll
      for (int t = 0; t < MT; ++t)
        acc[t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(wf[s], xs[b][s][t][lane], acc[t], 0, 0, 0);
    }
  };

  bf16x8 wA[KSTEPS], wB[KSTEPS], xr[XPT];
  load_w(kbeg, wA);
  load_x(kbeg, xr);
  store_x(0, xr);
  __syncthreads();
  for (int c = 0; c < nch; c += 2) {
    const bool h1 = c + 1 < nch;
    if (h1) {
      load_w(kbeg + (c + 1) * KC, wB);
      load_x(kbeg + (c + 1) * KC, xr);
    }
    compute(0, wA);
    if (h1) store_x(1, xr);
    __syncthreads();
    if (!h1) break;
    const bool h2 = c + 2 < nch;
    if (h2) {
      load_w(kbeg + (c + 2) * KC, wA);
      load_x(kbeg + (c + 2) * KC, xr);
    }
    compute(1, wB);
    if (h2) store_x(0, xr);
    __syncthreads();
  }
  // D layout: lane l holds D[4*(l/16) + r][l%16] = Y[m0 + 16t + l%16][n0 + 4*(l/16) + r]
  float* out = a.P + (size_t)blockIdx.y * a.slot_stride;
  const int nn = n0 + 4 * (lane >> 4);
#pragma unroll
  for (int t = 0; t < MT; ++t) {
    const int m = m0 + t * 16 + (lane & 15);
    if (m >= a.M) continue;
    if (nn + 4 <= a.N && (a.N & 3) == 0) {
      *reinterpret_cast<f32x4*>(out + (size_t)m * a.N + nn) = acc[t];
    } else {
      for (int r = 0; r < 4; ++r)
        if (nn + r < a.N) out[(size_t)m * a.N + nn + r] = acc[t][r];
    }
  }
}

// float32 path (small models): one thread per output, sequential K order.
__global__ __launch_bounds__(64) void gemm_f32_kernel(const float* X, int M, int K, const float* w0,
                                                       const float* w1, const float* w2, int r0,
                                                       int r1, int N, float* P) {
  const int n = blockIdx.x * 64 + threadIdx.x;
  const int m = blockIdx.y;
  if (n >= N || m >= M) return;
  const float* wb;
  int nl = n;
  if (nl < r0) {
    wb = w0;
  } else if ((nl -= r0) < r1) {
    wb = w1;
  } else {
    nl -= r1;
    wb = w2;
  }
  const float* wr = wb + (size_t)nl * K;
  const float* xr = X + (size_t)m * K;
  float acc = 0.f;
  for (int k = 0; k < K; ++k) acc = fmaf(xr[k], wr[k], acc);
  P[(size_t)m * N + n] = acc;
}

template <int MT>
void launch_mt(const GemmArgs& a, const GemmPlan& p, int M, hipStream_t st) {
  const int fb = 16 * p.waves;
  const dim3 grid((a.N + fb - 1) / fb, p.S, (M + 16 * MT - 1) / (16 * MT));
  if (p.waves == 8)
    hipLaunchKernelGGL((gemm_bf16_kernel<MT, 8>), grid, dim3(512), 0, st, a);
  else
    hipLaunchKernelGGL((gemm_bf16_kernel<MT, 4>), grid, dim3(256), 0, st, a);
}

}  // namespace

// The plan depends only on (N, K), never on M, so that a row's result is the
// same whatever the number of rows in the launch.
GemmPlan gemm_plan(int N, int K, int dtype) {
  GemmPlan p;
  p.waves = 4;
  if (dtype != TRI_BF16) {
    p.S = 1;
    p.Ks = K;
    return p;
  }
  // Measured on MI355X for the 8B/14B decode shapes (M = 32/33): 8-wave
  // workgroups everywhere; K per split about 512 for the d x d and QKV
  // projections, 768 for the long-K down projection, 1024 for the wide
  // gate/up projection; the lm_head (very wide N) runs unsplit.
  p.waves = N >= 128 ? 8 : 4;
  int Ks;
  if (N >= 65536)
    Ks = K;
  else if (N >= 16384)
    Ks = 1024;
  else if (K > 8192)
    Ks = 768;
  else
    Ks = 512;
  Ks = (Ks + KC - 1) / KC * KC;
  if (Ks > K) Ks = (K + 31) / 32 * 32;
  int S = (K + Ks - 1) / Ks;
  if (S > MAX_S) {
    Ks = ((K + MAX_S - 1) / MAX_S + KC - 1) / KC * KC;  // fewer, longer splits
    S = (K + Ks - 1) / Ks;
  }
  p.Ks = Ks;
  p.S = S;
  return p;
}

hipError_t launch_gemm(int dtype, const void* X, int M, int K, const WSeg* segs, int nseg, int N,
                       const GemmPlan& plan, float* P, size_t slot_stride, hipStream_t st) {
  const void* w0 = segs[0].ptr;
  const void* w1 = nseg > 1 ? segs[1].ptr : nullptr;
  const void* w2 = nseg > 2 ? segs[2].ptr : nullptr;
  const int r0 = segs[0].rows;
  const int r1 = nseg > 1 ? segs[1].rows : 0;
  const int r2 = nseg > 2 ? segs[2].rows : 0;
  if (M <= 0) return hipSuccess;
  if (dtype == TRI_BF16) {
    GemmArgs a;
    a.X = static_cast<const bf16_t*>(X);
    a.M = M;
    a.K = K;
    a.w0 = static_cast<const bf16_t*>(w0);
    a.w1 = static_cast<const bf16_t*>(w1);
    a.w2 = static_cast<const bf16_t*>(w2);
    a.r0 = r0;
    a.r1 = r1;
    a.r2 = r2;
    a.N = N;
    a.Ks = plan.Ks;
    a.P = P;
    a.slot_stride = slot_stride;
    const int mt = M >= 64 ? 4 : (M + 15) / 16;
    switch (mt) {
      case 1: launch_mt<1>(a, plan, M, st); break;
      case 2: launch_mt<2>(a, plan, M, st); break;
      case 3: launch_mt<3>(a, plan, M, st); break;
      default: launch_mt<4>(a, plan, M, st); break;
    }
  } else {
    dim3 grid((N + 63) / 64, M);
    hipLaunchKernelGGL(gemm_f32_kernel, grid, dim3(64), 0, st, static_cast<const float*>(X), M, K,
                       static_cast<const float*>(w0), static_cast<const float*>(w1),
                       static_cast<const float*>(w2), r0, r1, N, P);
  }
  return hipGetLastError();
}

}  // namespace tri
