// Projection GEMMs of the decode forward: Y = X W^T with X [M][K] (the rows of
// one forward) and W [N][K] (a weight matrix, streamed once per forward).
//
// At decode shapes M is 1..64 rows per 64-row tile while N*K is the whole
// weight matrix, so the kernel is bound by streaming W from HBM (every weight
// is loaded once per forward: [Blog], the paragraph on why AR decoding is
// memory bound).  The bf16 path runs the dot products on the matrix cores
// (v_mfma_f32_16x16x32_bf16: 16 features x 16 rows x 32 k per instruction).
//
// Weight layout.  At model creation every bf16 projection matrix is repacked
// once into MFMA-fragment order: the A operand of one MFMA (16 rows x 32 k,
// lane l holding row l%16, k-octet l/16) is one contiguous 1 KiB block, the 8
// fragments of a 128-row group at one k-step are adjacent, and k-steps follow
// each other.  A wave's load instruction therefore reads 1 KiB contiguous, a
// workgroup's K chunk is one contiguous block, and the whole matrix is swept
// almost linearly, in exactly the register layout the MFMA consumes.
//
// X rows are staged in LDS in fragment order (conflict-free 1 KiB reads) and
// shared by the 8 waves; W registers and X tiles are double-buffered over
// 256-wide K chunks so the loads of chunk c+1 are in flight while chunk c runs.
// Split-K across workgroups keeps enough workgroups in flight for the N = d
// projections; every split writes its own float32 partial slot and the
// consumer kernel (norm, RoPE, SwiGLU) adds the slots in slot order, so results
// are deterministic and independent of M (a row's value never depends on which
// other rows share the launch).
#include <algorithm>
#include <cstdlib>

#include "tri_common.h"

namespace tri {
namespace {

constexpr int KC = 256;          // K per stage
constexpr int KSTEPS = KC / 32;  // MFMA k-steps per stage
constexpr int MAX_S = 16;        // split-K slots (a LoRA slot may be added by the caller)
constexpr int WAVES_PER_WG = 8;  // waves per gemm workgroup, 16 features each
constexpr int GROUP = 16 * WAVES_PER_WG;  // rows per packing group (one workgroup's features)

__host__ __device__ __forceinline__ int kpad(int K) { return (K + KC - 1) / KC * KC; }

struct GemmArgs {
  const bf16_t* X;
  int M, K;
  const bf16_t* W;  // packed (step-major, see pack_bf16_kernel)
  int N, Ks, S;
  int nfb, ntiles;  // feature blocks; tiles = (M tiles) x nfb x S
  float* P;
  size_t slot_stride;
};

__device__ __forceinline__ bf16x8 ld16(const bf16_t* p) {
  return *reinterpret_cast<const bf16x8*>(p);
}

// Step-major packed layout of W for a plan (S splits of Ks, nfb blocks of 128
// features, G = nfb*S workgroup slots g = y*nfb + x).  A block is the 8 KiB one
// workgroup reads at one k-step: 8 fragments of 16 features x 32 k in MFMA A
// order (lane l holds feature 16w + l%16, k 8(l/16) .. +8).  Block (j, g), the
// j-th k-step of split y for feature block x, sits at index j*G + g, so at
// every k-step the workgroups of a launch read one contiguous window: measured
// on MI355X this sustains the linear-read rate, whereas one contiguous region
// per workgroup fell about 10% short.  K is zero-padded to S*Ks.
__global__ void pack_bf16_kernel(const bf16_t* w0, const bf16_t* w1, const bf16_t* w2, int r0, int r1, int N,
                                 int K, int nfb, int S, int steps, size_t npieces, bf16_t* dst) {
  const int G = nfb * S;
  for (size_t p = (size_t)blockIdx.x * blockDim.x + threadIdx.x; p < npieces;
       p += (size_t)gridDim.x * blockDim.x) {
    const size_t blk = p >> 9;
    const int w = (int)((p >> 6) & 7), lane = (int)(p & 63);
    const int j = (int)(blk / G), g = (int)(blk % G);
    const int x = g % nfb, y = g / nfb;
    const int row = (x * 8 + w) * 16 + (lane & 15);
    const int k = (y * steps + j) * 32 + (lane >> 4) * 8;
    bf16x8 v = {};
    if (row < N && k < K) {
      const bf16_t* src;
      if (row < r0)
        src = w0 + (size_t)row * K;
      else if (row < r0 + r1)
        src = w1 + (size_t)(row - r0) * K;
      else
        src = w2 + (size_t)(row - r0 - r1) * K;
      v = ld16(src + k);
    }
    *reinterpret_cast<bf16x8*>(dst + p * 8) = v;
  }
}

// float32 models keep row-major weights: the segments are concatenated.
__global__ void pack_f32_kernel(const float* w0, const float* w1, const float* w2, int r0, int r1, int N, int K,
                                float* dst) {
  const size_t n = (size_t)N * K;
  for (size_t p = (size_t)blockIdx.x * blockDim.x + threadIdx.x; p < n; p += (size_t)gridDim.x * blockDim.x) {
    const int row = (int)(p / K);
    const size_t c = p - (size_t)row * K;
    const float* src = row < r0 ? w0 + (size_t)row * K
                                : (row < r0 + r1 ? w1 + (size_t)(row - r0) * K : w2 + (size_t)(row - r0 - r1) * K);
    dst[p] = src[c];
  }
}

// One workgroup per tile (M tile z, K split y, feature block x), x fastest:
// blockIdx.x = z*G + g with g = y*nfb + x.  Wave w owns features
// [128x + 16w, +16) and writes them to split y's partial slot.
//
// A split is processed in passes of NCH stages of KC = 256 k (8 k-steps).
// Every pass is straight-line code (NCH is a template argument and the loops
// are fully unrolled).  Each wave keeps a ring of D W fragments in flight: the
// load for k-step j + D is issued right after the MFMAs of k-step j, and a
// scheduling barrier keeps the compiler from hoisting the loads (few loads in
// flight per wave, all workgroups reading one window, measured fastest).  X
// is double-buffered per stage in LDS; each stage's X loads are issued before
// the stage's W loads.  Rows past M read a clamped row whose results are never
// stored and padded k has zero weights, so no load is conditional.
//
// No W fragment is carried across a loop back-edge: with a runtime stage loop
// (fragments kept in registers from one iteration to the next) this compiler
// reused the upper half of a live 16x16x32 MFMA operand for other values, a
// miscompile that the operand check over the built assembly detects.
template <int MT, int NCH, int D>
__global__ __launch_bounds__(WAVES_PER_WG * 64) void gemm_bf16_kernel(GemmArgs a) {
  constexpr int WAVES = WAVES_PER_WG, NT = WAVES * 64, NS = NCH * KSTEPS;
  constexpr int XPIECES = MT * 16 * (KC / 8);  // 16-byte pieces of one X stage
  constexpr int XPT = XPIECES / NT;             // pieces per thread
  static_assert(XPIECES % NT == 0, "every thread stages the same number of X pieces");
  static_assert(D >= 1 && D <= KSTEPS, "ring depth");
  __shared__ bf16x8 xs[2][KSTEPS][MT][64];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int G = a.nfb * a.S;
  const int g = blockIdx.x % G;
  const int m0 = (blockIdx.x / G) * (MT * 16);
  const int fbx = g % a.nfb, y = g / a.nfb;
  const int kbeg = y * a.Ks;
  const int npass = a.Ks / (NCH * KC);
  const size_t wstep = (size_t)G * (WAVES * 512);  // elements between k-steps
  const bf16_t* wb = a.W + (size_t)g * (WAVES * 512) + wave * 512 + lane * 8;

  // B operand staging: xs[b][s][t][gg*16 + j] = X[m0 + 16t + j][k + 32s + 8gg .. +8]
  const bf16_t* xrow[XPT];
  int xk[XPT];
#pragma unroll
  for (int it = 0; it < XPT; ++it) {
    const int i = tid + it * NT;
    const int gg = i & 3, r = (i >> 2) % (MT * 16), s = (i >> 2) / (MT * 16);
    xrow[it] = a.X + (size_t)min(m0 + r, a.M - 1) * a.K;
    xk[it] = s * 32 + gg * 8;
  }
  f32x4 acc[MT];
#pragma unroll
  for (int t = 0; t < MT; ++t) acc[t] = f32x4{0.f, 0.f, 0.f, 0.f};

  for (int p = 0; p < npass; ++p) {
    const int k0 = kbeg + p * (NCH * KC);
    const bf16_t* wp = wb + (size_t)p * NS * wstep;
    bf16x8 ring[D], xr[XPT];
    auto load_x = [&](int c) {
#pragma unroll
      for (int it = 0; it < XPT; ++it)
        xr[it] = ld16(xrow[it] + min(k0 + c * KC + xk[it], a.K - 8));  // padded k: zero weights there
    };
    auto store_x = [&](int b) {
#pragma unroll
      for (int it = 0; it < XPT; ++it) {
        const int i = tid + it * NT;
        const int gg = i & 3, r = (i >> 2) % (MT * 16), s = (i >> 2) / (MT * 16);
        xs[b][s][r >> 4][gg * 16 + (r & 15)] = xr[it];
      }
    };
    if (p > 0) __syncthreads();  // the previous pass's last stage still reads xs
    load_x(0);
#pragma unroll
    for (int i = 0; i < D; ++i) ring[i] = ld16(wp + (size_t)i * wstep);
    store_x(0);
    __syncthreads();
#pragma unroll
    for (int c = 0; c < NCH; ++c) {
      if (c + 1 < NCH) load_x(c + 1);
#pragma unroll
      for (int s = 0; s < KSTEPS; ++s) {
        const int j = c * KSTEPS + s;
#pragma unroll
        for (int t = 0; t < MT; ++t)
          acc[t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ring[j % D], xs[c & 1][s][t][lane], acc[t], 0, 0, 0);
        if (j + D < NS) ring[j % D] = ld16(wp + (size_t)(j + D) * wstep);
        __builtin_amdgcn_sched_barrier(0);
      }
      if (c + 1 < NCH) {
        store_x((c + 1) & 1);
        __syncthreads();
      }
    }
  }
  // D layout: lane l holds D[4*(l/16) + r][l%16] = Y[m0 + 16t + l%16][n0 + 4*(l/16) + r]
  float* out = a.P + (size_t)y * a.slot_stride;
  const int nn = (fbx * WAVES + wave) * 16 + 4 * (lane >> 4);
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

// Large-M GEMM (prefill chunks, M > 64 rows): Y = X W^T with the arithmetic
// intensity of M / 2 flop per weight byte, built for the MFMA units.  One
// 256-thread workgroup per (128-row tile, 128-feature block, group of cs
// consecutive K splits of the packed layout), writing the group's slot; four
// waves of 64 features x 64 rows, each a 2 x 2 array of
// v_mfma_f32_32x32x16_bf16 tiles (A = W: lane l holds feature l%32, k
// 8(l/32)..+8; B = X^T: lane l holds row l%32, the same k; D: lane l,
// register r holds feature 8(r/4) + 4(l/32) + r%4 of row l%32).  A stage is
// 64 k: W as the two packed 8 KiB blocks, copied unchanged, and X with rows
// padded to 72 elements (the B reads of a 16-lane group then hit 16 distinct
// bank quads).  Stages travel global -> registers (a ring of R stages in
// flight per thread, so a stage's loads are issued R - 1 stages before they
// are needed) -> LDS (double-buffered, one barrier per stage); every W and X
// fragment read from LDS feeds two MFMAs.  The workgroups of one feature
// block get ids congruent modulo 8, so they run on one XCD and share its L2.
constexpr int BIG_BM = 128;            // rows per tile
constexpr int BIG_KST = 64;            // k per stage (two packed k-steps)
constexpr int BIG_XPAD = BIG_KST + 8;  // LDS row stride of the X tile (elements)
constexpr int BIG_R = 4;               // stages in flight per thread
typedef float f32x16 __attribute__((ext_vector_type(16)));

struct BigGrid {
  int ntm, nyg, cs;  // row tiles, K-split groups, packed splits per group
};

template <int R>
__global__ __launch_bounds__(256) void gemm_big_kernel(GemmArgs a, BigGrid bg) {
  const int id = blockIdx.x;
  const int q = id >> 3, per = bg.ntm * bg.nyg;
  const int fbx = (q / per) * 8 + (id & 7), rem = q - (q / per) * per;
  const int tm = rem % bg.ntm, yg = rem / bg.ntm;
  if (fbx >= a.nfb) return;
  __shared__ bf16x8 ws[2][2 * 512];                                          // 2 x 8 KiB per buffer
  __shared__ __attribute__((aligned(16))) bf16_t xs[2][BIG_BM * BIG_XPAD];  // 18 KiB per buffer
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wf = wave & 1, wm = wave >> 1;  // the wave's 64-feature and 64-row halves
  const int m0 = tm * BIG_BM;
  const int G = a.nfb * a.S;
  const int steps = a.Ks / 32;          // packed k-steps per split
  const int kk0 = yg * bg.cs * steps;   // first k-step of the group
  const int nst = bg.cs * steps / 2;    // stages of the group
  const int kx0 = yg * bg.cs * a.Ks;    // first k of the group

  bf16x8 wr[R][4], xr[R][4];
  auto load = [&](int st, bf16x8* w4, bf16x8* x4) {
    st = min(st, nst - 1);  // past the end: re-read the last stage (never used)
#pragma unroll
    for (int b = 0; b < 2; ++b) {
      const int kk = kk0 + 2 * st + b, y = kk / steps, j = kk - y * steps;
      const bf16_t* blk = a.W + ((size_t)j * G + (size_t)y * a.nfb + fbx) * 4096;
#pragma unroll
      for (int u = 0; u < 2; ++u) w4[b * 2 + u] = ld16(blk + (size_t)(tid + u * 256) * 8);
    }
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int pc = tid + u * 256, r = pc >> 3, o = pc & 7;
      x4[u] = ld16(a.X + (size_t)min(m0 + r, a.M - 1) * a.K + min(kx0 + st * BIG_KST + o * 8, a.K - 8));
    }
  };
  auto store = [&](int b, const bf16x8* w4, const bf16x8* x4) {
#pragma unroll
    for (int b2 = 0; b2 < 2; ++b2)
#pragma unroll
      for (int u = 0; u < 2; ++u) ws[b][b2 * 512 + tid + u * 256] = w4[b2 * 2 + u];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int pc = tid + u * 256, r = pc >> 3, o = pc & 7;
      *reinterpret_cast<bf16x8*>(&xs[b][r * BIG_XPAD + o * 8]) = x4[u];
    }
  };
  f32x16 acc[2][2];
#pragma unroll
  for (int tf = 0; tf < 2; ++tf)
#pragma unroll
    for (int tq = 0; tq < 2; ++tq)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[tf][tq][r] = 0.f;
  const int l32 = lane & 31, hi = lane >> 5;
  auto compute = [&](int b) {
#pragma unroll
    for (int h = 0; h < 4; ++h) {  // k 16h .. 16h + 16 of the stage
      const int blk = h >> 1, oct = 2 * (h & 1) + hi;
      bf16x8 af[2], bfr[2];
#pragma unroll
      for (int tf = 0; tf < 2; ++tf) {
        const int f = 64 * wf + 32 * tf + l32;  // feature inside the block
        af[tf] = ws[b][blk * 512 + (f >> 4) * 64 + oct * 16 + (f & 15)];
      }
#pragma unroll
      for (int tq = 0; tq < 2; ++tq) {
        const int r = 64 * wm + 32 * tq + l32;
        bfr[tq] = *reinterpret_cast<const bf16x8*>(&xs[b][r * BIG_XPAD + 16 * h + 8 * hi]);
      }
#pragma unroll
      for (int tf = 0; tf < 2; ++tf)
#pragma unroll
        for (int tq = 0; tq < 2; ++tq)
          acc[tf][tq] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[tf], bfr[tq], acc[tf][tq], 0, 0, 0);
    }
  };

  // Prologue: stages 0 .. R-1 in flight, stage 0 staged.
#pragma unroll
  for (int i = 0; i < R; ++i) load(i, wr[i], xr[i]);
  store(0, wr[0], xr[0]);
  load(R, wr[0], xr[0]);
  __syncthreads();
  // Stage st: multiply LDS buffer st&1, stage st+1 from its register set
  // into the other buffer (its loads were issued R - 1 stages ago), reload
  // that set with stage st+1+R, barrier.  Unrolled by R so the register sets
  // are fixed; iterations past nst only keep the barriers.
  for (int s0 = 0; s0 < nst; s0 += R) {
#pragma unroll
    for (int i = 0; i < R; ++i) {
      const int st = s0 + i;
      if (st < nst) compute(i & 1);
      store((i + 1) & 1, wr[(i + 1) % R], xr[(i + 1) % R]);
      load(st + 1 + R, wr[(i + 1) % R], xr[(i + 1) % R]);
      __syncthreads();
    }
  }

  float* out = a.P + (size_t)yg * a.slot_stride;
  const int n0 = fbx * 128;
#pragma unroll
  for (int tf = 0; tf < 2; ++tf)
#pragma unroll
    for (int tq = 0; tq < 2; ++tq) {
      const int m = m0 + 64 * wm + 32 * tq + l32;
      if (m >= a.M) continue;
#pragma unroll
      for (int g4 = 0; g4 < 4; ++g4) {
        const int n = n0 + 64 * wf + 32 * tf + 8 * g4 + 4 * hi;
        const f32x4 v = {acc[tf][tq][4 * g4], acc[tf][tq][4 * g4 + 1], acc[tf][tq][4 * g4 + 2],
                         acc[tf][tq][4 * g4 + 3]};
        if (n + 4 <= a.N && (a.N & 3) == 0) {
          *reinterpret_cast<f32x4*>(out + (size_t)m * a.N + n) = v;
        } else {
          for (int e = 0; e < 4; ++e)
            if (n + e < a.N) out[(size_t)m * a.N + n + e] = v[e];
        }
      }
    }
}

// float32 path (small models): one thread per output, sequential K order.
__global__ __launch_bounds__(64) void gemm_f32_kernel(const float* X, int M, int K, const float* W, int N,
                                                       float* P) {
  const int n = blockIdx.x * 64 + threadIdx.x;
  const int m = blockIdx.y;
  if (n >= N || m >= M) return;
  const float* wr = W + (size_t)n * K;
  const float* xr = X + (size_t)m * K;
  float acc = 0.f;
  for (int k = 0; k < K; ++k) acc = fmaf(xr[k], wr[k], acc);
  P[(size_t)m * N + n] = acc;
}

template <int MT, int NCH>
void launch_tiles(const GemmArgs& a, int depth, hipStream_t st) {
  if (depth == 2)
    hipLaunchKernelGGL((gemm_bf16_kernel<MT, NCH, 2>), dim3(a.ntiles), dim3(WAVES_PER_WG * 64), 0, st, a);
  else
    hipLaunchKernelGGL((gemm_bf16_kernel<MT, NCH, 4>), dim3(a.ntiles), dim3(WAVES_PER_WG * 64), 0, st, a);
}

template <int MT>
hipError_t launch_mt(GemmArgs a, const GemmPlan& p, int M, hipStream_t st) {
  a.nfb = (a.N + GROUP - 1) / GROUP;
  a.S = p.S;
  a.ntiles = a.nfb * p.S * ((M + 16 * MT - 1) / (16 * MT));
  switch (p.nch) {
    case 1: launch_tiles<MT, 1>(a, p.depth, st); break;
    case 2: launch_tiles<MT, 2>(a, p.depth, st); break;
    case 3: launch_tiles<MT, 3>(a, p.depth, st); break;
    case 4: launch_tiles<MT, 4>(a, p.depth, st); break;
    case 5: launch_tiles<MT, 5>(a, p.depth, st); break;
    case 6: launch_tiles<MT, 6>(a, p.depth, st); break;
    case 8: launch_tiles<MT, 8>(a, p.depth, st); break;
    default: return hipErrorInvalidValue;
  }
  return hipSuccess;
}

}  // namespace

// The plan depends only on (N, K), never on M, so that a row's result is the
// same whatever the number of rows in the launch.
GemmPlan gemm_plan(int N, int K, int dtype, bool unsplit) {
  GemmPlan p;
  if (dtype != TRI_BF16) {
    p.S = 1;
    p.Ks = K;
    p.nch = 1;
    return p;
  }
  // Target K per split, measured on MI355X for the 8B/14B decode shapes
  // (M = 32/33) with one workgroup per (128-feature block, K split): 512 for
  // the d x d projection, 1024 for QKV and the wide gate/up projection, 1536
  // for the long-K down projection; the lm_head (very wide N) runs unsplit.
  const int T = kpad(K) / KC;  // stages of the padded K
  int tgt;
  if (unsplit || N >= 65536)
    tgt = T;
  else if (K > 8192)
    tgt = 1536 / KC;
  else if (N > K)
    tgt = 1024 / KC;
  else
    tgt = 512 / KC;
  tgt = std::max(1, std::min(tgt, T));
  // Prefer a split count that divides the stages evenly, within a factor of
  // two of the target; otherwise every split is padded to the same length
  // with zero weights (the packed layout needs equal splits).
  const int S0 = std::min((T + tgt - 1) / tgt, MAX_S);
  int S = 0;
  for (int d = 0; d <= S0 && !S; ++d)
    for (int c : {S0 + d, S0 - d})
      if (!S && c >= 1 && c <= MAX_S && c <= 2 * S0 && 2 * c >= S0 && T % c == 0) S = c;
  if (!S) S = S0;
  const int ps = (T + S - 1) / S;  // stages per split
  p.S = (T + ps - 1) / ps;
  p.Ks = ps * KC;
  p.nch = 1;
  for (int c : {8, 6, 5, 4, 3, 2})
    if (ps % c == 0) {
      p.nch = c;
      break;
    }
  // W fragments in flight per wave: 2 k-steps for the wide gate/up shape,
  // 4 elsewhere (measured).
  p.depth = (!unsplit && N >= 16384) ? 2 : 4;
  return p;
}

size_t gemm_packed_bytes(const GemmPlan& p, int N, int K, int dtype) {
  if (dtype == TRI_BF16) return (size_t)((N + GROUP - 1) / GROUP) * GROUP * ((size_t)p.S * p.Ks) * 2;
  return (size_t)N * K * 4;
}

hipError_t launch_pack(int dtype, const WSeg* segs, int nseg, int N, int K, const GemmPlan& p, void* dst,
                       hipStream_t st) {
  const void* w0 = segs[0].ptr;
  const void* w1 = nseg > 1 ? segs[1].ptr : nullptr;
  const void* w2 = nseg > 2 ? segs[2].ptr : nullptr;
  const int r0 = segs[0].rows;
  const int r1 = nseg > 1 ? segs[1].rows : 0;
  if (dtype == TRI_BF16) {
    const size_t npieces = gemm_packed_bytes(p, N, K, dtype) / 16;
    hipLaunchKernelGGL(pack_bf16_kernel, dim3(2048), dim3(256), 0, st, static_cast<const bf16_t*>(w0),
                       static_cast<const bf16_t*>(w1), static_cast<const bf16_t*>(w2), r0, r1, N, K,
                       (N + GROUP - 1) / GROUP, p.S, p.Ks / 32, npieces, static_cast<bf16_t*>(dst));
  } else {
    hipLaunchKernelGGL(pack_f32_kernel, dim3(2048), dim3(256), 0, st, static_cast<const float*>(w0),
                       static_cast<const float*>(w1), static_cast<const float*>(w2), r0, r1, N, K,
                       static_cast<float*>(dst));
  }
  return hipGetLastError();
}

// Which kernel a bf16 GEMM of M rows runs on.  The decode kernel streams W
// once per 64-row tile; the large-M kernel once per launch but with fewer,
// fatter workgroups.  Measured on MI355X (8B shapes): the large-M kernel is
// faster from 65 rows for the wide (N >= 16K) and long-K (K >= 8K) shapes and
// from 256 rows for the others.
bool gemm_use_big(int M, int N, int K) { return M > 64 && (M >= 256 || N >= 16384 || K >= 8192); }

// Large-M grid: as few K-split groups (output slots) as keep >= 512
// workgroups in flight, otherwise one group per packed split.
static BigGrid big_grid(const GemmPlan& p, int M, int N) {
  BigGrid g;
  g.ntm = (M + BIG_BM - 1) / BIG_BM;
  const int nfb8 = ((N + GROUP - 1) / GROUP + 7) / 8 * 8;
  g.nyg = p.S;
  for (int c = 1; c <= p.S; ++c)
    if (p.S % c == 0 && nfb8 * g.ntm * c >= 512) {
      g.nyg = c;
      break;
    }
  g.cs = p.S / g.nyg;
  return g;
}

int gemm_out_slots(int dtype, const GemmPlan& p, int M, int N, int K) {
  if (dtype != TRI_BF16) return p.S;
  return gemm_use_big(M, N, K) ? big_grid(p, M, N).nyg : p.S;
}

hipError_t launch_gemm(int dtype, const void* X, int M, int K, const void* W, int N, const GemmPlan& plan, float* P,
                       size_t slot_stride, hipStream_t st) {
  if (M <= 0) return hipSuccess;
  if (dtype == TRI_BF16) {
    GemmArgs a;
    a.X = static_cast<const bf16_t*>(X);
    a.M = M;
    a.K = K;
    a.W = static_cast<const bf16_t*>(W);
    a.N = N;
    a.Ks = plan.Ks;
    a.P = P;
    a.slot_stride = slot_stride;
    if (gemm_use_big(M, N, K)) {
      a.S = plan.S;
      a.nfb = (N + GROUP - 1) / GROUP;
      const BigGrid g = big_grid(plan, M, N);
      a.ntiles = (a.nfb + 7) / 8 * 8 * g.ntm * g.nyg;
      hipLaunchKernelGGL((gemm_big_kernel<BIG_R>), dim3(a.ntiles), dim3(256), 0, st, a, g);
      return hipGetLastError();
    }
    const int mt = M >= 64 ? 4 : (M + 15) / 16;
    hipError_t e;
    switch (mt) {
      case 1: e = launch_mt<1>(a, plan, M, st); break;
      case 2: e = launch_mt<2>(a, plan, M, st); break;
      case 3: e = launch_mt<3>(a, plan, M, st); break;
      default: e = launch_mt<4>(a, plan, M, st); break;
    }
    if (e != hipSuccess) return e;
  } else {
    dim3 grid((N + 63) / 64, M);
    hipLaunchKernelGGL(gemm_f32_kernel, grid, dim3(64), 0, st, static_cast<const float*>(X), M, K,
                       static_cast<const float*>(W), N, P);
  }
  return hipGetLastError();
}

}  // namespace tri
