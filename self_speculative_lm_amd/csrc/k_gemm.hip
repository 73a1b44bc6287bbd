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
  bf16_t* H;  // SwiGLU epilogue output [M][N/2] (gate/up projection only)
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
// PACK_GATEUP: the two segments (gate and up, r0 rows each) interleave in
// groups of 16 rows: packed rows [32j, 32j+16) are segment 0's rows
// [16j, 16j+16) and [32j+16, 32j+32) segment 1's, so one MFMA fragment pair
// holds matching gate and up features.
__device__ __forceinline__ int pack_row(int row, int r0, int order) {
  if (order != PACK_GATEUP) return row;
  const int j = row >> 4, w = row & 15;
  return (j & 1) ? r0 + (j >> 1) * 16 + w : (j >> 1) * 16 + w;
}

__global__ void pack_bf16_kernel(const bf16_t* w0, const bf16_t* w1, const bf16_t* w2, int r0, int r1, int N,
                                 int K, int nfb, int S, int steps, size_t npieces, int il, bf16_t* dst) {
  const int G = nfb * S;
  for (size_t p = (size_t)blockIdx.x * blockDim.x + threadIdx.x; p < npieces;
       p += (size_t)gridDim.x * blockDim.x) {
    const size_t blk = p >> 9;
    const int w = (int)((p >> 6) & 7), lane = (int)(p & 63);
    const int j = (int)(blk / G), g = (int)(blk % G);
    const int x = g % nfb, y = g / nfb;
    const int prow = (x * 8 + w) * 16 + (lane & 15);
    const int k = (y * steps + j) * 32 + (lane >> 4) * 8;
    bf16x8 v = {};
    if (prow < N && k < K) {
      const int row = pack_row(prow, r0, il);
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
                                int il, float* dst) {
  const size_t n = (size_t)N * K;
  for (size_t p = (size_t)blockIdx.x * blockDim.x + threadIdx.x; p < n; p += (size_t)gridDim.x * blockDim.x) {
    const int prow = (int)(p / K);
    const size_t c = p - (size_t)prow * K;
    const int row = pack_row(prow, r0, il);
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

// Large-M grid: row tiles, K-split groups (one output slot each) and packed
// splits per group.
struct BigGrid {
  int ntm, nyg, cs;
  int fpw;  // feature fragments per wave (packed 128-feature blocks per workgroup = fpw)
};

// Large-M GEMM (prefill chunks and wide batches): the skinny kernel's
// structure with FPW feature fragments per wave, so that MFMA operands are
// reused in registers instead of re-read.  W fragments stream from HBM/L2
// straight into MFMA A operands (the packed layout is already in A order), a
// ring of D k-steps of them in flight per wave; X (MT row tiles of 16) is
// staged in LDS per 256-wide stage, double-buffered.  Every B fragment read
// from LDS feeds FPW MFMAs and every A fragment MT, so LDS carries one 1 KiB
// fragment per FPW MFMAs.  A workgroup of WAVES waves covers WAVES*FPW
// fragments (WAVES*FPW/8 packed blocks of 128 features) x MT*16 rows over a
// group of cs consecutive K splits (output slot yg); one pass covers a whole
// split (or an equal part of it) in straight-line code, so no fragment
// crosses a back-edge.  The workgroups of one feature group get ids
// congruent modulo 8, so they run on one XCD and share its L2 for W.
//
// CHAIN: each K split of the group is accumulated from zero and the splits'
// partials are added in split order in a second register set, which is
// exactly what a consumer does with one slot per split: the single slot then
// holds the decode kernel's bits (batch-invariant outputs in one slot).
//
// SWIGLU (gate/up projection, one slot): the packed features interleave gate
// and up fragments, so fragments 2j and 2j + 1 of a wave hold matching gate
// and up sums in the same lanes; the epilogue writes bf16(silu(g) * u) with
// the SwiGLU kernel's arithmetic instead of the float32 sums.
template <int MT, int NCH, int D, int FPW, int WAVES, bool CHAIN, bool SWIGLU = false>
__global__ __launch_bounds__(WAVES * 64) void gemm_wide_kernel(GemmArgs a, BigGrid bg) {
  constexpr int NT = WAVES * 64, NS = NCH * KSTEPS;
  constexpr int BPW = WAVES * FPW / 8;           // packed blocks per workgroup
  constexpr int XPIECES = MT * 16 * (KC / 8);    // 16-byte pieces of one X stage
  constexpr int XPT = XPIECES / NT;
  static_assert(XPIECES % NT == 0 && (WAVES * FPW) % 8 == 0 && 8 % FPW == 0, "shape");
  // Prefetch of LDS B fragments one k-step ahead: for the 128-row form only,
  // whose waves run two per SIMD anyway (the 64-row forms would lose their
  // second workgroup per CU: 118 -> 130 VGPRs).
  constexpr bool BPREF = MT >= 8;
  __shared__ bf16x8 xs[2][KSTEPS][MT][64];
  const int id = blockIdx.x;
  const int q = id >> 3, per = bg.ntm * bg.nyg;
  const int fgx = (q / per) * 8 + (id & 7), rem = q - (q / per) * per;  // feature group (BPW blocks)
  const int tm = rem % bg.ntm, yg = rem / bg.ntm;
  if (fgx * BPW >= a.nfb) return;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int G = a.nfb * a.S;
  const int m0 = tm * (MT * 16);
  const int blkx = fgx * BPW + (wave * FPW) / 8;  // this wave's packed block
  const int fg0 = (wave * FPW) % 8;               // its first fragment in the block
  const bool wvalid = blkx < a.nfb;
  const int bx = wvalid ? blkx : a.nfb - 1;       // clamped: loads stay inside W
  const size_t wstep = (size_t)G * 4096;          // elements between k-steps
  const int npass_split = a.Ks / (NCH * KC);

  const bf16_t* xrow[XPT];
  int xk[XPT];
#pragma unroll
  for (int it = 0; it < XPT; ++it) {
    const int i = tid + it * NT;
    const int gg = i & 3, r = (i >> 2) % (MT * 16), s = (i >> 2) / (MT * 16);
    xrow[it] = a.X + (size_t)min(m0 + r, a.M - 1) * a.K;
    xk[it] = s * 32 + gg * 8;
  }
  f32x4 acc[FPW][MT];
  f32x4 tot[CHAIN ? FPW : 1][CHAIN ? MT : 1];
#pragma unroll
  for (int f = 0; f < FPW; ++f)
#pragma unroll
    for (int t = 0; t < MT; ++t) acc[f][t] = f32x4{0.f, 0.f, 0.f, 0.f};

  for (int pp = 0; pp < bg.cs * npass_split; ++pp) {
    const int y = yg * bg.cs + pp / npass_split, p = pp % npass_split;
    if (CHAIN && pp > 0 && p == 0) {  // split y - 1 is complete: add its partial in split order
#pragma unroll
      for (int f = 0; f < FPW; ++f)
#pragma unroll
        for (int t = 0; t < MT; ++t) {
          tot[CHAIN ? f : 0][CHAIN ? t : 0] = pp == npass_split ? acc[f][t] : tot[CHAIN ? f : 0][CHAIN ? t : 0] + acc[f][t];
          acc[f][t] = f32x4{0.f, 0.f, 0.f, 0.f};
        }
    }
    const int k0 = y * a.Ks + p * (NCH * KC);
    const bf16_t* wp = a.W + ((size_t)(p * NS) * G + (size_t)y * a.nfb + bx) * 4096 + fg0 * 512 + lane * 8;
    bf16x8 ring[D][FPW], xr[XPT];
    auto load_x = [&](int c) {
#pragma unroll
      for (int it = 0; it < XPT; ++it) xr[it] = ld16(xrow[it] + min(k0 + c * KC + xk[it], a.K - 8));
    };
    auto store_x = [&](int b) {
#pragma unroll
      for (int it = 0; it < XPT; ++it) {
        const int i = tid + it * NT;
        const int gg = i & 3, r = (i >> 2) % (MT * 16), s = (i >> 2) / (MT * 16);
        xs[b][s][r >> 4][gg * 16 + (r & 15)] = xr[it];
      }
    };
    if (pp > 0) __syncthreads();  // the previous pass's last stage still reads xs
    load_x(0);
#pragma unroll
    for (int i = 0; i < D; ++i)
#pragma unroll
      for (int f = 0; f < FPW; ++f) ring[i][f] = ld16(wp + (size_t)i * wstep + f * 512);
    store_x(0);
    __syncthreads();
#pragma unroll
    for (int c = 0; c < NCH; ++c) {
      if (c + 1 < NCH) load_x(c + 1);
      // BPREF: the B fragments of the stage's next k-step are read from LDS
      // before the MFMAs of this one, so their latency hides behind them.
      bf16x8 bcur[MT];
      if constexpr (BPREF) {
#pragma unroll
        for (int t = 0; t < MT; ++t) bcur[t] = xs[c & 1][0][t][lane];
      }
#pragma unroll
      for (int s = 0; s < KSTEPS; ++s) {
        const int j = c * KSTEPS + s;
        bf16x8 bnext[MT];
        if constexpr (BPREF) {
          if (s + 1 < KSTEPS) {
#pragma unroll
            for (int t = 0; t < MT; ++t) bnext[t] = xs[c & 1][s + 1][t][lane];
          }
        }
#pragma unroll
        for (int t = 0; t < MT; ++t) {
          const bf16x8 bv = BPREF ? bcur[t] : xs[c & 1][s][t][lane];
#pragma unroll
          for (int f = 0; f < FPW; ++f)
            acc[f][t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ring[j % D][f], bv, acc[f][t], 0, 0, 0);
        }
        if (j + D < NS) {
#pragma unroll
          for (int f = 0; f < FPW; ++f) ring[j % D][f] = ld16(wp + (size_t)(j + D) * wstep + f * 512);
        }
        __builtin_amdgcn_sched_barrier(0);
        if constexpr (BPREF) {
          if (s + 1 < KSTEPS) {
#pragma unroll
            for (int t = 0; t < MT; ++t) bcur[t] = bnext[t];
          }
        }
      }
      if (c + 1 < NCH) {
        store_x((c + 1) & 1);
        __syncthreads();
      }
    }
  }
  if (!wvalid) return;
  if (CHAIN && bg.cs > 1) {
#pragma unroll
    for (int f = 0; f < FPW; ++f)
#pragma unroll
      for (int t = 0; t < MT; ++t) acc[f][t] = tot[CHAIN ? f : 0][CHAIN ? t : 0] + acc[f][t];
  }
  if constexpr (SWIGLU) {
    static_assert(FPW % 2 == 0, "gate/up fragment pairs");
    const int ffn = a.N >> 1;
#pragma unroll
    for (int f = 0; f < FPW; f += 2) {
      const int col = ((blkx * 8 + fg0 + f) >> 1) * 16 + 4 * (lane >> 4);
#pragma unroll
      for (int t = 0; t < MT; ++t) {
        const int m = m0 + t * 16 + (lane & 15);
        if (m >= a.M || col >= ffn) continue;
        f32x4 o;
#pragma unroll
        for (int e = 0; e < 4; ++e) o[e] = acc[f][t][e] / (1.0f + expf(-acc[f][t][e])) * acc[f + 1][t][e];
        Elem<bf16_t>::store4(a.H, (size_t)m * ffn + col, o);
      }
    }
    return;
  }
  // D layout: lane l holds D[4*(l/16) + r][l%16] = Y[m0 + 16t + l%16][n + 4*(l/16) + r]
  float* out = a.P + (size_t)yg * a.slot_stride;
#pragma unroll
  for (int f = 0; f < FPW; ++f) {
    const int nn = blkx * 128 + (fg0 + f) * 16 + 4 * (lane >> 4);
#pragma unroll
    for (int t = 0; t < MT; ++t) {
      const int m = m0 + t * 16 + (lane & 15);
      if (m >= a.M) continue;
      if (nn + 4 <= a.N && (a.N & 3) == 0) {
        *reinterpret_cast<f32x4*>(out + (size_t)m * a.N + nn) = acc[f][t];
      } else {
        for (int r = 0; r < 4; ++r)
          if (nn + r < a.N) out[(size_t)m * a.N + nn + r] = acc[f][t][r];
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
                       int interleave, hipStream_t st) {
  if (interleave == PACK_GATEUP && (nseg != 2 || segs[0].rows != segs[1].rows || segs[0].rows % 16))
    return hipErrorInvalidValue;
  const void* w0 = segs[0].ptr;
  const void* w1 = nseg > 1 ? segs[1].ptr : nullptr;
  const void* w2 = nseg > 2 ? segs[2].ptr : nullptr;
  const int r0 = segs[0].rows;
  const int r1 = nseg > 1 ? segs[1].rows : 0;
  if (dtype == TRI_BF16) {
    const size_t npieces = gemm_packed_bytes(p, N, K, dtype) / 16;
    hipLaunchKernelGGL(pack_bf16_kernel, dim3(2048), dim3(256), 0, st, static_cast<const bf16_t*>(w0),
                       static_cast<const bf16_t*>(w1), static_cast<const bf16_t*>(w2), r0, r1, N, K,
                       (N + GROUP - 1) / GROUP, p.S, p.Ks / 32, npieces, interleave, static_cast<bf16_t*>(dst));
  } else {
    hipLaunchKernelGGL(pack_f32_kernel, dim3(2048), dim3(256), 0, st, static_cast<const float*>(w0),
                       static_cast<const float*>(w1), static_cast<const float*>(w2), r0, r1, N, K, interleave,
                       static_cast<float*>(dst));
  }
  return hipGetLastError();
}

// Which kernel a bf16 GEMM of M rows runs on.  The decode kernel streams W
// once per 64-row tile; the large-M kernel once per 64-row tile too (once for
// all rows in its 128-row form), but its waves hold several fragments, so
// each W and X fragment feeds several MFMAs.  Measured on MI355X (8B shapes):
// the large-M kernel is faster from 65 rows for the wide (N >= 16K) and
// long-K (K >= 8K) shapes and from 192 rows for the others (decode forwards
// of 224 / 255 rows 9.55 / 9.85 -> 9.29 / 9.56 ms; at 129 rows QKV and o_proj
// on it were slower).
bool gemm_use_big(int M, int N, int K) { return M > 64 && (M >= 192 || N >= 16384 || K >= 8192); }

// Large-M form: 8 waves x 2 or 4 fragments (256 or 512 features) x 4 row
// tiles (64 rows), 4 k-steps in flight.  With two fragments a wave stays
// under 128 VGPRs, so two workgroups share a CU (their 64 KB X tiles fit its
// LDS); with four (~180 VGPRs) one workgroup runs per CU but stages each X
// tile for twice the features.  The chained form (one slot for all K splits)
// keeps a running total per fragment, which takes the two-fragment wave to
// 146 VGPRs: one workgroup per CU either way, so there four fragments win.
// big_grid picks per launch.  Measured on MI355X: the 511-row prefill chunk
// 12.9 -> 11.9 ms with two fragments; 8B-class decode forwards of 256 rows
// 10.25 -> 9.42 ms with four.  Four row tiles of 128 rows or two of 32 were
// slower.
constexpr int BIGM_MT = 4, BIGM_D = 4, BIGM_WAVES = 8;
// Tall form for 65..128 rows: one 128-row tile (8 row tiles) x 1 fragment
// per wave, so W is streamed once for all the rows instead of once per
// 64-row tile.  Its per-split partials have the same bits as the other
// forms (same MFMA, same k order per element).  One fragment per wave
// (128 features per workgroup) rather than two: its X tiles fill a CU's LDS,
// so one workgroup runs per CU, and with two fragments the 8B gate/up
// projection of a decode forward needed 384 workgroups (a second, half-empty
// round); with one it is 192 workgroups chaining all four K splits into one
// slot, which the SwiGLU kernel then reads instead of four.  Measured on
// MI355X, 8B-class diffusion at 4 sequences (128-row forwards): 7.54 ->
// 6.89 ms per forward.
constexpr int TALL_MT = 8, TALL_FPW = 1;
__host__ __forceinline__ bool big_tall(int M) { return M <= TALL_MT * 16; }

// Large-M grid: as few K-split groups (output slots) as keep >= 192
// workgroups in flight, otherwise one group per packed split.  With
// `invariant` a row's result must not depend on how many rows share the
// launch: each split's partial is bit-identical to the decode kernel's (same
// MFMA, same k order from a zero accumulator) and consumers add slots in
// order, so either one slot per split, or one slot for all splits with the
// partials chained in split order (CHAIN); groups of some splits would add
// in a different order.
static BigGrid big_grid_for(const GemmPlan& p, int M, int N, bool invariant, int fpw) {
  BigGrid g;
  const int rows = big_tall(M) ? TALL_MT * 16 : BIGM_MT * 16, bpw = BIGM_WAVES * fpw / 8;
  g.fpw = fpw;
  g.ntm = (M + rows - 1) / rows;
  const int nfg8 = (((N + GROUP - 1) / GROUP + bpw - 1) / bpw + 7) / 8 * 8;
  g.nyg = p.S;
  for (int c = 1; c <= p.S; ++c)
    if (p.S % c == 0 && nfg8 * g.ntm * c >= 192) {
      g.nyg = c;
      break;
    }
  if (invariant && g.nyg != 1) g.nyg = p.S;
  g.cs = p.S / g.nyg;
  return g;
}

// Fragments per wave of a large-M launch.  One for the 128-row form.  Two
// where the split count is free (prefill chunks): two workgroups per CU and
// the fewest slots.  Under `invariant`: the fewer output slots first (two
// fragments can chain all K splits into one slot where four cannot; the
// consumer kernels then read one slot instead of one per split), then the
// lighter load on the busiest CU, in two-fragment workgroups' worth of work:
// a four-fragment workgroup counts 2, a two-fragment one 1, and a chained
// two-fragment one 1.25 (its running totals take a wave to 146 VGPRs, so it
// runs alone on its CU with half the waves in flight of two unchained ones).
// Ties take four fragments, which stage each X tile for twice the features.
// Fitted to 8B-class decode forwards of 256 to 2112 rows on MI355X (the
// factor 1.25 is the one value between 1.2 and 1.33 that orders all of them).
static double big_load(const BigGrid& g, int nfb) {
  const int bpw = BIGM_WAVES * g.fpw / 8;
  const long n = (long)((nfb + bpw - 1) / bpw + 7) / 8 * 8 * g.ntm * g.nyg;
  const double per_cu = (double)((n + 255) / 256);
  if (g.fpw == 4) return 2.0 * per_cu;
  return g.cs > 1 ? 1.25 * per_cu : per_cu;
}

static BigGrid big_grid(const GemmPlan& p, int M, int N, bool invariant) {
  if (big_tall(M)) return big_grid_for(p, M, N, invariant, TALL_FPW);
  const BigGrid g2 = big_grid_for(p, M, N, invariant, 2);
  if (!invariant) return g2;
  const BigGrid g4 = big_grid_for(p, M, N, invariant, 4);
  if (g2.nyg != g4.nyg) return g2.nyg < g4.nyg ? g2 : g4;
  const int nfb = (N + GROUP - 1) / GROUP;
  return big_load(g2, nfb) < big_load(g4, nfb) ? g2 : g4;
}

template <int MT, int NCH, int FPW>
void launch_wide_form(const GemmArgs& a, const BigGrid& g, bool chain, bool swiglu, hipStream_t st) {
  const dim3 grid(a.ntiles), block(BIGM_WAVES * 64);
  // the SwiGLU epilogue pairs fragments: forms of one fragment per wave never
  // take it (gemm_swiglu_fused says so)
  constexpr bool SW = FPW % 2 == 0;
  if (chain && swiglu && SW)
    hipLaunchKernelGGL((gemm_wide_kernel<MT, NCH, BIGM_D, FPW, BIGM_WAVES, true, SW>), grid, block, 0, st, a, g);
  else if (chain)
    hipLaunchKernelGGL((gemm_wide_kernel<MT, NCH, BIGM_D, FPW, BIGM_WAVES, true>), grid, block, 0, st, a, g);
  else if (swiglu && SW)
    hipLaunchKernelGGL((gemm_wide_kernel<MT, NCH, BIGM_D, FPW, BIGM_WAVES, false, SW>), grid, block, 0, st, a, g);
  else
    hipLaunchKernelGGL((gemm_wide_kernel<MT, NCH, BIGM_D, FPW, BIGM_WAVES, false>), grid, block, 0, st, a, g);
}

template <int NCH>
void launch_wide(const GemmArgs& a, const BigGrid& g, bool chain, bool swiglu, bool tall, hipStream_t st) {
  if (tall)
    launch_wide_form<TALL_MT, NCH, TALL_FPW>(a, g, chain, swiglu, st);
  else if (g.fpw == 4)
    launch_wide_form<BIGM_MT, NCH, 4>(a, g, chain, swiglu, st);
  else
    launch_wide_form<BIGM_MT, NCH, 2>(a, g, chain, swiglu, st);
}

// Passes of the large-M kernel as long as possible: the largest NCH <= 8
// dividing the stages per split (one pass per split for every 8B/14B
// projection plan).
static int wide_nch(const GemmPlan& plan) {
  const int ps = plan.Ks / KC;
  for (int c : {8, 6, 5, 4, 3, 2})
    if (ps % c == 0) return c;
  return 1;
}

int gemm_out_slots(int dtype, const GemmPlan& p, int M, int N, int K, bool invariant) {
  if (dtype != TRI_BF16) return p.S;
  return gemm_use_big(M, N, K) ? big_grid(p, M, N, invariant).nyg : p.S;
}

bool gemm_swiglu_fused(int dtype, const GemmPlan& p, int M, int N, int K, bool invariant) {
  if (dtype != TRI_BF16 || !gemm_use_big(M, N, K)) return false;
  const BigGrid g = big_grid(p, M, N, invariant);
  return g.fpw % 2 == 0 && g.nyg == 1;
}

hipError_t launch_gemm(int dtype, const void* X, int M, int K, const void* W, int N, const GemmPlan& plan, float* P,
                       size_t slot_stride, bool invariant, hipStream_t st, void* swiglu_out) {
  if (M <= 0) return hipSuccess;
  if (swiglu_out && !gemm_swiglu_fused(dtype, plan, M, N, K, invariant)) return hipErrorInvalidValue;
  if (dtype == TRI_BF16) {
    GemmArgs a;
    a.H = static_cast<bf16_t*>(swiglu_out);
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
      const BigGrid g = big_grid(plan, M, N, invariant);
      const bool tall = big_tall(M);
      const int bpw = BIGM_WAVES * g.fpw / 8;
      a.ntiles = ((a.nfb + bpw - 1) / bpw + 7) / 8 * 8 * g.ntm * g.nyg;
      const int nch = wide_nch(plan);
      const bool chain = invariant && g.cs > 1, sw = swiglu_out != nullptr;
      switch (nch) {
        case 1: launch_wide<1>(a, g, chain, sw, tall, st); break;
        case 2: launch_wide<2>(a, g, chain, sw, tall, st); break;
        case 3: launch_wide<3>(a, g, chain, sw, tall, st); break;
        case 4: launch_wide<4>(a, g, chain, sw, tall, st); break;
        case 5: launch_wide<5>(a, g, chain, sw, tall, st); break;
        case 6: launch_wide<6>(a, g, chain, sw, tall, st); break;
        case 8: launch_wide<8>(a, g, chain, sw, tall, st); break;
        default: return hipErrorInvalidValue;
      }
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

// One past the highest packed W element that launch_gemm's kernel reads for
// these arguments: both kernels' address arithmetic (block j*G + g of the
// step-major layout, the wave's fragment, lane 63's 8 elements, the last
// ring refill of the last pass) evaluated on the host over every workgroup
// and wave of the launch grid.  The packed matrix holds
// gemm_packed_bytes / 2 elements; 0 for float32 models.
size_t gemm_w_reach(int dtype, const GemmPlan& plan, int M, int N, int K, bool invariant) {
  if (dtype != TRI_BF16 || M <= 0) return 0;
  const int nfb = (N + GROUP - 1) / GROUP, G = nfb * plan.S;
  const size_t wstep = (size_t)G * (WAVES_PER_WG * 512);
  size_t reach = 0;
  if (gemm_use_big(M, N, K)) {
    const BigGrid bg = big_grid(plan, M, N, invariant);
    const int FPW = bg.fpw, BPW = BIGM_WAVES * FPW / 8;
    const int nch = wide_nch(plan), NS = nch * KSTEPS, npass_split = plan.Ks / (nch * KC);
    const long ntiles = (long)((nfb + BPW - 1) / BPW + 7) / 8 * 8 * bg.ntm * bg.nyg;
    for (long id = 0; id < ntiles; ++id) {
      const long q = id >> 3, per = (long)bg.ntm * bg.nyg;
      const long fgx = (q / per) * 8 + (id & 7), rem = q - (q / per) * per;
      if (fgx * BPW >= nfb) continue;
      const int yg = (int)(rem / bg.ntm);
      for (int wave = 0; wave < BIGM_WAVES; ++wave) {
        const long blkx = fgx * BPW + (wave * FPW) / 8;
        const long bx = blkx < nfb ? blkx : nfb - 1;
        const int fg0 = (wave * FPW) % 8;
        for (int pp = 0; pp < bg.cs * npass_split; ++pp) {
          const int y = yg * bg.cs + pp / npass_split, p = pp % npass_split;
          const size_t base = ((size_t)(p * NS) * G + (size_t)y * nfb + bx) * 4096 + fg0 * 512 + 63 * 8;
          reach = std::max(reach, base + (size_t)(NS - 1) * wstep + (FPW - 1) * 512 + 8);
        }
      }
    }
  } else {
    const int mt = M >= 64 ? 4 : (M + 15) / 16;
    const int NS = plan.nch * KSTEPS, npass = plan.Ks / (plan.nch * KC);
    const long ntiles = (long)G * ((M + 16 * mt - 1) / (16 * mt));
    for (long b = 0; b < ntiles; ++b) {
      const int g = (int)(b % G);
      for (int wave = 0; wave < WAVES_PER_WG; ++wave)
        for (int p = 0; p < npass; ++p) {
          const size_t base = (size_t)g * (WAVES_PER_WG * 512) + wave * 512 + 63 * 8 + (size_t)p * NS * wstep;
          reach = std::max(reach, base + (size_t)(NS - 1) * wstep + 8);
        }
    }
  }
  return reach;
}

}  // namespace tri
