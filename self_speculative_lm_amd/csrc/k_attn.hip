// Block-causal grouped-query attention over the KV cache.
//
// Every query row r attends to keys [0, hi[r]) of its sequence: a clean row at
// position p has hi = p + 1 (causal), a row of the noisy block [L, L + B) has
// hi = L + B (bidirectional inside the block, causal over the prefix)
// [Notes §3.2; Digest, Method].  Query head h reads kv head h / (hq / hkv).
//
// bf16 kernel (gfx950 MFMA): one workgroup per (split of kv_split keys,
// group of query vectors, sequence x kv head).  All query heads of a kv head
// share the K/V tiles, so K [64 keys][128] and V^T [128][64 keys] tiles are
// staged in LDS (V is cached transposed, so both tiles are contiguous 16-byte
// loads) and read by every wave that needs them.  The waves form two key
// groups that walk alternate tiles of the split, each with its own
// double-buffered tiles, and are merged through LDS at the end.  Tile loads
// are unconditional (a tile never crosses the cache capacity; keys past a
// row's limit are masked through their scores, and V past the last valid key
// is zeroed when staged).  Each wave owns QT tiles of 16 query vectors and
// computes S^T = K Q^T with v_mfma_f32_16x16x32_bf16, reading every K and V
// fragment from LDS once for its QT query tiles.  The K rows fed to the MFMA
// are permuted so that a lane ends up holding 8 scores of one query for 8
// consecutive keys: the softmax row statistics then need only two cross-lane
// steps, and the same registers, rounded to fp16, are directly the B operand
// of O^T = V^T P^T (no LDS round trip for P).  P.V runs in fp16 (V converted
// from bf16 when staged, exact inside the fp16 range and saturated at
// +-65504): P keeps 11 significant bits instead of bf16's 8, which measurably
// moved the logits of 4096-wide models.  Online softmax in float32 (exp2 with
// the scale folded in, a lazily moved maximum, masks only on tiles that cross
// a query's limit).  Splits write unnormalised partials (O, m, l) that a
// combine kernel merges in split order; a launch with a single split
// normalises in place.  A row's result depends only on its own q, its keys
// and kv_split, not on the other rows of the launch.
#include <math.h>

#include <algorithm>
#include <cmath>

#include "tri_common.h"

namespace tri {
namespace {

typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));

constexpr int HD = 128;
constexpr int KT = 64;
constexpr int KPAD = HD + 8;  // LDS row stride (elements) of the K tile
constexpr int VPAD = KT + 8;  // LDS row stride (elements) of the V^T tile

// The first 32 bytes hold what the prologue needs before anything else (one
// scalar load), so the sequence lookups follow it directly.
struct AttnArgs {
  const int32_t* seq_start;
  const int32_t* slot_seq;
  const int32_t* row_hi;
  int hq, hkv;
  const bf16_t* q;
  const bf16_t* kc;
  const bf16_t* vc;
  int rows, ctx, kv_split, nsplit;
  float scale_log2;
  bf16_t* out;
  float* part_o;   // [nsplit][rows][hq][HD]
  float* part_ml;  // [nsplit][rows][hq][2]
  int qgroups, nz;  // query groups per (split, sequence x kv head); n_seq * hkv
  int force_part;   // write partials even with one split (a combine follows)
  // Compacted grid (NULL: every sequence gets qgroups query groups): entry w
  // = slot * 65536 + query group, only the groups that hold query vectors;
  // workgroup id = (w * hkv + kv head) * nsplit + split.
  const int32_t* work;
  int nwork;
};

__device__ __forceinline__ bf16x8 ld16(const bf16_t* p) {
  return *reinterpret_cast<const bf16x8*>(p);
}

// Cross-lane reductions without an LDS round trip.  v_permlane16_swap
// (v_permlane32_swap) exchanges the odd 16-lane rows (the upper 32 lanes) of
// one register with the even rows (the lower 32 lanes) of another; fed the same
// value twice, the two results of lane l are x[l] and x[l ^ 16] (x[l ^ 32]).
__device__ __forceinline__ float max_xor16(float x) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float max_xor32(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float sum_xor16(float x) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
__device__ __forceinline__ float sum_xor32(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// A workgroup has KW key groups of QW waves.  Every wave of a key group owns
// QT tiles of 16 query vectors (the query slots are the same in every key
// group); key group kg handles the tiles kg, kg + KW, kg + 2 KW, ... of the
// split, with its own double-buffered LDS tiles staged by its own waves, and
// the key groups' (m, l, O) are merged through LDS at the end (exactly: a key
// group without a valid key contributes with weight exp2(-1e30 - M) = 0).
// The tile order inside a key group, and so every rounding, depends only on
// kv_split and KW, never on the other rows of the launch.
// VF16: the V cache already holds the fp16 form of every element (the
// session writes it so), and staging copies the bits.
template <int QW, int KW, int QT, bool VF16 = false>
__global__ __launch_bounds__(QW * KW * 64) void attn_bf16_kernel(AttnArgs a) {
  constexpr int GTH = QW * 64;         // threads of a key group
  constexpr int PIECES = KT * HD / 8;  // 16-byte pieces of one K (or V^T) tile
  constexpr int PPT = PIECES / GTH;    // per thread
  static_assert(PIECES % GTH == 0, "every thread stages the same number of pieces");
  __shared__ __attribute__((aligned(16))) bf16_t ks[KW * 2][KT * KPAD];
  __shared__ __attribute__((aligned(16))) _Float16 vs[KW * 2][HD * VPAD];  // V^T tiles in fp16
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int kg = wave / QW, qs = wave - kg * QW;  // key group, query slot
  const int tg = tid - kg * GTH;                  // thread index inside the key group
  // Workgroup id -> (split bx, query group bq, sequence x kv head bz).  The
  // query groups of one (split, kv head) get ids 8 apart, so they run on one
  // XCD one after the other and the later ones find the K/V tiles in its L2.
  int bq, bx, seq, kvh;
  if (a.work) {
    // compacted grid: the query groups of one (slot, kv head, split) are
    // hkv * nsplit ids apart (a multiple of 8 for 8 kv heads: one XCD)
    const int id = (int)blockIdx.x;
    bx = id % a.nsplit;
    const int t = id / a.nsplit;
    kvh = t % a.hkv;
    const int e = a.work[t / a.hkv];
    seq = e >> 16;
    bq = e & 0xffff;
  } else {
    const int per = 8 * a.qgroups;
    const int pr = ((int)blockIdx.x / per) * 8 + ((int)blockIdx.x & 7);
    if (pr >= a.nsplit * a.nz) return;
    bq = ((int)blockIdx.x % per) >> 3;
    bx = pr % a.nsplit;
    const int bz = pr / a.nsplit;
    seq = bz / a.hkv;
    kvh = bz - seq * a.hkv;
  }
  const int G = a.hq / a.hkv;
  const int cseq = a.slot_seq ? a.slot_seq[seq] : seq;
  const int r0 = a.seq_start[seq];
  const int nq = (a.seq_start[seq + 1] - r0) * G;
  const int qbase = bq * (QW * 16 * QT);
  if (qbase >= nq) return;
  const int kbeg = bx * a.kv_split;
  const bf16_t* kbase = a.kc + (size_t)(cseq * a.hkv + kvh) * a.ctx * HD;
  const bf16_t* vbase = a.vc + (size_t)(cseq * a.hkv + kvh) * HD * a.ctx;

  // Tile staging: registers <- global (whole 64-key tiles, clamped inside the
  // cache capacity), then LDS.
  auto load_tile = [&](int t0, bf16x8* kr, bf16x8* vr) {
    t0 = min(t0, a.ctx - KT);
#pragma unroll
    for (int u = 0; u < PPT; ++u) {
      const int i = tg + u * GTH;
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
      const int i = tg + u * GTH;
      *reinterpret_cast<bf16x8*>(&ks[b][(i >> 4) * KPAD + (i & 15) * 8]) = kr[u];
      f16x8 vv;
      if constexpr (VF16) {
        vv = __builtin_bit_cast(f16x8, vr[u]);
      } else {
#pragma unroll
        for (int e = 0; e < 8; ++e) vv[e] = (_Float16)fminf(fmaxf((float)vr[u][e], -65504.f), 65504.f);
      }
      if (vlim < KT) {
#pragma unroll
        for (int e = 0; e < 8; ++e)
          if ((i & 7) * 8 + e >= vlim) vv[e] = (_Float16)0.0f;
      }
      *reinterpret_cast<f16x8*>(&vs[b][(i >> 3) * VPAD + (i & 7) * 8]) = vv;
    }
  };

  // 1. Loads, in the order their results are needed: the key limits of the
  //    workgroup's rows (every wave reads all of them, lane-strided, so the
  //    key range needs no LDS or barrier), each lane's own query limits, the
  //    key group's first tile (a tile past the split's end re-reads a
  //    clamped tile and is never used) and the queries.
  constexpr int QV = QW * 16 * QT;        // query vectors of a workgroup
  constexpr int NRL = QV / 64 + 1;        // >= rows they span / 64
  const int qend = min(nq, qbase + QV);
  const int rw0 = qbase / G, nrw = (qend - 1) / G - rw0 + 1;
  int rh[NRL];
#pragma unroll
  for (int i = 0; i < NRL; ++i) rh[i] = a.row_hi[r0 + rw0 + min(lane + 64 * i, nrw - 1)];
  const int j = lane & 15, g = lane >> 4;
  // Query vector v of the sequence is (row r0 + v / G, head kvh * G + v % G).
  auto qrow = [&](int q) {
    const int v = qbase + (qs * QT + q) * 16 + j;
    return v < nq ? r0 + v / G : r0;
  };
  auto qhead = [&](int q) {
    const int v = qbase + (qs * QT + q) * 16 + j;
    return kvh * G + (v < nq ? v % G : 0);
  };
  bool valid[QT];
  int rhi[QT];
#pragma unroll
  for (int q = 0; q < QT; ++q) {
    valid[q] = qbase + (qs * QT + q) * 16 + j < nq;
    rhi[q] = a.row_hi[qrow(q)];
  }
  __builtin_amdgcn_sched_barrier(0);
  bf16x8 ka[PPT], va[PPT];
  load_tile(kbeg + kg * KT, ka, va);
  bf16x8 qf[QT][4];
#pragma unroll
  for (int q = 0; q < QT; ++q) {
    const bf16_t* qp = a.q + ((size_t)qrow(q) * a.hq + qhead(q)) * HD + g * 8;
#pragma unroll
    for (int ds = 0; ds < 4; ++ds) qf[q][ds] = ld16(qp + ds * 32);
  }
  __builtin_amdgcn_sched_barrier(0);

  // 2. Key range of this workgroup: up to the largest limit of its rows.
  int myhi = rh[0];
#pragma unroll
  for (int i = 1; i < NRL; ++i) myhi = max(myhi, rh[i]);
  const int wg_hi = __builtin_amdgcn_readfirstlane(wave_max_i32(myhi));
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
  // Wave-uniform facts: whether the wave holds any valid query, and the
  // smallest key limit of its valid queries (tiles that end at or below it
  // need no mask).
  int wmin = 0x7fffffff;
  bool any_valid = false;
#pragma unroll
  for (int q = 0; q < QT; ++q) {
    if (valid[q]) wmin = min(wmin, lim[q]);
    any_valid |= valid[q];
  }
  wmin = __builtin_amdgcn_readfirstlane(wave_min_i32(wmin));
  const bool wave_active = __builtin_amdgcn_ballot_w64(any_valid) != 0;

  // One 64-key tile from LDS buffer b starting at key t0.
  //
  // The running maximum is lazy: the exponent base m_run moves (and O, l are
  // rescaled) only when a score exceeds it by more than RESCALE (log2 units),
  // so P = exp2(s * scale - m_run) <= 2^RESCALE.  O and l stay relative to
  // the same m_run, so the normalised result is the same function; P keeps
  // fp16's 11 significant bits at any magnitude below 65504.
  constexpr float RESCALE = 8.f;
  auto compute = [&](int b, int t0) {
    // S^T tile t of key group m: MFMA row i loads key 32m + 8(i/4) + 4t + i%4,
    // so output lane (j, g) gets keys 32m + 8g + (4t + r) of query j.
    float sc[QT][2][8];
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
        for (int q = 0; q < QT; ++q)
#pragma unroll
          for (int r = 0; r < 4; ++r) sc[q][m][4 * t + r] = s[q][r];
      }
    }
    if (t0 + KT > wmin) {  // a tile that crosses some valid query's limit
#pragma unroll
      for (int q = 0; q < QT; ++q)
#pragma unroll
        for (int m = 0; m < 2; ++m)
#pragma unroll
          for (int e = 0; e < 8; ++e)
            if (t0 + 32 * m + 8 * g + e >= lim[q]) sc[q][m][e] = -INFINITY;
    }
    // Raw-score maxima (scale > 0, so the scaled maximum is the maximum
    // scaled), then one wave-uniform decision whether any base must move.
    float mcand[QT];
    bool need[QT], any_need = false;
#pragma unroll
    for (int q = 0; q < QT; ++q) {
      float tm = sc[q][0][0];
#pragma unroll
      for (int e = 1; e < 16; ++e) tm = fmaxf(tm, sc[q][e >> 3][e & 7]);
      tm = max_xor32(max_xor16(tm));
      mcand[q] = tm * a.scale_log2;
      need[q] = mcand[q] > m_run[q] + RESCALE;
      any_need |= need[q];
    }
    // Only the queries that need it move their base (alpha = 1 exactly for
    // the others), so a query's result does not depend on its wave mates.
    if (__builtin_amdgcn_ballot_w64(any_need) != 0) {
#pragma unroll
      for (int q = 0; q < QT; ++q) {
        const float m_new = need[q] ? mcand[q] : m_run[q];
        const float alpha = __builtin_amdgcn_exp2f(m_run[q] - m_new);
        m_run[q] = m_new;
        l_run[q] *= alpha;
#pragma unroll
        for (int dt = 0; dt < 8; ++dt) oacc[q][dt] *= alpha;
      }
    }
    f16x8 pb[QT][2];
#pragma unroll
    for (int q = 0; q < QT; ++q) {
      float psum = 0.f;
#pragma unroll
      for (int m = 0; m < 2; ++m) {
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const float pv = __builtin_amdgcn_exp2f(fmaf(sc[q][m][e], a.scale_log2, -m_run[q]));
          psum += pv;
          pb[q][m][e] = (_Float16)pv;
        }
      }
      l_run[q] += psum;
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

  // 3. Tiles: iteration i of key group kg stages tile kg + KW i into the
  //    group's LDS buffer i&1, issues the loads of its next tile into the
  //    registers just staged (they are in flight during the multiply), and
  //    multiplies.  Buffer i&1 was last read at iteration i-2, which every
  //    wave finished before the barrier of iteration i-1.  The loads are
  //    unconditional (the last iteration re-reads a clamped tile), so the
  //    wait before staging covers exactly one tile.
  const int niter = (ntiles + KW - 1) / KW;
  for (int it = 0; it < niter; ++it) {
    const int tile = kg + KW * it;
    const int b = kg * 2 + (it & 1);
    if (tile < ntiles) store_tile(b, ka, va, tile + 1 == ntiles ? tail : KT);
    load_tile(kbeg + min(tile + KW, ntiles - 1) * KT, ka, va);
    __syncthreads();
    if (tile < ntiles && wave_active) compute(b, kbeg + tile * KT);
  }

  // 4. Merge the key groups into key group 0 (per lane and query: the lanes
  //    of one query share m_run, and l is reduced across them afterwards).
  //    The two-term sums are written as explicit fmaf: left to contraction,
  //    the compiler fused one product or the other depending on the
  //    instantiation, and a query's last bit then depended on the launch
  //    shape (two query tiles per wave differed in single elements).
  if constexpr (KW > 1) {
    constexpr int NC = 34;  // O^T fragment (32 floats), m, l
    static_assert((KW - 1) * QW * QT * NC * 64 * 4 <= (int)sizeof(ks), "merge area fits the K tiles");
    float* mb = reinterpret_cast<float*>(&ks[0][0]);
    __syncthreads();  // every wave is done with the tiles
    if (kg > 0) {
#pragma unroll
      for (int q = 0; q < QT; ++q) {
        float* d = mb + ((size_t)(((kg - 1) * QW + qs) * QT + q) * NC) * 64 + lane;
#pragma unroll
        for (int dt = 0; dt < 8; ++dt)
#pragma unroll
          for (int r = 0; r < 4; ++r) d[(dt * 4 + r) * 64] = oacc[q][dt][r];
        d[32 * 64] = m_run[q];
        d[33 * 64] = l_run[q];
      }
    }
    __syncthreads();
    if (kg > 0) return;
#pragma unroll
    for (int k2 = 1; k2 < KW; ++k2) {
#pragma unroll
      for (int q = 0; q < QT; ++q) {
        const float* d = mb + ((size_t)(((k2 - 1) * QW + qs) * QT + q) * NC) * 64 + lane;
        const float m2 = d[32 * 64], l2 = d[33 * 64];
        const float M = fmaxf(m_run[q], m2);
        const float w1 = __builtin_amdgcn_exp2f(m_run[q] - M), w2 = __builtin_amdgcn_exp2f(m2 - M);
#pragma unroll
        for (int dt = 0; dt < 8; ++dt)
#pragma unroll
          for (int r = 0; r < 4; ++r) oacc[q][dt][r] = fmaf(d[(dt * 4 + r) * 64], w2, oacc[q][dt][r] * w1);
        l_run[q] = fmaf(l2, w2, l_run[q] * w1);
        m_run[q] = M;
      }
    }
  }

#pragma unroll
  for (int q = 0; q < QT; ++q) {
    float l = l_run[q];
    l = sum_xor32(sum_xor16(l));
    if (!valid[q]) continue;
    // lane (j, g) holds O^T[16dt + 4g + r][query j]
    if (a.nsplit == 1 && !a.force_part) {
      bf16_t* op = a.out + ((size_t)qrow(q) * a.hq + qhead(q)) * HD + 4 * g;
      const float inv = 1.f / l;
#pragma unroll
      for (int dt = 0; dt < 8; ++dt) {
        uint32_t lo = (uint32_t)f32_to_bf16(oacc[q][dt][0] * inv) | ((uint32_t)f32_to_bf16(oacc[q][dt][1] * inv) << 16);
        uint32_t hi = (uint32_t)f32_to_bf16(oacc[q][dt][2] * inv) | ((uint32_t)f32_to_bf16(oacc[q][dt][3] * inv) << 16);
        *reinterpret_cast<uint2*>(op + 16 * dt) = make_uint2(lo, hi);
      }
    } else {
      const size_t base = ((size_t)bx * a.rows + qrow(q)) * a.hq + qhead(q);
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
// pass.  The partials of up to 16 splits are loaded at once, issued together
// with the row's key limit (indices clamped to the launch's nsplit), and only
// the row's own splits, ceil(hi / kv_split) of them, are merged.  The merge
// starts from the first split's partial and normalises as the unsplit
// epilogue does (O * (1 / l)), so a row whose keys all lie in its first
// split gets the same bits whether or not other rows of the launch need
// more splits.
// One workgroup per (row, 4 heads), one thread per output element.
// B: partials loaded per batch, the launch's split count rounded up to 4, 8
// or 16 (the merge order, and so the result, does not depend on it).
template <typename T, int B>
__global__ __launch_bounds__(512) void attn_combine_kernel(const float* part_o, const float* part_ml,
                                                           const int32_t* row_hi, int rows, int hq, int hd,
                                                           int kv_split, int nsplit, T* out) {
  const int row = blockIdx.x, head = blockIdx.y * 4 + (int)threadIdx.x / HD, d = threadIdx.x % HD;
  if (head >= hq) return;
  const int hi = row_hi[row];
  float M = -1e30f, L = 0.f, O = 0.f;
  for (int c0 = 0; c0 < nsplit; c0 += B) {
    float m[B], l[B], o[B];
#pragma unroll
    for (int i = 0; i < B; ++i) {
      const size_t base = ((size_t)min(c0 + i, nsplit - 1) * rows + row) * hq + head;
      m[i] = part_ml[base * 2];
      l[i] = part_ml[base * 2 + 1];
      o[i] = d < hd ? part_o[base * hd + d] : 0.f;
    }
    const int ns = (hi + kv_split - 1) / kv_split;
#pragma unroll
    for (int i = 0; i < B; ++i) {
      if (c0 + i == 0) {
        M = m[0];
        L = l[0];
        O = o[0];
      } else if (c0 + i < ns) {
        const float Mn = fmaxf(M, m[i]);
        const float wa = exp2f(M - Mn), wb = exp2f(m[i] - Mn);
        L = fmaf(l[i], wb, L * wa);
        O = fmaf(o[i], wb, O * wa);
        M = Mn;
      }
    }
    if (c0 + B >= ns) break;
  }
  const float inv = 1.f / L;
  if (d < hd) Elem<T>::store(out, ((size_t)row * hq + head) * hd + d, O * inv);
}

// The split merge of attn_combine_kernel followed, for a row of a
// quadratic-speculation block (row_blk[row] >= 0), by its block's keys: the
// blk_len keys of the forward's row scratch starting at row row_blk[row]
// (scores q.k scaled into the log2 domain, one thread per key, then one
// online step over the block); then O * (1 / L).  A row without a block
// gets attn_combine_kernel's bits (the AR pathway's rows of the same
// forward are the AR rows).
template <typename T>
__global__ __launch_bounds__(512) void attn_qcombine_kernel(const float* part_o, const float* part_ml,
                                                            const int32_t* row_hi, const int32_t* row_blk,
                                                            const T* q, const T* ks, const T* vs, int blk_len,
                                                            int rows, int hq, int hkv, int kv_split, int nsplit,
                                                            float scale_log2, T* out) {
  constexpr int B = 16;
  __shared__ float sc[4][64];
  const int row = blockIdx.x, hl = (int)threadIdx.x / HD, head = blockIdx.y * 4 + hl, d = threadIdx.x % HD;
  const bool hv = head < hq;
  const int hh = hv ? head : hq - 1;
  const int hi = row_hi[row];
  float M = -1e30f, L = 0.f, O = 0.f;
  for (int c0 = 0; c0 < nsplit; c0 += B) {
    float m[B], l[B], o[B];
#pragma unroll
    for (int i = 0; i < B; ++i) {
      const size_t base = ((size_t)min(c0 + i, nsplit - 1) * rows + row) * hq + hh;
      m[i] = part_ml[base * 2];
      l[i] = part_ml[base * 2 + 1];
      o[i] = part_o[base * HD + d];
    }
    const int ns = (hi + kv_split - 1) / kv_split;
#pragma unroll
    for (int i = 0; i < B; ++i) {
      if (c0 + i == 0) {
        M = m[0];
        L = l[0];
        O = o[0];
      } else if (c0 + i < ns) {
        const float Mn = fmaxf(M, m[i]);
        const float wa = exp2f(M - Mn), wb = exp2f(m[i] - Mn);
        L = fmaf(l[i], wb, L * wa);
        O = fmaf(o[i], wb, O * wa);
        M = Mn;
      }
    }
    if (c0 + B >= ns) break;
  }
  const int blk = row_blk[row];
  if (blk >= 0) {  // the same for every thread of the workgroup
    const int kvh = hh / (hq / hkv);
    if (d < blk_len) {
      const T* qp = q + ((size_t)row * hq + hh) * HD;
      const T* kp = ks + ((size_t)(blk + d) * hkv + kvh) * HD;
      float acc = 0.f;
      for (int e = 0; e < HD; ++e) acc = fmaf(Elem<T>::load(qp, e), Elem<T>::load(kp, e), acc);
      sc[hl][d] = acc * scale_log2;
    }
    __syncthreads();
    float m2 = -1e30f;
    for (int j = 0; j < blk_len; ++j) m2 = fmaxf(m2, sc[hl][j]);
    float l2 = 0.f, o2 = 0.f;
    for (int j = 0; j < blk_len; ++j) {
      const float p = exp2f(sc[hl][j] - m2);
      l2 += p;
      o2 = fmaf(p, Elem<T>::load(vs, ((size_t)(blk + j) * hkv + kvh) * HD + d), o2);
    }
    const float Mn = fmaxf(M, m2);
    const float wa = exp2f(M - Mn), wb = exp2f(m2 - Mn);
    L = fmaf(l2, wb, L * wa);
    O = fmaf(o2, wb, O * wa);
  }
  const float inv = 1.f / L;
  if (hv) Elem<T>::store(out, ((size_t)row * hq + head) * HD + d, O * inv);
}

// float32 path: one wave per (row, head), keys 64 at a time, one pass.
// A row of a quadratic-speculation block (row_blk[row] >= 0) continues the
// same online pass over its block's blk_len keys from the row scratch
// ks / vs [rows][hkv][hd].
__global__ __launch_bounds__(64) void attn_f32_kernel(const float* q, const float* kc, const float* vc,
                                                       const int32_t* seq_start, const int32_t* slot_seq,
                                                       int n_seq, const int32_t* row_hi, int hq, int hkv, int hd,
                                                       int ctx, float scale, float* out, const int32_t* row_blk,
                                                       const float* ks, const float* vs, int blk_len) {
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
    l = fmaf(l, alpha, ps);
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
  const int blk = row_blk ? row_blk[row] : -1;
  if (blk >= 0) {
    const int key = lane;
    float s = -INFINITY;
    if (key < blk_len) {
      float acc = 0.f;
      const float* kp = ks + ((size_t)(blk + key) * hkv + kvh) * hd;
      for (int d = 0; d < hd; ++d) acc = fmaf(qs[d], kp[d], acc);
      s = acc * scale;
    }
    float cmax = s;
    for (int off = 32; off > 0; off >>= 1) cmax = fmaxf(cmax, __shfl_xor(cmax, off));
    const float m_new = fmaxf(m, cmax);
    const float alpha = expf(m - m_new);
    const float p = (key < blk_len) ? expf(s - m_new) : 0.f;
    float ps = p;
    for (int off = 32; off > 0; off >>= 1) ps += __shfl_xor(ps, off);
    l = fmaf(l, alpha, ps);
    o0 *= alpha;
    o1 *= alpha;
    for (int jj = 0; jj < blk_len; ++jj) {
      const float pj = __shfl(p, jj);
      const float* vp = vs + ((size_t)(blk + jj) * hkv + kvh) * hd;
      if (lane < hd) o0 = fmaf(pj, vp[lane], o0);
      if (lane + 64 < hd) o1 = fmaf(pj, vp[lane + 64], o1);
    }
  }
  float* op = out + ((size_t)row * hq + head) * hd;
  if (lane < hd) op[lane] = o0 / l;
  if (lane + 64 < hd) op[lane + 64] = o1 / l;
}

}  // namespace

// Launch shape: query slots per key group (qw) and query tiles per slot (qt).
// Two slots for short prefixes or few query tiles (more workgroups), four
// otherwise; two query tiles per slot for long prefixes with more than eight
// query tiles per kv head (each K/V tile read once per 128 query vectors).
// The rounding depends on neither choice.
static void attn_shape(int qtiles, int max_hi, int* qw, int* qt) {
  if (qtiles >= 64) {  // prefill-sized blocks (>= 256 rows of one sequence)
    *qw = 4;
    *qt = max_hi > 1024 ? 2 : 1;
    return;
  }
  *qt = (qtiles >= 8 && max_hi > 4096) ? 2 : 1;
  *qw = (*qt == 1 && (qtiles <= 2 || max_hi <= 1536)) ? 2 : 4;
}

int attn_pick_split(int max_ctx, int n_seq, int hq, int hkv) {
  // Keys per split for a session of n_seq sequences of up to max_ctx keys.
  // One sequence: the largest power of two at most max_ctx / 16, within
  // [128, 2048].  Measured on MI355X for 32-row blocks at batch 1 (attention
  // + combine): 1K keys 12.0 us with 256-key splits (15.6 with 128), 2K keys
  // 13.9 with 256, 8K keys 24.7 with 512, 16K keys 32.8 with 1024; a
  // session's contexts usually stay below its capacity, which the shorter
  // splits also serve.  Several sequences: the launch model below at the session's
  // capacity and a 33-row block per sequence (their workgroups fill the chip
  // without short splits: at 4 sequences x 1K keys 22 us unsplit against 34
  // with 128-key splits, at 16 x 1K 43 against 111).  A session keeps one
  // split size, so a row's result never depends on the launch.
  if (n_seq > 1) return attn_pick_split_launch(max_ctx, n_seq, 33, hq, hkv);
  int s = 128;
  const double lim = (double)max_ctx / 16.0;
  while (s < 2048 && 2.0 * s <= lim) s *= 2;
  // Long-context sessions (their decode forwards do run near capacity): a
  // workgroup holds a CU's LDS, so a launch of more than 256 workgroups runs
  // in two rounds, the second as long as the first.  Take the smallest
  // multiple of 64 keys, up to twice the split above, that keeps a
  // full-capacity launch of 33-row blocks in one round (for example the
  // 14B-class heads, 40q/8kv with two query groups per split, behind a 16K
  // prefix: 16 splits of 1088 keys, 256 workgroups, instead of 17 of 1024).
  if (max_ctx >= 8192 && hkv > 0) {
    const int qtiles = (33 * (hq / hkv) + 15) / 16;
    int qw, qt;
    attn_shape(qtiles, max_ctx, &qw, &qt);
    const long per_split = (long)((qtiles + qw * qt - 1) / (qw * qt)) * hkv;
    const long ns_max = 256 / per_split;
    if (ns_max >= 1) {
      const int s2 = (int)(((max_ctx + ns_max - 1) / ns_max + 63) / 64 * 64);
      if (s2 > s && s2 <= 2 * s) s = s2;
    }
  }
  return s;
}

int attn_pick_split_launch(int max_hi, int n_seq, int rows_per_seq, int hq, int hkv) {
  // Keys per split for one launch (the C-ABI's kv_split = 0): the power of two
  // in [128, 4096] with the lowest modelled time, or the multiple of 64 with
  // the lowest modelled time when that is at least 10% lower (a split that
  // fills whole rounds of 256 workgroups; the margin keeps near-ties, where
  // the model's error decides, on the measured powers of two: at 16 sequences
  // x 1.7K keys its 2% edge for 832-key splits was a 7% loss per forward).
  // Model, fitted to MI355X measurements at 32q/8kv heads, 32-row blocks,
  // prefixes 512..32K, 1 and 8 sequences: a workgroup costs 4 us plus 1.8 us
  // per 128 keys it walks (two key groups of 64-key tiles), workgroups run one
  // per CU in waves of 256, and more than one split adds a 4 us combine.
  // Workgroups of two query tiles per wave (long prefixes) were fitted
  // separately, at prefixes 4K..32K: 13 us plus 2.8 us per 128 keys, no
  // measurable combine term.
  const int G = hkv > 0 ? hq / hkv : 1;
  const int qtiles = std::max(1, (rows_per_seq * G + 15) / 16);
  int qw, qt;
  attn_shape(qtiles, max_hi, &qw, &qt);
  const long qg = (qtiles + qw * qt - 1) / (qw * qt);
  const double fixed = qt == 2 ? 13.0 : 4.0, per128 = qt == 2 ? 2.8 : 1.8, combine = qt == 2 ? 0.0 : 4.0;
  auto model = [&](int sp) {
    const long ns = std::max(1, (max_hi + sp - 1) / sp);
    const long nwg = ns * qg * std::max(1, n_seq) * std::max(1, hkv);
    return std::ceil(nwg / 256.0) * (fixed + per128 * std::ceil(std::min(sp, std::max(max_hi, 1)) / 128.0)) +
           (ns > 1 ? combine : 0.0);
  };
  int best2 = 128, best64 = 128;
  double t2 = 1e30, t64 = 1e30;
  for (int sp = 128; sp <= 4096; sp += 64) {
    const double t = model(sp);
    if ((sp & (sp - 1)) == 0 && t < t2) {
      t2 = t;
      best2 = sp;
    }
    if (t < t64) {
      t64 = t;
      best64 = sp;
    }
  }
  return t64 <= 0.9 * t2 ? best64 : best2;
}

int attn_group_vectors(int max_rows_per_seq, int G, int max_hi) {
  int qw, qt;
  attn_shape((max_rows_per_seq * G + 15) / 16, max_hi, &qw, &qt);
  return qw * 16 * qt;
}

// Compacted attention grid of a forward (see AttnArgs::work): one entry per
// (slot, query group) that holds query vectors, under the launch shape
// launch_attn takes for these rows.  0 when every slot has the same number
// of groups (the regular grid launches no empty workgroup) or the table
// would pass `cap` entries.  Measured on MI355X, 64 sequences with one
// 33-row block among single rows: the regular grid launched 2048-2560
// workgroups, most of them empty, and the attention took 44-94 us against
// 36 us for single rows only.
int attn_work_table(const int32_t* seq_start, int n_slots, int hq, int hkv, int max_hi, int32_t* out, int cap) {
  if (n_slots < 2 || hkv < 1) return 0;
  const int G = hq / hkv;
  int max_rows = 0;
  for (int i = 0; i < n_slots; ++i) max_rows = std::max(max_rows, seq_start[i + 1] - seq_start[i]);
  const int qv = attn_group_vectors(max_rows, G, max_hi);
  int w = 0;
  bool uniform = true;
  const int g0 = ((seq_start[1] - seq_start[0]) * G + qv - 1) / qv;
  for (int i = 0; i < n_slots; ++i) {
    const int groups = ((seq_start[i + 1] - seq_start[i]) * G + qv - 1) / qv;
    uniform = uniform && groups == g0;
    if (groups > 65535 || w + groups > cap) return 0;
    for (int g = 0; g < groups; ++g) out[w++] = i * 65536 + g;
  }
  return uniform ? 0 : w;
}

size_t attn_ws_bytes(int rows, int hq, int hd, int max_hi, int kv_split) {
  if (kv_split <= 0) kv_split = 128;  // the shortest split any pick makes: an upper bound
  const size_t ns = (size_t)((max_hi + kv_split - 1) / kv_split);
  if (ns <= 1) return 256;
  return ns * (size_t)rows * hq * (hd + 2) * sizeof(float) + 256;
}

hipError_t launch_attn(int dtype, const AttnLaunch& L, hipStream_t st) {
  if (L.rows <= 0) return hipSuccess;
  if (L.row_blk && (L.blk_len < 1 || L.blk_len > 64 || !L.k_scr || !L.v_scr)) return hipErrorInvalidValue;
  if (dtype == TRI_F32) {
    hipLaunchKernelGGL(attn_f32_kernel, dim3(L.rows, L.hq), dim3(64), 0, st, static_cast<const float*>(L.q),
                       static_cast<const float*>(L.kc), static_cast<const float*>(L.vc), L.seq_start, L.slot_seq,
                       L.n_seq, L.row_hi, L.hq, L.hkv, L.hd, L.ctx, L.scale, static_cast<float*>(L.out), L.row_blk,
                       static_cast<const float*>(L.k_scr), static_cast<const float*>(L.v_scr), L.blk_len);
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
  a.force_part = L.row_blk != nullptr;
  const size_t np = (size_t)a.nsplit * L.rows * L.hq;
  a.part_o = L.part;
  a.part_ml = L.part + np * HD;
  const int G = L.hq / L.hkv;
  const int qtiles = (L.max_rows_per_seq * G + 15) / 16;
  // Two key groups always (the tile order inside a key group, and so the
  // rounding, then depends only on kv_split).
  int qw, qt;
  attn_shape(qtiles, L.max_hi, &qw, &qt);
  const int qgroups = (qtiles + qw * qt - 1) / (qw * qt);
  a.qgroups = qgroups;
  a.nz = L.n_seq * L.hkv;
  a.work = L.work;
  a.nwork = L.nwork;
  const long pairs8 = ((long)a.nsplit * a.nz + 7) / 8 * 8;
  if (pairs8 * qgroups > 0x7fffffffL) return hipErrorInvalidValue;
  if (L.work && (L.nwork < 1 || (long)L.nwork * L.hkv * a.nsplit > 0x7fffffffL)) return hipErrorInvalidValue;
  const dim3 grid(L.work ? (unsigned)((long)L.nwork * L.hkv * a.nsplit) : (unsigned)(pairs8 * qgroups));
  if (L.v_f16) {
    if (qw == 2)
      hipLaunchKernelGGL((attn_bf16_kernel<2, 2, 1, true>), grid, dim3(256), 0, st, a);
    else if (qt == 1)
      hipLaunchKernelGGL((attn_bf16_kernel<4, 2, 1, true>), grid, dim3(512), 0, st, a);
    else
      hipLaunchKernelGGL((attn_bf16_kernel<4, 2, 2, true>), grid, dim3(512), 0, st, a);
  } else if (qw == 2) {
    hipLaunchKernelGGL((attn_bf16_kernel<2, 2, 1>), grid, dim3(256), 0, st, a);
  } else if (qt == 1) {
    hipLaunchKernelGGL((attn_bf16_kernel<4, 2, 1>), grid, dim3(512), 0, st, a);
  } else {
    hipLaunchKernelGGL((attn_bf16_kernel<4, 2, 2>), grid, dim3(512), 0, st, a);
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  if (L.row_blk) {
    hipLaunchKernelGGL(attn_qcombine_kernel<bf16_t>, dim3(L.rows, (L.hq + 3) / 4), dim3(4 * HD), 0, st, a.part_o,
                       a.part_ml, L.row_hi, L.row_blk, a.q, static_cast<const bf16_t*>(L.k_scr),
                       static_cast<const bf16_t*>(L.v_scr), L.blk_len, L.rows, L.hq, L.hkv, L.kv_split, a.nsplit,
                       a.scale_log2, a.out);
    return hipGetLastError();
  }
  if (a.nsplit == 1) return e;
  const dim3 cgrid(L.rows, (L.hq + 3) / 4), cblock(4 * HD);
  if (a.nsplit <= 4)
    hipLaunchKernelGGL((attn_combine_kernel<bf16_t, 4>), cgrid, cblock, 0, st, a.part_o, a.part_ml, L.row_hi,
                       L.rows, L.hq, HD, L.kv_split, a.nsplit, a.out);
  else if (a.nsplit <= 8)
    hipLaunchKernelGGL((attn_combine_kernel<bf16_t, 8>), cgrid, cblock, 0, st, a.part_o, a.part_ml, L.row_hi,
                       L.rows, L.hq, HD, L.kv_split, a.nsplit, a.out);
  else
    hipLaunchKernelGGL((attn_combine_kernel<bf16_t, 16>), cgrid, cblock, 0, st, a.part_o, a.part_ml, L.row_hi,
                       L.rows, L.hq, HD, L.kv_split, a.nsplit, a.out);
  return hipGetLastError();
}

}  // namespace tri
