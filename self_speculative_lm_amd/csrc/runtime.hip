// Host runtime of libtrimode.so: the C-ABI, model/session bookkeeping and the
// decode state machine of the three modes.  All arithmetic of the path runs in
// the gfx950 kernels of k_gemm.hip, k_attn.hip and k_misc.hip; this file only
// lays out rows, launches kernels on the session stream and reads back the few
// integers that decide the next step.
//
// Decode state of a sequence (the pending-token bookkeeping of speculative
// decoding, reading R4 of the design notes): committed tokens x[0..L) and a KV
// cache holding causal K/V of positions [0, kv_len); the tokens x[kv_len..L)
// are pending and ride as clean causal rows at the head of the next forward.
#include <stdarg.h>
#include <stdio.h>
#include <string.h>

#include <algorithm>
#include <cmath>
#include <mutex>
#include <string>
#include <vector>

#include "tri_common.h"

using namespace tri;

namespace {

thread_local std::string g_err;

int fail(int code, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_err = buf;
  return code;
}

#define HIPCHK(expr)                                                                   \
  do {                                                                                 \
    hipError_t e_ = (expr);                                                            \
    if (e_ != hipSuccess) return fail(TRI_EHIP, "%s: %s", #expr, hipGetErrorString(e_)); \
  } while (0)

size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

// One layer's weights inside the model buffer (projections packed for the GEMM).
struct Layer {
  const void *qkv, *o, *gu, *down;
  const float *n1, *n2;
  const void *la, *lb;
};

}  // namespace

struct tri_model {
  tri_model_desc d;
  const void* embed;
  std::vector<Layer> layers;
  const float* final_norm;
  const void* lm_head;
  size_t esz;
  GemmPlan p_qkv, p_o, p_gu, p_down, p_lm, p_la, p_lb;
  int qkv_n;
};

namespace {

struct Seq {
  std::vector<int32_t> tokens;
  int kv_len = 0;
  int written_hi = 0;  // clean rows written by forwards: [0, written_hi) usable by kv_append
  bool active = false;
  // controlled-acceptance override (benchmark hook)
  std::vector<int32_t> ref;
  int a_star = -1;
  // controlled commit rate (benchmark hook): per-forward commit counts of a diffusion block
  std::vector<int32_t> sched;
  // quadratic self-speculation: drafts for positions L .. L+k-1 carried from
  // the previous round (empty: the next round starts without drafts)
  std::vector<int32_t> qdrafts;
};

// Row metadata of one forward: a host (pinned) mirror and a device copy.
struct MetaLayout {
  size_t tok, pos, hi, seq, lora, kind, blk, seq_start, slot_seq, block_start, sidx, didx, awork, size;
  int awork_cap;
};
MetaLayout meta_layout(int max_rows, int max_batch) {
  MetaLayout L;
  size_t o = 0;
  auto take = [&](size_t n) {
    size_t r = o;
    o += (n + 63) & ~size_t(63);
    return r;
  };
  L.tok = take(max_rows);
  L.pos = take(max_rows);
  L.hi = take(max_rows);
  L.seq = take(max_rows);
  L.lora = take(max_rows);
  L.kind = take(max_rows);
  L.blk = take(max_rows);
  L.seq_start = take(max_batch + 1);
  L.slot_seq = take(max_batch);
  L.block_start = take(max_batch + 1);
  L.sidx = take(2 * (size_t)max_rows + 2 * max_batch);
  L.didx = take(2 * (size_t)max_rows + 2 * max_batch);
  L.awork_cap = max_rows + max_batch;  // (slot, query group) entries: enough up to 32 query heads per kv head
  L.awork = take((size_t)L.awork_cap);
  L.size = o;
  return L;
}

struct Meta {
  int32_t *tok, *pos, *hi, *seq, *lora, *kind, *blk, *seq_start, *slot_seq, *block_start, *sidx, *didx, *awork;
};
Meta meta_ptrs(int32_t* base, size_t off, const MetaLayout& L) {
  int32_t* b = base + off;
  return Meta{b + L.tok,  b + L.pos,       b + L.hi,          b + L.seq,         b + L.lora, b + L.kind, b + L.blk,
              b + L.seq_start, b + L.slot_seq, b + L.block_start, b + L.sidx, b + L.didx, b + L.awork};
}

// The layout of a forward's metadata is sized by its own rows (rounded up to
// 64, at most max_rows), so the upload of a decode forward stays small when
// the session allows long prefill chunks.  Every user of a staged set reads
// its layout from the session.
MetaLayout forward_layout(int n, int max_rows, int max_batch) {
  return meta_layout(std::min((n + 63) & ~63, max_rows), max_batch);
}

// Host-side rows of one forward.  blk: per row the first row of its
// quadratic-speculation block or -1 (only filled when blk_len > 0: the rows
// of a block attend to the cache keys [0, hi) and to the blk_len rows of
// their block).
struct HostRows {
  std::vector<int32_t> tok, pos, hi, seq, lora, kind, blk;
  int blk_len = 0;
  std::vector<int32_t> seq_start{0};  // per slot (one slot per participating sequence)
  std::vector<int32_t> slot_seq;
  std::vector<int32_t> block_start;   // per block (empty: no blocks)
  int n() const { return (int)tok.size(); }
  void add(int t, int p, int h, int s, int l, int k, int b = -1) {
    tok.push_back(t);
    pos.push_back(p);
    hi.push_back(h);
    seq.push_back(s);
    lora.push_back(l);
    kind.push_back(k);
    blk.push_back(b);
  }
  void close_slot(int s) {
    seq_start.push_back(n());
    slot_seq.push_back(s);
  }
};

struct TraceRec {
  std::vector<int32_t> seq, tok, pos, hi, lora;
  std::vector<float> logits;  // empty for forwards without an lm_head
};

enum ProfClass { PROF_GU = 0, PROF_DOWN, PROF_QKV, PROF_O, PROF_LM, PROF_ATTN, PROF_FWD, PROF_N };

}  // namespace

struct tri_session {
  const tri_model* m;
  int max_batch, max_ctx, ctx, max_rows;
  hipStream_t st;
  int kv_split;
  char* kbuf;
  char* vbuf;
  size_t css;  // cache elements per (layer, sequence)
  float* rope;
  float* x;
  void* ybuf;
  void* ybuf2;  // the fused gate/up + SwiGLU writes here; the two swap roles
  void* qbuf;
  void* abuf;
  float* part;
  float* part2;
  void* attn_ws;
  void* kscr;  // quadratic-speculation block rows' K and V [max_rows][hkv][hd] each
  void* vscr;
  float* logits;
  void* vws;
  int32_t* dints;
  float* dconf;
  size_t nints;
  int32_t* hints;
  float* hconf;
  size_t o_meta[2];
  size_t o_out_tok, o_out_commit, o_status, o_accept, o_committed, o_kvlen, o_drafts, o_ars;
  std::vector<Seq> seqs;
  bool lora_on = false;
  bool tracing = false;
  std::vector<TraceRec> trace;
  MetaLayout mlay[2];                          // layout of each metadata set as last staged
  hipEvent_t meta_ev[2] = {nullptr, nullptr};  // recorded after each metadata upload
  int awork_n[2] = {0, 0};                     // entries of each set's compacted attention grid
  bool meta_pending[2] = {false, false};
  int prof_class = -1;
  std::vector<hipEvent_t> ev;  // start/stop pairs
  size_t ev_used = 0;
};

namespace {

struct SessionLayout {
  size_t k, v, rope, x, y, y2, q, a, part, part2, attn, kscr, vscr, logits, vws, ints, conf, total;
  size_t part_floats, part2_floats, attn_bytes, nints;
  size_t o_meta0, o_meta1, o_out_tok, o_out_commit, o_status, o_accept, o_committed, o_kvlen, o_drafts, o_ars;
  int ctx, kv_split;
  size_t css;
};

SessionLayout session_layout(const tri_model* m, int max_batch, int max_ctx, int max_rows) {
  const tri_model_desc& d = m->d;
  SessionLayout S;
  S.ctx = (max_ctx + 63) / 64 * 64;
  S.kv_split = attn_pick_split(S.ctx, max_batch, d.n_q_heads, d.n_kv_heads);
  S.css = (size_t)d.n_kv_heads * S.ctx * d.head_dim;
  const size_t cache_bytes = (size_t)d.n_layers * max_batch * S.css * m->esz;
  const size_t qd = (size_t)d.n_q_heads * d.head_dim;
  const size_t ywidth = std::max<size_t>({(size_t)d.d_model, (size_t)d.d_ffn, qd, (size_t)std::max(d.lora_rank, 1)});
  auto slotsN = [&](const GemmPlan& p, int N, int extra) { return (size_t)(p.S + extra) * N; };
  const size_t pf = std::max({slotsN(m->p_qkv, m->qkv_n, 0), slotsN(m->p_o, d.d_model, m->p_lb.S),
                              slotsN(m->p_gu, 2 * d.d_ffn, 0), slotsN(m->p_down, d.d_model, 0)});
  S.part_floats = pf * max_rows;
  S.part2_floats = d.lora_rank > 0 ? (size_t)m->p_la.S * d.lora_rank * max_rows : 64;
  // a forward with quadratic-speculation blocks writes split partials even
  // when its keys fit one split
  S.attn_bytes = std::max(attn_ws_bytes(max_rows, d.n_q_heads, d.head_dim, S.ctx, S.kv_split),
                          (size_t)max_rows * d.n_q_heads * (d.head_dim + 2) * sizeof(float) + 256);
  const MetaLayout ML = meta_layout(max_rows, max_batch);
  size_t o = 0;
  auto take = [&](size_t n) {
    size_t r = o;
    o += (n + 63) & ~size_t(63);
    return r;
  };
  S.o_meta0 = take(ML.size);
  S.o_meta1 = take(ML.size);
  S.o_out_tok = take(max_rows);
  S.o_out_commit = take(max_rows);
  S.o_status = take(4);
  S.o_accept = take(max_batch);
  S.o_committed = take((size_t)max_batch * 65);
  S.o_kvlen = take(max_batch);
  S.o_drafts = take((size_t)max_batch * 64);
  S.o_ars = take((size_t)max_batch * 65);
  S.nints = o;
  size_t off = 0;
  auto region = [&](size_t bytes) {
    size_t r = off;
    off = align256(off + bytes);
    return r;
  };
  S.k = region(cache_bytes);
  S.v = region(cache_bytes);
  S.rope = region((size_t)S.ctx * (d.head_dim / 2) * 2 * sizeof(float));
  S.x = region((size_t)max_rows * d.d_model * sizeof(float));
  S.y = region((size_t)max_rows * ywidth * m->esz);
  S.y2 = region((size_t)max_rows * ywidth * m->esz);
  S.q = region((size_t)max_rows * qd * m->esz);
  S.a = region((size_t)max_rows * qd * m->esz);
  S.part = region(S.part_floats * sizeof(float));
  S.part2 = region(S.part2_floats * sizeof(float));
  S.attn = region(S.attn_bytes);
  S.kscr = region((size_t)max_rows * d.n_kv_heads * d.head_dim * m->esz);
  S.vscr = region((size_t)max_rows * d.n_kv_heads * d.head_dim * m->esz);
  S.logits = region((size_t)max_rows * d.vocab * sizeof(float));
  S.vws = region(vocab_ws_bytes(max_rows, d.vocab));
  S.ints = region(S.nints * sizeof(int32_t));
  S.conf = region((size_t)max_rows * sizeof(float));
  S.total = off;
  return S;
}

// ------------------------------------------------------------------ profiling
int prof_begin(tri_session* s, int cls, size_t* slot) {
  if (s->prof_class != cls) return TRI_OK;
  if (s->ev_used + 2 > s->ev.size()) {
    for (int i = 0; i < 64; ++i) {
      hipEvent_t e;
      HIPCHK(hipEventCreate(&e));
      s->ev.push_back(e);
    }
  }
  *slot = s->ev_used;
  s->ev_used += 2;
  HIPCHK(hipEventRecord(s->ev[*slot], s->st));
  return TRI_OK;
}
int prof_end(tri_session* s, int cls, size_t slot) {
  if (s->prof_class != cls) return TRI_OK;
  HIPCHK(hipEventRecord(s->ev[slot + 1], s->st));
  return TRI_OK;
}
#define PROF(cls, call)                        \
  do {                                         \
    size_t slot_ = 0;                          \
    int rc_ = prof_begin(s, (cls), &slot_);    \
    if (rc_) return rc_;                       \
    HIPCHK(call);                              \
    rc_ = prof_end(s, (cls), slot_);           \
    if (rc_) return rc_;                       \
  } while (0)

// ------------------------------------------------------------------ forward
// The pinned host mirror of a metadata set is the source of an asynchronous
// copy: before it is rewritten, wait until the GPU has consumed the previous
// upload of that set (back-to-back forwards, e.g. prefill chunks, would
// otherwise upload another forward's rows).
int stage_meta(tri_session* s, int which, const HostRows& R, const std::vector<int32_t>& sidx,
               const std::vector<int32_t>& didx) {
  if (s->meta_pending[which]) {
    HIPCHK(hipEventSynchronize(s->meta_ev[which]));
    s->meta_pending[which] = false;
  }
  const MetaLayout ML = forward_layout(R.n(), s->max_rows, s->max_batch);
  if (sidx.size() > ML.didx - ML.sidx) return fail(TRI_ECAPACITY, "too many scatter entries");
  s->mlay[which] = ML;
  Meta h = meta_ptrs(s->hints, s->o_meta[which], ML);
  const size_t n = R.n();
  memcpy(h.tok, R.tok.data(), n * 4);
  memcpy(h.pos, R.pos.data(), n * 4);
  memcpy(h.hi, R.hi.data(), n * 4);
  memcpy(h.seq, R.seq.data(), n * 4);
  memcpy(h.lora, R.lora.data(), n * 4);
  memcpy(h.kind, R.kind.data(), n * 4);
  if (R.blk_len > 0) memcpy(h.blk, R.blk.data(), n * 4);
  memcpy(h.seq_start, R.seq_start.data(), R.seq_start.size() * 4);
  memcpy(h.slot_seq, R.slot_seq.data(), R.slot_seq.size() * 4);
  if (!R.block_start.empty()) memcpy(h.block_start, R.block_start.data(), R.block_start.size() * 4);
  if (!sidx.empty()) {
    memcpy(h.sidx, sidx.data(), sidx.size() * 4);
    memcpy(h.didx, didx.data(), didx.size() * 4);
  }
  // the attention's compacted grid (bf16 attention only; 0 = regular grid)
  int max_hi = 0;
  for (int32_t v : R.hi) max_hi = std::max(max_hi, (int)v);
  const tri_model_desc& d = s->m->d;
  s->awork_n[which] = d.dtype == TRI_BF16
                          ? attn_work_table(R.seq_start.data(), (int)R.slot_seq.size(), d.n_q_heads, d.n_kv_heads,
                                            max_hi, h.awork, ML.awork_cap)
                          : 0;
  return TRI_OK;
}

int upload_meta(tri_session* s, int which) {
  const MetaLayout& ML = s->mlay[which];
  HIPCHK(hipMemcpyAsync(s->dints + s->o_meta[which], s->hints + s->o_meta[which], ML.size * 4,
                        hipMemcpyHostToDevice, s->st));
  HIPCHK(hipEventRecord(s->meta_ev[which], s->st));
  s->meta_pending[which] = true;
  return TRI_OK;
}

// Run the model over the rows of metadata set `which`.  logits_out: where the
// lm_head writes [n][vocab]; NULL skips the final norm and lm_head (prefill).
int forward(tri_session* s, int which, const HostRows& R, float* logits_out) {
  const tri_model* m = s->m;
  const tri_model_desc& d = m->d;
  const int n = R.n();
  if (n <= 0) return TRI_OK;
  Meta dm = meta_ptrs(s->dints, s->o_meta[which], s->mlay[which]);
  const int dt = d.dtype;
  const int hq = d.n_q_heads, hkv = d.n_kv_heads, hd = d.head_dim, D = d.d_model;
  const int qd = hq * hd;
  const int nslot = (int)R.slot_seq.size();
  int max_rows_per_seq = 0, max_hi = 0;
  bool any_lora = false;
  for (int i = 0; i < nslot; ++i) max_rows_per_seq = std::max(max_rows_per_seq, R.seq_start[i + 1] - R.seq_start[i]);
  for (int i = 0; i < n; ++i) {
    max_hi = std::max(max_hi, R.hi[i]);
    any_lora = any_lora || (R.lora[i] != 0);
  }
  any_lora = any_lora && s->lora_on && d.lora_rank > 0;
  size_t fslot = 0;
  int rc = prof_begin(s, PROF_FWD, &fslot);
  if (rc) return rc;
  const size_t layer_elems = (size_t)s->max_batch * s->css;
  // Decode forwards (with logits) keep every row's result independent of the
  // rows beside it, so self-speculation, AR and mixed batches of any size
  // take the same greedy decisions; prefill chunks use the fastest slot count.
  const bool inv = logits_out != nullptr;
  int32_t* vsat = s->dints + s->o_status + 3;
  HIPCHK(launch_embed(dt, dm.tok, n, m->embed, d.vocab + 1, D, s->x, s->st));
  int prev_slots = 0;
  size_t prev_stride = 0;
  const float scale = 1.0f / std::sqrt((float)hd);
  for (int l = 0; l < d.n_layers; ++l) {
    const Layer& L = m->layers[l];
    char* kc = s->kbuf + l * layer_elems * m->esz;
    char* vc = s->vbuf + l * layer_elems * m->esz;
    HIPCHK(launch_resid_norm(dt, s->x, s->part, prev_slots, prev_stride, n, D, L.n1, d.rms_eps, s->ybuf, s->st));
    {
      const size_t stride = (size_t)n * m->qkv_n;
      PROF(PROF_QKV, launch_gemm(dt, s->ybuf, n, D, L.qkv, m->qkv_n, m->p_qkv, s->part, stride, inv, s->st));
      // bf16 sessions keep V in the attention's fp16 form (same bits, staged without conversion)
      HIPCHK(launch_rope_kv(dt, s->part, gemm_out_slots(dt, m->p_qkv, n, m->qkv_n, D, inv), stride, n, hq, hkv, hd,
                            dm.seq, dm.pos, s->rope, s->qbuf, kc, vc, s->ctx, s->css, s->st, dt == TRI_BF16,
                            vsat, R.blk_len > 0 ? dm.blk : nullptr, s->kscr, s->vscr));
    }
    {
      AttnLaunch a;
      a.q = s->qbuf;
      a.kc = kc;
      a.vc = vc;
      a.seq_start = dm.seq_start;
      a.slot_seq = dm.slot_seq;
      a.row_hi = dm.hi;
      a.n_seq = nslot;
      a.rows = n;
      a.max_rows_per_seq = max_rows_per_seq;
      a.max_hi = max_hi;
      a.hq = hq;
      a.hkv = hkv;
      a.hd = hd;
      a.ctx = s->ctx;
      a.scale = scale;
      // Decode forwards keep the session's split (a row's rounding then never
      // depends on the launch).  A prefill chunk (no logits) has many rows
      // over a short prefix: one split per 4096 keys, so short prompts need
      // no combine.
      a.kv_split = s->kv_split;
      if (!logits_out)
        while (a.kv_split < 4096 && a.kv_split < max_hi) a.kv_split *= 2;
      a.out = s->abuf;
      a.part = static_cast<float*>(s->attn_ws);
      if (s->awork_n[which] > 0) {
        a.work = dm.awork;
        a.nwork = s->awork_n[which];
      }
      a.v_f16 = dt == TRI_BF16;
      if (R.blk_len > 0) {
        a.row_blk = dm.blk;
        a.k_scr = s->kscr;
        a.v_scr = s->vscr;
        a.blk_len = R.blk_len;
      }
      PROF(PROF_ATTN, launch_attn(dt, a, s->st));
    }
    const size_t ostride = (size_t)n * D;
    int oslots = gemm_out_slots(dt, m->p_o, n, D, qd, inv);
    {
      PROF(PROF_O, launch_gemm(dt, s->abuf, n, qd, L.o, D, m->p_o, s->part, ostride, inv, s->st));
    }
    if (any_lora) {
      const int rk = d.lora_rank;
      const size_t astride = (size_t)n * rk;
      HIPCHK(launch_gemm(dt, s->abuf, n, qd, L.la, rk, m->p_la, s->part2, astride, inv, s->st));
      HIPCHK(launch_lora_mid(dt, s->part2, gemm_out_slots(dt, m->p_la, n, rk, qd, inv), astride, n, rk, dm.lora, s->ybuf, s->st));
      HIPCHK(launch_gemm(dt, s->ybuf, n, rk, L.lb, D, m->p_lb, s->part + (size_t)oslots * ostride, ostride, inv, s->st));
      oslots += gemm_out_slots(dt, m->p_lb, n, D, rk, inv);
    }
    HIPCHK(launch_resid_norm(dt, s->x, s->part, oslots, ostride, n, D, L.n2, d.rms_eps, s->ybuf, s->st));
    {
      const size_t stride = (size_t)n * 2 * d.d_ffn;
      if (gemm_swiglu_fused(dt, m->p_gu, n, 2 * d.d_ffn, D, inv)) {
        PROF(PROF_GU, launch_gemm(dt, s->ybuf, n, D, L.gu, 2 * d.d_ffn, m->p_gu, s->part, stride, inv, s->st,
                                  s->ybuf2));
        std::swap(s->ybuf, s->ybuf2);  // h is the down projection's input
      } else {
        PROF(PROF_GU, launch_gemm(dt, s->ybuf, n, D, L.gu, 2 * d.d_ffn, m->p_gu, s->part, stride, inv, s->st));
        HIPCHK(launch_swiglu(dt, s->part, gemm_out_slots(dt, m->p_gu, n, 2 * d.d_ffn, D, inv), stride, n, d.d_ffn,
                             s->ybuf, s->st));
      }
    }
    {
      prev_stride = (size_t)n * D;
      PROF(PROF_DOWN, launch_gemm(dt, s->ybuf, n, d.d_ffn, L.down, D, m->p_down, s->part, prev_stride, inv, s->st));
      prev_slots = gemm_out_slots(dt, m->p_down, n, D, d.d_ffn, inv);
    }
  }
  if (logits_out) {
    HIPCHK(launch_resid_norm(dt, s->x, s->part, prev_slots, prev_stride, n, D, m->final_norm, d.rms_eps, s->ybuf,
                             s->st));
    PROF(PROF_LM, launch_gemm(dt, s->ybuf, n, D, m->lm_head, d.vocab, m->p_lm, logits_out, (size_t)n * d.vocab, inv, s->st));
  }
  rc = prof_end(s, PROF_FWD, fslot);
  if (rc) return rc;
  if (s->tracing) {
    TraceRec rec;
    rec.seq = R.seq;
    rec.pos = R.pos;
    rec.hi = R.hi;
    rec.lora = R.lora;
    if (!any_lora) std::fill(rec.lora.begin(), rec.lora.end(), 0);
    rec.tok.resize(n);
    HIPCHK(hipMemcpyAsync(rec.tok.data(), dm.tok, (size_t)n * 4, hipMemcpyDeviceToHost, s->st));
    if (logits_out) {
      rec.logits.resize((size_t)n * d.vocab);
      HIPCHK(hipMemcpyAsync(rec.logits.data(), logits_out, rec.logits.size() * 4, hipMemcpyDeviceToHost, s->st));
    }
    HIPCHK(hipStreamSynchronize(s->st));
    s->trace.push_back(std::move(rec));
  }
  return TRI_OK;
}

int sample(tri_session* s, int which, const HostRows& R, const float* logits, float threshold, int status_slot) {
  Meta dm = meta_ptrs(s->dints, s->o_meta[which], s->mlay[which]);
  const int nb = R.block_start.empty() ? 0 : (int)R.block_start.size() - 1;
  HIPCHK(launch_sample_commit(logits, R.n(), s->m->d.vocab, dm.kind, dm.block_start, nb, threshold,
                              s->dints + s->o_out_tok, s->dconf, s->dints + s->o_out_commit,
                              s->dints + s->o_status + status_slot, s->vws, s->st));
  return TRI_OK;
}

int d2h_ints(tri_session* s, size_t off, size_t n) {
  HIPCHK(hipMemcpyAsync(s->hints + off, s->dints + off, n * 4, hipMemcpyDeviceToHost, s->st));
  return TRI_OK;
}

// After a step's synchronisation: a V value that left the fp16 range of the
// V cache (status[3], set by the RoPE/cache-write kernels; cleared here), or
// non-finite logits in one of the step's first nslots sampling slots.  Either
// fails the call with TRI_ENUMERIC before any sequence state moves.
int check_status(tri_session* s, int nslots, const char* what) {
  if (s->hints[s->o_status + 3]) {
    s->hints[s->o_status + 3] = 0;
    HIPCHK(hipMemsetAsync(s->dints + s->o_status + 3, 0, 4, s->st));
    HIPCHK(hipStreamSynchronize(s->st));
    return fail(TRI_ENUMERIC, "%s: a V value lies outside the fp16 range of the V cache (|v| > 65504)", what);
  }
  for (int i = 0; i < nslots; ++i)
    if (s->hints[s->o_status + i]) return fail(TRI_ENUMERIC, "non-finite logits in %s", what);
  return TRI_OK;
}

int check_seq(tri_session* s, int seq) {
  if (!s) return fail(TRI_EINVAL, "null session");
  if (seq < 0 || seq >= s->max_batch) return fail(TRI_EINVAL, "seq %d out of range [0,%d)", seq, s->max_batch);
  return TRI_OK;
}

void pending_rows(const Seq& S, int seq, HostRows& R, int last_kind) {
  const int L = (int)S.tokens.size();
  for (int p = S.kv_len; p < L; ++p) R.add(S.tokens[p], p, p + 1, seq, 0, p == L - 1 ? last_kind : 0);
}

// ------------------------------------------------------------------ modes
// Carried quadratic-speculation drafts belong to the state they were drafted
// from: any other step, prefill, append or rollback of the sequence drops them.
void drop_qdrafts(tri_session* s, const std::vector<int>& act) {
  for (int b : act) s->seqs[b].qdrafts.clear();
}

int step_ar(tri_session* s, const std::vector<int>& act, int stride, int32_t* out_tokens, tri_seq_stats* st) {
  drop_qdrafts(s, act);
  HostRows R;
  std::vector<int> last_row(act.size());
  for (size_t j = 0; j < act.size(); ++j) {
    pending_rows(s->seqs[act[j]], act[j], R, 1);
    last_row[j] = R.n() - 1;
    R.close_slot(act[j]);
  }
  int rc = stage_meta(s, 0, R, {}, {});
  if (!rc) rc = upload_meta(s, 0);
  if (!rc) rc = forward(s, 0, R, s->logits);
  if (!rc) rc = sample(s, 0, R, s->logits, 0.f, 0);
  if (!rc) rc = d2h_ints(s, s->o_out_tok, R.n());
  if (!rc) rc = d2h_ints(s, s->o_status, 4);
  if (rc) return rc;
  HIPCHK(hipStreamSynchronize(s->st));
  rc = check_status(s, 1, "AR step");
  if (rc) return rc;
  for (size_t j = 0; j < act.size(); ++j) {
    Seq& S = s->seqs[act[j]];
    const int L = (int)S.tokens.size();
    const int tok = s->hints[s->o_out_tok + last_row[j]];
    S.kv_len = L;
    S.written_hi = L;
    S.tokens.push_back(tok);
    out_tokens[(size_t)act[j] * stride] = tok;
    if (st) st[act[j]] = tri_seq_stats{1, 1, -1, 0};
  }
  return TRI_OK;
}

// order (optional): the positions of each block in the order they were committed.
int step_diffusion(tri_session* s, const std::vector<int>& act, int B, float tau, int stride, int32_t* out_tokens,
                   tri_seq_stats* st, std::vector<std::vector<int>>* order = nullptr, bool use_sched = true) {
  drop_qdrafts(s, act);
  const int mask = s->m->d.vocab;
  const size_t na = act.size();
  std::vector<std::vector<int32_t>> y(na, std::vector<int32_t>(B, mask));
  std::vector<std::vector<char>> done(na, std::vector<char>(B, 0));
  std::vector<int> remaining(na, B), fwd(na, 0), flags(na, 0);
  bool first = true;
  for (;;) {
    HostRows R;
    std::vector<int> blk_row(na, -1);
    for (size_t j = 0; j < na; ++j) {
      if (remaining[j] == 0) continue;
      const Seq& S = s->seqs[act[j]];
      const int L = (int)S.tokens.size();
      if (first) pending_rows(S, act[j], R, 0);
      R.block_start.push_back(R.n());
      blk_row[j] = R.n();
      for (int i = 0; i < B; ++i) R.add(y[j][i], L + i, L + B, act[j], 0, done[j][i] ? 3 : 2);
      R.close_slot(act[j]);
    }
    if (R.n() == 0) break;
    R.block_start.push_back(R.n());
    int rc = stage_meta(s, 0, R, {}, {});
    if (!rc) rc = upload_meta(s, 0);
    if (!rc) rc = forward(s, 0, R, s->logits);
    if (!rc) rc = sample(s, 0, R, s->logits, tau, 0);
    if (!rc) rc = d2h_ints(s, s->o_out_tok, R.n());
    if (!rc) rc = d2h_ints(s, s->o_out_commit, R.n());
    if (!rc) rc = d2h_ints(s, s->o_status, 4);
    if (rc) return rc;
    HIPCHK(hipMemcpyAsync(s->hconf, s->dconf, (size_t)R.n() * 4, hipMemcpyDeviceToHost, s->st));
    HIPCHK(hipStreamSynchronize(s->st));
    rc = check_status(s, 1, "diffusion step");
    if (rc) return rc;
    for (size_t j = 0; j < na; ++j) {
      if (blk_row[j] < 0) continue;
      const std::vector<int32_t>& sched = s->seqs[act[j]].sched;
      if (use_sched && !sched.empty()) {
        // the n most confident masked positions (lowest position on ties)
        // replace the threshold rule's commits
        std::vector<int> cand;
        for (int i = 0; i < B; ++i)
          if (!done[j][i]) cand.push_back(i);
        const float* cf = s->hconf + blk_row[j];
        std::stable_sort(cand.begin(), cand.end(), [&](int a, int b) { return cf[a] > cf[b]; });
        const size_t n = std::min<size_t>(cand.size(), (size_t)sched[fwd[j] % sched.size()]);
        for (int i = 0; i < B; ++i) s->hints[s->o_out_commit + blk_row[j] + i] = 0;
        for (size_t c = 0; c < n; ++c) s->hints[s->o_out_commit + blk_row[j] + cand[c]] = 1;
      }
      ++fwd[j];
      for (int i = 0; i < B; ++i) {
        const int r = blk_row[j] + i;
        if (done[j][i] || !s->hints[s->o_out_commit + r]) continue;
        y[j][i] = s->hints[s->o_out_tok + r];
        done[j][i] = 1;
        --remaining[j];
        if (order) (*order)[j].push_back(i);
        if (std::fabs(s->hconf[r] - tau) < 1e-6f) ++flags[j];
      }
    }
    first = false;
  }
  for (size_t j = 0; j < na; ++j) {
    Seq& S = s->seqs[act[j]];
    const int L = (int)S.tokens.size();
    S.kv_len = L;
    S.written_hi = L;
    S.tokens.insert(S.tokens.end(), y[j].begin(), y[j].end());
    for (int i = 0; i < B; ++i) out_tokens[(size_t)act[j] * stride + i] = y[j][i];
    if (st) st[act[j]] = tri_seq_stats{B, fwd[j], -1, flags[j]};
  }
  return TRI_OK;
}

// The parallel pass of the speed-of-light analysis [Notes §7]: from the state
// before the block, every forward commits each masked position whose greedy
// token already equals its target, or, when none does, the next position of
// the serial order.  The sampler still computes every row's greedy token on
// the device; only the comparison with the target runs here.  step[j][i] gets
// the forward at which position i of act[j] was committed, fwd[j] the count.
int sol_parallel(tri_session* s, const std::vector<int>& act, int B, const std::vector<std::vector<int32_t>>& target,
                 const std::vector<std::vector<int>>& order, std::vector<std::vector<int>>& step,
                 std::vector<int>& fwd) {
  const int mask = s->m->d.vocab;
  const size_t na = act.size();
  std::vector<std::vector<int32_t>> y(na, std::vector<int32_t>(B, mask));
  std::vector<int> remaining(na, B), next(na, 0);
  step.assign(na, std::vector<int>(B, -1));
  fwd.assign(na, 0);
  bool first = true;
  for (;;) {
    HostRows R;
    std::vector<int> blk_row(na, -1);
    for (size_t j = 0; j < na; ++j) {
      if (remaining[j] == 0) continue;
      const Seq& S = s->seqs[act[j]];
      const int L = (int)S.tokens.size();
      if (first) pending_rows(S, act[j], R, 0);
      R.block_start.push_back(R.n());
      blk_row[j] = R.n();
      for (int i = 0; i < B; ++i) R.add(y[j][i], L + i, L + B, act[j], 0, y[j][i] == mask ? 2 : 3);
      R.close_slot(act[j]);
    }
    if (R.n() == 0) break;
    R.block_start.push_back(R.n());
    int rc = stage_meta(s, 0, R, {}, {});
    if (!rc) rc = upload_meta(s, 0);
    if (!rc) rc = forward(s, 0, R, s->logits);
    if (!rc) rc = sample(s, 0, R, s->logits, 1.f, 0);
    if (!rc) rc = d2h_ints(s, s->o_out_tok, R.n());
    if (!rc) rc = d2h_ints(s, s->o_status, 4);
    if (rc) return rc;
    HIPCHK(hipStreamSynchronize(s->st));
    rc = check_status(s, 1, "the speed-of-light pass");
    if (rc) return rc;
    for (size_t j = 0; j < na; ++j) {
      if (blk_row[j] < 0) continue;
      std::vector<int> now;
      for (int i = 0; i < B; ++i)
        if (y[j][i] == mask && s->hints[s->o_out_tok + blk_row[j] + i] == target[j][i]) now.push_back(i);
      if (now.empty()) {
        while (y[j][order[j][next[j]]] != mask) ++next[j];
        now.push_back(order[j][next[j]]);
      }
      for (int i : now) {
        y[j][i] = target[j][i];
        step[j][i] = fwd[j];
      }
      remaining[j] -= (int)now.size();
      ++fwd[j];
    }
    first = false;
  }
  return TRI_OK;
}

// One round of two forwards over the stepped sequences.  spec[j] picks the
// mode of act[j]:
// * self-speculation: the draft forward runs the pending rows and k [MASK]
//   rows, the verify forward the k drafts as causal rows; 1..k+1 tokens;
// * AR (mixed steps only): the pending rows, then the row of the token the
//   first forward committed; one greedy token per forward, 2 per step.
// Every token that feeds the second forward moves on the device (gather
// into the verify metadata), so the two forwards run back to back.
int step_round(tri_session* s, const std::vector<int>& act, const std::vector<char>& spec, int k, int stride,
               int32_t* out_tokens, tri_seq_stats* st) {
  drop_qdrafts(s, act);
  const int mask = s->m->d.vocab;
  const size_t na = act.size();
  int nv = 0;
  bool any_ar = false;
  for (size_t j = 0; j < na; ++j) {
    nv += spec[j] ? k : 1;
    any_ar = any_ar || !spec[j];
  }
  const MetaLayout ML = forward_layout(nv, s->max_rows, s->max_batch);  // the second forward's layout
  HostRows D, V;
  std::vector<int32_t> s1, d1, s2, d2;
  const int lora = s->lora_on ? 1 : 0;
  std::vector<int> vrow0(na);
  for (size_t j = 0; j < na; ++j) {
    const Seq& S = s->seqs[act[j]];
    const int L = (int)S.tokens.size();
    const int32_t ars = (int32_t)(s->o_ars + j * (k + 1));
    pending_rows(S, act[j], D, 1);
    const int g0row = D.n() - 1;
    vrow0[j] = V.n();
    // after the first forward: ars[j][0] = g0
    s1.push_back((int32_t)(s->o_out_tok + g0row));
    d1.push_back(ars);
    if (!spec[j]) {
      D.close_slot(act[j]);
      V.add(0, L, L + 1, act[j], 0, 1);  // token g0, gathered after the first forward
      V.close_slot(act[j]);
      s1.push_back((int32_t)(s->o_out_tok + g0row));
      d1.push_back((int32_t)(s->o_meta[1] + ML.tok + vrow0[j]));
      s2.push_back((int32_t)(s->o_out_tok + vrow0[j]));
      d2.push_back(ars + 1);
      continue;
    }
    const int mrow0 = D.n();
    for (int i = 0; i < k; ++i) D.add(mask, L + i, L + k, act[j], lora, 1);
    D.close_slot(act[j]);
    for (int i = 0; i < k; ++i) V.add(0, L + i, L + i + 1, act[j], 0, 1);
    V.close_slot(act[j]);
    // drafts[j][i] = d_i; verify token i = d_i
    for (int i = 0; i < k; ++i) {
      s1.push_back((int32_t)(s->o_out_tok + mrow0 + i));
      d1.push_back((int32_t)(s->o_drafts + j * k + i));
      s1.push_back((int32_t)(s->o_out_tok + mrow0 + i));
      d1.push_back((int32_t)(s->o_meta[1] + ML.tok + vrow0[j] + i));
    }
    // after the verify: ars[j][1 + i] = g_{i+1}
    for (int i = 0; i < k; ++i) {
      s2.push_back((int32_t)(s->o_out_tok + vrow0[j] + i));
      d2.push_back(ars + 1 + i);
    }
  }
  if (V.n() != nv) return fail(TRI_EINVAL, "verify rows");
  int rc = stage_meta(s, 0, D, s1, d1);
  if (!rc) rc = stage_meta(s, 1, V, s2, d2);
  if (rc) return rc;
  Meta m0 = meta_ptrs(s->dints, s->o_meta[0], s->mlay[0]);
  Meta m1 = meta_ptrs(s->dints, s->o_meta[1], s->mlay[1]);
  if (!rc) rc = upload_meta(s, 0);
  if (!rc) rc = upload_meta(s, 1);
  if (!rc) rc = forward(s, 0, D, s->logits);
  if (!rc) rc = sample(s, 0, D, s->logits, 0.f, 0);
  if (rc) return rc;
  HIPCHK(launch_scatter_gather(s->dints, m0.sidx, m0.didx, (int)s1.size(), s->dints, s->st));
  // controlled-acceptance override: replace drafts (and verify tokens) by the reference
  for (size_t j = 0; j < na; ++j) {
    const Seq& S = s->seqs[act[j]];
    if (S.a_star < 0 || !spec[j]) continue;
    if (s->meta_pending[1]) {  // the verify rows' host mirror is rewritten below
      HIPCHK(hipEventSynchronize(s->meta_ev[1]));
      s->meta_pending[1] = false;
    }
    const int L = (int)S.tokens.size();
    int32_t* hd = s->hints + s->o_drafts + j * k;
    for (int i = 0; i < k; ++i) {
      const int p = L + i;
      int32_t t = p < (int)S.ref.size() ? S.ref[p] : 0;
      if (i == S.a_star) t = (t + 1) % mask;
      hd[i] = t;
      s->hints[s->o_meta[1] + ML.tok + vrow0[j] + i] = t;
    }
    HIPCHK(hipMemcpyAsync(s->dints + s->o_drafts + j * k, hd, (size_t)k * 4, hipMemcpyHostToDevice, s->st));
    HIPCHK(hipMemcpyAsync(s->dints + s->o_meta[1] + ML.tok + vrow0[j], s->hints + s->o_meta[1] + ML.tok + vrow0[j],
                          (size_t)k * 4, hipMemcpyHostToDevice, s->st));
  }
  rc = forward(s, 1, V, s->logits);
  if (!rc) rc = sample(s, 1, V, s->logits, 0.f, 1);
  if (rc) return rc;
  HIPCHK(launch_scatter_gather(s->dints, m1.sidx, m1.didx, (int)s2.size(), s->dints, s->st));
  // accept lengths for every sequence; an AR sequence's entries are not read
  HIPCHK(launch_verify_accept(s->dints + s->o_drafts, s->dints + s->o_ars, (int)na, k, s->dints + s->o_accept,
                              s->dints + s->o_committed, nullptr, s->st));
  rc = d2h_ints(s, s->o_accept, na);
  if (!rc) rc = d2h_ints(s, s->o_committed, na * (k + 1));
  if (!rc && any_ar) rc = d2h_ints(s, s->o_ars, na * (k + 1));
  if (!rc) rc = d2h_ints(s, s->o_status, 4);
  if (rc) return rc;
  HIPCHK(hipStreamSynchronize(s->st));
  rc = check_status(s, 2, "a self-speculation / mixed round");
  if (rc) return rc;
  for (size_t j = 0; j < na; ++j) {
    Seq& S = s->seqs[act[j]];
    const int L = (int)S.tokens.size();
    if (!spec[j]) {
      const int32_t* g = s->hints + s->o_ars + j * (k + 1);
      for (int i = 0; i < 2; ++i) {
        S.tokens.push_back(g[i]);
        out_tokens[(size_t)act[j] * stride + i] = g[i];
      }
      S.kv_len = L + 1;
      S.written_hi = L + 1;
      if (st) st[act[j]] = tri_seq_stats{2, 2, -1, 0};
      continue;
    }
    const int a = s->hints[s->o_accept + j];
    const int32_t* c = s->hints + s->o_committed + j * (k + 1);
    for (int i = 0; i <= a; ++i) {
      S.tokens.push_back(c[i]);
      out_tokens[(size_t)act[j] * stride + i] = c[i];
    }
    S.kv_len = L + a;
    S.written_hi = L + a;
    if (st) st[act[j]] = tri_seq_stats{a + 1, 2, a, 0};
  }
  return TRI_OK;
}

int step_selfspec(tri_session* s, const std::vector<int>& act, int k, int stride, int32_t* out_tokens,
                  tri_seq_stats* st) {
  return step_round(s, act, std::vector<char>(act.size(), 1), k, stride, out_tokens, st);
}

// Quadratic self-speculation ([Notes §8.1]; [Blog], performance highlights;
// reading R24): one forward per round.  Per sequence, its pending rows and
// the drafts carried from the previous round are clean causal rows (the AR
// pathway: their greedy tokens g_0..g_n verify the drafts), followed by one
// block of k+1 [MASK] rows at L+b .. L+b+k for every possible accept length
// b = 0..n (the diffusion pathway drafts every outcome's continuation; LoRA
// rows): a block row attends to the cache keys [0, L+b) and to its own
// block.  a = the accept length; g_0..g_a are committed, the K/V of the
// pending rows and d_0..d_{a-1} stay, g_a is the new pending token, and
// block a's greedy tokens at L+a+1 .. L+a+k are the next drafts.  Without
// carried drafts (the first round, or after any other step) the forward is
// the pending rows and block 0, and commits g_0.  The accept length is taken
// on the host from the tokens the sampler returns.
int step_quad(tri_session* s, const std::vector<int>& act, int k, int stride, int32_t* out_tokens,
              tri_seq_stats* st) {
  const int mask = s->m->d.vocab;
  const int lora = s->lora_on ? 1 : 0;
  const size_t na = act.size();
  HostRows R;
  R.blk_len = k + 1;
  std::vector<int> g0row(na), blk0(na);
  std::vector<std::vector<int32_t>> drafts(na);
  for (size_t j = 0; j < na; ++j) {
    Seq& S = s->seqs[act[j]];
    const int L = (int)S.tokens.size();
    drafts[j] = S.qdrafts;
    if (S.a_star >= 0 && !drafts[j].empty()) {  // controlled acceptance (benchmark hook)
      for (int i = 0; i < (int)drafts[j].size(); ++i) {
        int32_t t = L + i < (int)S.ref.size() ? S.ref[L + i] : 0;
        if (i == S.a_star) t = (t + 1) % mask;
        drafts[j][i] = t;
      }
    }
    pending_rows(S, act[j], R, 1);
    g0row[j] = R.n() - 1;
    const int nd = (int)drafts[j].size();
    for (int i = 0; i < nd; ++i) R.add(drafts[j][i], L + i, L + i + 1, act[j], 0, 1);
    blk0[j] = R.n();
    for (int b = 0; b <= nd; ++b) {
      const int first = R.n();
      for (int i = 0; i <= k; ++i) R.add(mask, L + b + i, L + b, act[j], lora, 1, first);
    }
    R.close_slot(act[j]);
  }
  int rc = stage_meta(s, 0, R, {}, {});
  if (!rc) rc = upload_meta(s, 0);
  if (!rc) rc = forward(s, 0, R, s->logits);
  if (!rc) rc = sample(s, 0, R, s->logits, 0.f, 0);
  if (!rc) rc = d2h_ints(s, s->o_out_tok, R.n());
  if (!rc) rc = d2h_ints(s, s->o_status, 4);
  if (rc) return rc;
  HIPCHK(hipStreamSynchronize(s->st));
  rc = check_status(s, 1, "a quadratic self-speculation round");
  if (rc) return rc;
  for (size_t j = 0; j < na; ++j) {
    Seq& S = s->seqs[act[j]];
    const int L = (int)S.tokens.size();
    const int nd = (int)drafts[j].size();
    const int32_t* g = s->hints + s->o_out_tok + g0row[j];
    int a = 0;
    while (a < nd && drafts[j][a] == g[a]) ++a;
    for (int i = 0; i <= a; ++i) {
      S.tokens.push_back(g[i]);
      out_tokens[(size_t)act[j] * stride + i] = g[i];
    }
    S.kv_len = L + a;
    S.written_hi = L + a;
    const int32_t* nb = s->hints + s->o_out_tok + blk0[j] + a * (k + 1) + 1;
    S.qdrafts.assign(nb, nb + k);
    if (st) st[act[j]] = tri_seq_stats{a + 1, 1, a, 0};
  }
  return TRI_OK;
}

// Mode choice by concurrency ([Notes] §2 mode table and §11; [Digest], Limitations): forward cost from
// the measured points, linear between them, the first point's time below
// the first, the line through the last two beyond the last.
double cost_ms(const int32_t* gr, const double* gm, int ng, double rows) {
  if (ng == 1 || rows <= gr[0]) return gm[0];
  for (int i = 1; i < ng; ++i)
    if (rows <= gr[i] || i == ng - 1)
      return gm[i - 1] + (gm[i] - gm[i - 1]) * (rows - gr[i - 1]) / (double)(gr[i] - gr[i - 1]);
  return gm[ng - 1];
}

}  // namespace

// =================================================================== C-ABI
extern "C" {

const char* tri_last_error(void) { return g_err.c_str(); }

}  // extern "C"

namespace {

int validate_desc(const tri_model_desc& d) {
  if (d.n_layers <= 0 || d.d_model <= 0 || d.n_q_heads <= 0 || d.n_kv_heads <= 0 || d.head_dim <= 0 ||
      d.d_ffn <= 0 || d.vocab <= 0 || d.lora_rank < 0)
    return fail(TRI_EINVAL, "non-positive model dimension");
  if (d.n_q_heads % d.n_kv_heads) return fail(TRI_EINVAL, "n_q_heads must be a multiple of n_kv_heads");
  if (d.head_dim % 2) return fail(TRI_EINVAL, "head_dim must be even");
  if (d.d_model > 8192 || d.d_model % 4) return fail(TRI_EINVAL, "d_model must be a multiple of 4, <= 8192");
  if (d.d_ffn % 16) return fail(TRI_EINVAL, "d_ffn must be a multiple of 16");
  if (!(d.rms_eps > 0) || !(d.rope_base > 1)) return fail(TRI_EINVAL, "bad rms_eps/rope_base");
  if (d.dtype == TRI_BF16) {
    if (d.head_dim != 128) return fail(TRI_EINVAL, "bf16 models need head_dim == 128");
    const int qd = d.n_q_heads * d.head_dim, kd = d.n_kv_heads * d.head_dim;
    if (d.d_model % 64 || qd % 64 || kd % 64 || d.d_ffn % 64 || (d.lora_rank % 64))
      return fail(TRI_EINVAL, "bf16 models need d, hq*hd, hkv*hd, ffn and lora_rank multiples of 64");
  } else if (d.dtype == TRI_F32) {
    if (d.head_dim > 128) return fail(TRI_EINVAL, "float32 models need head_dim <= 128");
  } else {
    return fail(TRI_EINVAL, "bad dtype %d", d.dtype);
  }
  return TRI_OK;
}

// Offsets of everything the model keeps in its buffer.
struct ModelLayout {
  struct L {
    size_t qkv, o, gu, down, n1, n2, la, lb;
  };
  size_t embed, final_norm, lm_head, total;
  std::vector<L> layers;
};

// GEMM plans of a model; the packed weight layout depends on them.
struct ModelPlans {
  GemmPlan qkv, o, gu, down, lm, la, lb;
};

ModelPlans model_plans(const tri_model_desc& d) {
  const int qd = d.n_q_heads * d.head_dim, kd = d.n_kv_heads * d.head_dim;
  ModelPlans P;
  P.qkv = gemm_plan(qd + 2 * kd, d.d_model, d.dtype);
  P.o = gemm_plan(d.d_model, qd, d.dtype);
  P.gu = gemm_plan(2 * d.d_ffn, d.d_model, d.dtype);
  P.down = gemm_plan(d.d_model, d.d_ffn, d.dtype);
  P.lm = gemm_plan(d.vocab, d.d_model, d.dtype, /*unsplit=*/true);
  P.la = d.lora_rank > 0 ? gemm_plan(d.lora_rank, qd, d.dtype) : GemmPlan{1, qd};
  P.lb = d.lora_rank > 0 ? gemm_plan(d.d_model, d.lora_rank, d.dtype) : GemmPlan{0, 0};
  return P;
}

ModelLayout model_layout(const tri_model_desc& d) {
  ModelLayout M;
  const ModelPlans P = model_plans(d);
  const size_t esz = d.dtype == TRI_BF16 ? 2 : 4;
  const int qd = d.n_q_heads * d.head_dim, kd = d.n_kv_heads * d.head_dim;
  size_t off = 0;
  auto take = [&](size_t bytes) {
    const size_t r = off;
    off = align256(off + bytes);
    return r;
  };
  M.embed = take((size_t)(d.vocab + 1) * d.d_model * esz);
  M.layers.resize(d.n_layers);
  for (auto& L : M.layers) {
    L.qkv = take(gemm_packed_bytes(P.qkv, qd + 2 * kd, d.d_model, d.dtype));
    L.o = take(gemm_packed_bytes(P.o, d.d_model, qd, d.dtype));
    L.gu = take(gemm_packed_bytes(P.gu, 2 * d.d_ffn, d.d_model, d.dtype));
    L.down = take(gemm_packed_bytes(P.down, d.d_model, d.d_ffn, d.dtype));
    L.n1 = take((size_t)d.d_model * 4);
    L.n2 = take((size_t)d.d_model * 4);
    L.la = d.lora_rank > 0 ? take(gemm_packed_bytes(P.la, d.lora_rank, qd, d.dtype)) : 0;
    L.lb = d.lora_rank > 0 ? take(gemm_packed_bytes(P.lb, d.d_model, d.lora_rank, d.dtype)) : 0;
  }
  M.final_norm = take((size_t)d.d_model * 4);
  M.lm_head = take(gemm_packed_bytes(P.lm, d.vocab, d.d_model, d.dtype));
  M.total = off;
  return M;
}

}  // namespace

extern "C" {

int tri_model_bytes(const tri_model_desc* desc, size_t* bytes) {
  if (!desc || !bytes) return fail(TRI_EINVAL, "null argument");
  int rc = validate_desc(*desc);
  if (rc) return rc;
  *bytes = model_layout(*desc).total;
  return TRI_OK;
}

int tri_model_create(const tri_model_desc* desc, const void* const* weights, int n_weights, void* model_buf,
                     size_t bytes, void* stream, tri_model** out) {
  if (!desc || !weights || !out || !model_buf) return fail(TRI_EINVAL, "null argument");
  const tri_model_desc& d = *desc;
  int rc = validate_desc(d);
  if (rc) return rc;
  const int expect = 1 + 9 * d.n_layers + 2 + (d.lora_rank > 0 ? 2 * d.n_layers : 0);
  if (n_weights != expect) return fail(TRI_EINVAL, "expected %d weight pointers, got %d", expect, n_weights);
  for (int i = 0; i < n_weights; ++i)
    if (!weights[i]) return fail(TRI_EINVAL, "weight pointer %d is null", i);
  const ModelLayout ML = model_layout(d);
  const ModelPlans P = model_plans(d);
  if (bytes < ML.total) return fail(TRI_ECAPACITY, "model buffer has %zu bytes, needs %zu", bytes, ML.total);
  if (reinterpret_cast<uintptr_t>(model_buf) & 255) return fail(TRI_EINVAL, "model buffer must be 256-byte aligned");
  hipStream_t st = static_cast<hipStream_t>(stream);
  char* base = static_cast<char*>(model_buf);
  const size_t esz = d.dtype == TRI_BF16 ? 2 : 4;
  const int qd = d.n_q_heads * d.head_dim, kd = d.n_kv_heads * d.head_dim;
  const int dt = d.dtype;
  // Copy the embedding and norm gains, repack every projection matrix.
  int w = 0;
  HIPCHK(hipMemcpyAsync(base + ML.embed, weights[w++], (size_t)(d.vocab + 1) * d.d_model * esz,
                        hipMemcpyDeviceToDevice, st));
  std::vector<int> la_idx(d.n_layers), lb_idx(d.n_layers);
  for (int l = 0; l < d.n_layers; ++l) {
    const ModelLayout::L& L = ML.layers[l];
    WSeg qkv[3] = {{weights[w], qd}, {weights[w + 1], kd}, {weights[w + 2], kd}};
    HIPCHK(launch_pack(dt, qkv, 3, qd + 2 * kd, d.d_model, P.qkv, base + L.qkv, PACK_PLAIN, st));
    WSeg o = {weights[w + 3], d.d_model};
    HIPCHK(launch_pack(dt, &o, 1, d.d_model, qd, P.o, base + L.o, PACK_PLAIN, st));
    WSeg gu[2] = {{weights[w + 4], d.d_ffn}, {weights[w + 5], d.d_ffn}};
    HIPCHK(launch_pack(dt, gu, 2, 2 * d.d_ffn, d.d_model, P.gu, base + L.gu, PACK_GATEUP, st));
    WSeg dn = {weights[w + 6], d.d_model};
    HIPCHK(launch_pack(dt, &dn, 1, d.d_model, d.d_ffn, P.down, base + L.down, PACK_PLAIN, st));
    HIPCHK(hipMemcpyAsync(base + L.n1, weights[w + 7], (size_t)d.d_model * 4, hipMemcpyDeviceToDevice, st));
    HIPCHK(hipMemcpyAsync(base + L.n2, weights[w + 8], (size_t)d.d_model * 4, hipMemcpyDeviceToDevice, st));
    w += 9;
  }
  HIPCHK(hipMemcpyAsync(base + ML.final_norm, weights[w++], (size_t)d.d_model * 4, hipMemcpyDeviceToDevice, st));
  {
    WSeg lm = {weights[w++], d.vocab};
    HIPCHK(launch_pack(dt, &lm, 1, d.vocab, d.d_model, P.lm, base + ML.lm_head, PACK_PLAIN, st));
  }
  if (d.lora_rank > 0)
    for (int l = 0; l < d.n_layers; ++l) {
      WSeg a = {weights[w++], d.lora_rank};
      HIPCHK(launch_pack(dt, &a, 1, d.lora_rank, qd, P.la, base + ML.layers[l].la, PACK_PLAIN, st));
      WSeg b = {weights[w++], d.d_model};
      HIPCHK(launch_pack(dt, &b, 1, d.d_model, d.lora_rank, P.lb, base + ML.layers[l].lb, PACK_PLAIN, st));
    }
  HIPCHK(hipStreamSynchronize(st));
  tri_model* m = new tri_model();
  m->d = d;
  m->esz = esz;
  m->embed = base + ML.embed;
  m->layers.resize(d.n_layers);
  for (int l = 0; l < d.n_layers; ++l) {
    const ModelLayout::L& L = ML.layers[l];
    Layer& Y = m->layers[l];
    Y.qkv = base + L.qkv;
    Y.o = base + L.o;
    Y.gu = base + L.gu;
    Y.down = base + L.down;
    Y.n1 = reinterpret_cast<const float*>(base + L.n1);
    Y.n2 = reinterpret_cast<const float*>(base + L.n2);
    Y.la = d.lora_rank > 0 ? base + L.la : nullptr;
    Y.lb = d.lora_rank > 0 ? base + L.lb : nullptr;
  }
  m->final_norm = reinterpret_cast<const float*>(base + ML.final_norm);
  m->lm_head = base + ML.lm_head;
  m->qkv_n = qd + 2 * kd;
  m->p_qkv = P.qkv;
  m->p_o = P.o;
  m->p_gu = P.gu;
  m->p_down = P.down;
  m->p_lm = P.lm;
  m->p_la = P.la;
  m->p_lb = P.lb;
  *out = m;
  return TRI_OK;
}

int tri_model_destroy(tri_model* model) {
  delete model;
  return TRI_OK;
}

int tri_session_bytes(const tri_model* m, int max_batch, int max_ctx, int max_rows, size_t* bytes) {
  if (!m || !bytes) return fail(TRI_EINVAL, "null argument");
  if (max_batch <= 0 || max_batch > 64 || max_ctx <= 1 || max_ctx > (1 << 20) || max_rows <= 0 || max_rows > 8192)
    return fail(TRI_EINVAL, "bad session limits (batch 1..64, ctx 2..2^20, rows 1..8192)");
  *bytes = session_layout(m, max_batch, max_ctx, max_rows).total;
  return TRI_OK;
}

int tri_session_create(const tri_model* m, int max_batch, int max_ctx, int max_rows, void* workspace, size_t bytes,
                       void* stream, tri_session** out) {
  if (!m || !workspace || !out) return fail(TRI_EINVAL, "null argument");
  size_t need = 0;
  int rc = tri_session_bytes(m, max_batch, max_ctx, max_rows, &need);
  if (rc) return rc;
  if (bytes < need) return fail(TRI_ECAPACITY, "workspace has %zu bytes, needs %zu", bytes, need);
  if (reinterpret_cast<uintptr_t>(workspace) & 255) return fail(TRI_EINVAL, "workspace must be 256-byte aligned");
  const SessionLayout S = session_layout(m, max_batch, max_ctx, max_rows);
  tri_session* s = new tri_session();
  s->m = m;
  s->max_batch = max_batch;
  s->max_ctx = max_ctx;
  s->ctx = S.ctx;
  s->max_rows = max_rows;
  s->st = static_cast<hipStream_t>(stream);
  s->kv_split = S.kv_split;
  char* base = static_cast<char*>(workspace);
  s->kbuf = base + S.k;
  s->vbuf = base + S.v;
  s->css = S.css;
  s->rope = reinterpret_cast<float*>(base + S.rope);
  s->x = reinterpret_cast<float*>(base + S.x);
  s->ybuf = base + S.y;
  s->ybuf2 = base + S.y2;
  s->qbuf = base + S.q;
  s->abuf = base + S.a;
  s->part = reinterpret_cast<float*>(base + S.part);
  s->part2 = reinterpret_cast<float*>(base + S.part2);
  s->attn_ws = base + S.attn;
  s->kscr = base + S.kscr;
  s->vscr = base + S.vscr;
  s->logits = reinterpret_cast<float*>(base + S.logits);
  s->vws = base + S.vws;
  s->dints = reinterpret_cast<int32_t*>(base + S.ints);
  s->dconf = reinterpret_cast<float*>(base + S.conf);
  s->nints = S.nints;
  s->o_meta[0] = S.o_meta0;
  s->o_meta[1] = S.o_meta1;
  s->o_out_tok = S.o_out_tok;
  s->o_out_commit = S.o_out_commit;
  s->o_status = S.o_status;
  s->o_accept = S.o_accept;
  s->o_committed = S.o_committed;
  s->o_kvlen = S.o_kvlen;
  s->o_drafts = S.o_drafts;
  s->o_ars = S.o_ars;
  s->seqs.resize(max_batch);
  s->hints = nullptr;
  s->hconf = nullptr;
  hipError_t e = hipHostMalloc(reinterpret_cast<void**>(&s->hints), S.nints * 4, hipHostMallocDefault);
  if (e == hipSuccess)
    e = hipHostMalloc(reinterpret_cast<void**>(&s->hconf), (size_t)max_rows * 4 + 64, hipHostMallocDefault);
  if (e != hipSuccess) {
    if (s->hints) (void)hipHostFree(s->hints);
    delete s;
    return fail(TRI_EHIP, "hipHostMalloc: %s", hipGetErrorString(e));
  }
  memset(s->hints, 0, S.nints * 4);
  for (int i = 0; i < 2 && e == hipSuccess; ++i) e = hipEventCreateWithFlags(&s->meta_ev[i], hipEventDisableTiming);
  if (e != hipSuccess) {
    for (int i = 0; i < 2; ++i)
      if (s->meta_ev[i]) (void)hipEventDestroy(s->meta_ev[i]);
    (void)hipHostFree(s->hints);
    (void)hipHostFree(s->hconf);
    delete s;
    return fail(TRI_EHIP, "hipEventCreate: %s", hipGetErrorString(e));
  }
  // RoPE table: angle pos * base^(-2i/hd) in double, stored as float cos/sin.
  const tri_model_desc& d = m->d;
  const int half = d.head_dim / 2;
  std::vector<float> tab((size_t)S.ctx * half * 2);
  for (int p = 0; p < S.ctx; ++p)
    for (int i = 0; i < half; ++i) {
      const double th = (double)p * std::pow((double)d.rope_base, -2.0 * i / d.head_dim);
      tab[((size_t)p * half + i) * 2] = (float)std::cos(th);
      tab[((size_t)p * half + i) * 2 + 1] = (float)std::sin(th);
    }
  e = hipMemcpyAsync(s->rope, tab.data(), tab.size() * 4, hipMemcpyHostToDevice, s->st);
  if (e == hipSuccess) e = hipMemcpyAsync(s->dints, s->hints, S.nints * 4, hipMemcpyHostToDevice, s->st);
  // The KV cache starts cleared: attention stages whole 64-key tiles, so slots
  // past a sequence's length are read (and masked) and must hold finite values.
  if (e == hipSuccess) e = launch_zero_f32(reinterpret_cast<float*>(s->kbuf), (S.v - S.k) / 4 * 2, s->st);
  if (e == hipSuccess) e = hipStreamSynchronize(s->st);
  if (e != hipSuccess) {
    for (hipEvent_t ev : s->meta_ev) (void)hipEventDestroy(ev);
    (void)hipHostFree(s->hints);
    (void)hipHostFree(s->hconf);
    delete s;
    return fail(TRI_EHIP, "session init: %s", hipGetErrorString(e));
  }
  *out = s;
  return TRI_OK;
}

int tri_session_destroy(tri_session* s) {
  if (!s) return TRI_OK;
  (void)hipStreamSynchronize(s->st);
  for (hipEvent_t e : s->ev) (void)hipEventDestroy(e);
  for (hipEvent_t e : s->meta_ev)
    if (e) (void)hipEventDestroy(e);
  (void)hipHostFree(s->hints);
  (void)hipHostFree(s->hconf);
  delete s;
  return TRI_OK;
}

int tri_prefill(tri_session* s, int seq, const int32_t* tokens, int n) {
  int rc = check_seq(s, seq);
  if (rc) return rc;
  if (!tokens || n <= 0) return fail(TRI_EINVAL, "empty prompt");
  if (n >= s->max_ctx) return fail(TRI_ECAPACITY, "prompt of %d tokens leaves no room in max_ctx %d", n, s->max_ctx);
  for (int i = 0; i < n; ++i)
    if (tokens[i] < 0 || tokens[i] >= s->m->d.vocab) return fail(TRI_EINVAL, "prompt token %d out of range", i);
  Seq& S = s->seqs[seq];
  S.tokens.assign(tokens, tokens + n);
  S.kv_len = 0;
  S.written_hi = 0;
  S.active = true;
  S.a_star = -1;
  S.ref.clear();
  S.sched.clear();
  S.qdrafts.clear();
  for (int b = 0; b < n - 1; b += s->max_rows) {
    const int e = std::min(n - 1, b + s->max_rows);
    HostRows R;
    for (int p = b; p < e; ++p) R.add(tokens[p], p, p + 1, seq, 0, 0);
    R.close_slot(seq);
    rc = stage_meta(s, 0, R, {}, {});
    if (!rc) rc = upload_meta(s, 0);
    if (!rc) rc = forward(s, 0, R, nullptr);
    if (rc) {
      S.active = false;
      return rc;
    }
  }
  rc = d2h_ints(s, s->o_status, 4);
  if (rc) {
    S.active = false;
    return rc;
  }
  HIPCHK(hipStreamSynchronize(s->st));
  rc = check_status(s, 0, "prefill");
  if (rc) {
    S.active = false;
    return rc;
  }
  S.kv_len = n - 1;
  S.written_hi = n - 1;
  return TRI_OK;
}

int tri_decode_step(tri_session* s, int mode, int block, float threshold, int32_t* out_tokens,
                    tri_seq_stats* out_stats) {
  if (!s || !out_tokens) return fail(TRI_EINVAL, "null argument");
  if (mode != TRI_AR && mode != TRI_DIFFUSION && mode != TRI_SELFSPEC && mode != TRI_QUADSPEC)
    return fail(TRI_EINVAL, "bad mode %d", mode);
  if (block < 1 || block > 64) return fail(TRI_EINVAL, "block %d outside [1, 64]", block);
  if (mode == TRI_QUADSPEC && block > 63) return fail(TRI_EINVAL, "quadratic self-speculation needs k <= 63");
  if (mode == TRI_DIFFUSION && !(threshold >= 0.f && threshold <= 1.f))
    return fail(TRI_EINVAL, "threshold must be in [0, 1]");
  std::vector<int> act;
  int rows = 0;
  for (int b = 0; b < s->max_batch; ++b) {
    const Seq& S = s->seqs[b];
    if (!S.active) continue;
    const int L = (int)S.tokens.size();
    const int pend = L - S.kv_len;
    if (pend < 1) return fail(TRI_ESTATE, "sequence %d has no pending token (kv_len %d, L %d)", b, S.kv_len, L);
    const int nd = mode == TRI_QUADSPEC ? (int)S.qdrafts.size() : 0;  // carried drafts
    const int need = mode == TRI_AR ? L + 1
                     : mode == TRI_DIFFUSION ? L + block
                     : mode == TRI_SELFSPEC ? L + block + 1
                                            : L + nd + block + 1;  // the last block's last row
    if (need > s->max_ctx) return fail(TRI_ECAPACITY, "sequence %d would pass max_ctx %d", b, s->max_ctx);
    const int r = mode == TRI_AR ? pend
                  : mode == TRI_DIFFUSION ? pend + block
                  : mode == TRI_SELFSPEC ? std::max(pend + block, block)
                                         : pend + nd + (nd + 1) * (block + 1);
    rows += r;
    act.push_back(b);
  }
  if (act.empty()) return fail(TRI_ESTATE, "no prefilled sequence");
  if (rows > s->max_rows) return fail(TRI_ECAPACITY, "step needs %d rows, session allows %d", rows, s->max_rows);
  const int stride = block + 1;
  for (size_t i = 0; i < (size_t)s->max_batch * stride; ++i) out_tokens[i] = -1;
  if (out_stats)
    for (int b = 0; b < s->max_batch; ++b) out_stats[b] = tri_seq_stats{0, 0, -1, 0};
  s->ev_used = s->prof_class >= 0 ? s->ev_used : 0;
  switch (mode) {
    case TRI_AR: return step_ar(s, act, stride, out_tokens, out_stats);
    case TRI_DIFFUSION: return step_diffusion(s, act, block, threshold, stride, out_tokens, out_stats);
    case TRI_QUADSPEC: return step_quad(s, act, block, stride, out_tokens, out_stats);
    default: return step_selfspec(s, act, block, stride, out_tokens, out_stats);
  }
}

int tri_decode_step_mixed(tri_session* s, const int32_t* modes, int block, int32_t* out_tokens,
                          tri_seq_stats* out_stats) {
  if (!s || !modes || !out_tokens) return fail(TRI_EINVAL, "null argument");
  if (block < 1 || block > 64) return fail(TRI_EINVAL, "block %d outside [1, 64]", block);
  std::vector<int> act;
  std::vector<char> spec;
  int rows1 = 0, rows2 = 0;
  for (int b = 0; b < s->max_batch; ++b) {
    const int md = modes[b];
    if (md < 0) continue;
    if (md != TRI_AR && md != TRI_SELFSPEC)
      return fail(TRI_EINVAL, "mode %d of sequence %d cannot take part in a mixed step", md, b);
    const Seq& S = s->seqs[b];
    if (!S.active) return fail(TRI_ESTATE, "sequence %d is not prefilled", b);
    const int L = (int)S.tokens.size();
    const int pend = L - S.kv_len;
    if (pend < 1) return fail(TRI_ESTATE, "sequence %d has no pending token (kv_len %d, L %d)", b, S.kv_len, L);
    const bool sp = md == TRI_SELFSPEC;
    if ((sp ? L + block + 1 : L + 2) > s->max_ctx)
      return fail(TRI_ECAPACITY, "sequence %d would pass max_ctx %d", b, s->max_ctx);
    rows1 += pend + (sp ? block : 0);
    rows2 += sp ? block : 1;
    act.push_back(b);
    spec.push_back(sp ? 1 : 0);
  }
  if (act.empty()) return fail(TRI_ESTATE, "no sequence to step");
  if (std::max(rows1, rows2) > s->max_rows)
    return fail(TRI_ECAPACITY, "step needs %d rows, session allows %d", std::max(rows1, rows2), s->max_rows);
  const int stride = block + 1;
  for (size_t i = 0; i < (size_t)s->max_batch * stride; ++i) out_tokens[i] = -1;
  if (out_stats)
    for (int b = 0; b < s->max_batch; ++b) out_stats[b] = tri_seq_stats{0, 0, -1, 0};
  s->ev_used = s->prof_class >= 0 ? s->ev_used : 0;
  return step_round(s, act, spec, block, stride, out_tokens, out_stats);
}

int tri_sol_block(tri_session* s, int block, int32_t* out_target, int32_t* out_order, int32_t* out_step,
                  int32_t* out_forwards) {
  if (!s || !out_target || !out_order || !out_step || !out_forwards) return fail(TRI_EINVAL, "null argument");
  if (block < 1 || block > 64) return fail(TRI_EINVAL, "block %d outside [1, 64]", block);
  std::vector<int> act;
  int rows = 0;
  for (int b = 0; b < s->max_batch; ++b) {
    const Seq& S = s->seqs[b];
    if (!S.active) continue;
    const int L = (int)S.tokens.size();
    const int pend = L - S.kv_len;
    if (pend < 1) return fail(TRI_ESTATE, "sequence %d has no pending token (kv_len %d, L %d)", b, S.kv_len, L);
    if (L + block > s->max_ctx) return fail(TRI_ECAPACITY, "sequence %d would pass max_ctx %d", b, s->max_ctx);
    rows += pend + block;
    act.push_back(b);
  }
  if (act.empty()) return fail(TRI_ESTATE, "no prefilled sequence");
  if (rows > s->max_rows) return fail(TRI_ECAPACITY, "step needs %d rows, session allows %d", rows, s->max_rows);
  const size_t na = act.size(), cells = (size_t)s->max_batch * block;
  for (size_t i = 0; i < cells; ++i) out_target[i] = out_order[i] = out_step[i] = -1;
  for (int b = 0; b < s->max_batch; ++b) out_forwards[b] = -1;
  s->ev_used = s->prof_class >= 0 ? s->ev_used : 0;
  struct Saved {
    size_t L;
    int kv_len, written_hi;
  };
  std::vector<Saved> saved(na);
  for (size_t j = 0; j < na; ++j) {
    const Seq& S = s->seqs[act[j]];
    saved[j] = Saved{S.tokens.size(), S.kv_len, S.written_hi};
  }
  // serial denoising: the diffusion block at threshold 1 commits exactly one
  // position per forward (no confidence exceeds 1)
  std::vector<int32_t> toks(cells + (size_t)s->max_batch, -1);
  std::vector<std::vector<int>> order(na);
  int rc = step_diffusion(s, act, block, 1.f, block, toks.data(), nullptr, &order, false);
  if (rc) return rc;
  std::vector<std::vector<int32_t>> target(na);
  for (size_t j = 0; j < na; ++j) {
    Seq& S = s->seqs[act[j]];
    target[j].assign(S.tokens.end() - block, S.tokens.end());
    S.tokens.resize(saved[j].L);
    S.kv_len = saved[j].kv_len;
    S.written_hi = saved[j].written_hi;
  }
  std::vector<std::vector<int>> step;
  std::vector<int> fwd;
  rc = sol_parallel(s, act, block, target, order, step, fwd);
  if (rc) return rc;  // the sequences stay as before the call
  for (size_t j = 0; j < na; ++j) {
    Seq& S = s->seqs[act[j]];
    const int L = (int)saved[j].L;
    S.kv_len = L;  // as after the serial block
    S.written_hi = L;
    S.tokens.insert(S.tokens.end(), target[j].begin(), target[j].end());
    const size_t o = (size_t)act[j] * block;
    for (int i = 0; i < block; ++i) {
      out_target[o + i] = target[j][i];
      out_order[o + i] = order[j][i];
      out_step[o + i] = step[j][i];
    }
    out_forwards[act[j]] = fwd[j];
  }
  return TRI_OK;
}

int tri_choose_modes(const int32_t* grid_rows, const double* grid_ms, int n_grid, int n_seq, const double* expected,
                     const int32_t* pending, int block, int32_t* modes) {
  if (n_seq < 0 || n_grid < 1 || !grid_rows || !grid_ms) return fail(TRI_EINVAL, "bad cost grid or batch");
  if (n_seq > 0 && (!expected || !modes)) return fail(TRI_EINVAL, "null argument");
  if (block < 1 || block > 64) return fail(TRI_EINVAL, "block %d outside [1, 64]", block);
  for (int i = 0; i < n_grid; ++i) {
    if (!(grid_ms[i] > 0.0) || !std::isfinite(grid_ms[i])) return fail(TRI_EINVAL, "cost grid time %d", i);
    if (i > 0 && grid_rows[i] <= grid_rows[i - 1]) return fail(TRI_EINVAL, "cost grid rows must increase");
  }
  double prows = 0;
  for (int j = 0; j < n_seq; ++j) {
    if (!(expected[j] >= 1.0 && expected[j] <= block + 1.0))
      return fail(TRI_EINVAL, "expected tokens of sequence %d outside [1, block + 1]", j);
    const int p = pending ? pending[j] : 1;
    if (p < 1) return fail(TRI_EINVAL, "pending rows of sequence %d", j);
    prows += p;
  }
  // rows depend only on how many sequences speculate, so for each count the
  // best set is the largest expected rounds (ties: lowest index)
  std::vector<int> order(n_seq);
  for (int j = 0; j < n_seq; ++j) order[j] = j;
  std::stable_sort(order.begin(), order.end(), [&](int a, int b) { return expected[a] > expected[b]; });
  auto rate = [&](int ns, double gain) {
    const double tok = 2.0 * (n_seq - ns) + gain;
    const double r1 = prows + (double)ns * block, r2 = (double)(n_seq - ns) + (double)ns * block;
    return tok / (cost_ms(grid_rows, grid_ms, n_grid, r1) + cost_ms(grid_rows, grid_ms, n_grid, r2));
  };
  int best = 0;
  double best_rate = n_seq > 0 ? rate(0, 0.0) : 0.0, gain = 0.0;
  for (int ns = 1; ns <= n_seq; ++ns) {
    gain += expected[order[ns - 1]];
    const double r = rate(ns, gain);
    if (r > best_rate) {
      best_rate = r;
      best = ns;
    }
  }
  for (int i = 0; i < n_seq; ++i) modes[order[i]] = i < best ? TRI_SELFSPEC : TRI_AR;
  return TRI_OK;
}

int tri_set_lora(tri_session* s, int enabled) {
  if (!s) return fail(TRI_EINVAL, "null session");
  if (enabled && s->m->d.lora_rank <= 0) return fail(TRI_EINVAL, "model has no LoRA adapter");
  s->lora_on = enabled != 0;
  return TRI_OK;
}

int kv_append(tri_session* s, int seq, int n) {
  int rc = check_seq(s, seq);
  if (rc) return rc;
  Seq& S = s->seqs[seq];
  if (n < 0) return fail(TRI_EINVAL, "negative append");
  if (S.kv_len + n > s->max_ctx) return fail(TRI_ECAPACITY, "kv_len %d + %d passes max_ctx %d", S.kv_len, n, s->max_ctx);
  if (S.kv_len + n > (int)S.tokens.size() || S.kv_len + n > S.written_hi)
    return fail(TRI_ESTATE, "append of %d rows passes the committed (%d) or written (%d) rows", n, (int)S.tokens.size(),
                S.written_hi);
  S.kv_len += n;
  S.qdrafts.clear();
  return TRI_OK;
}

int kv_rollback(tri_session* s, int seq, int n) {
  int rc = check_seq(s, seq);
  if (rc) return rc;
  Seq& S = s->seqs[seq];
  if (n < 0) return fail(TRI_EINVAL, "negative rollback");
  if (n > S.kv_len) return fail(TRI_ESTATE, "rollback of %d rows with kv_len %d", n, S.kv_len);
  S.kv_len -= n;
  S.written_hi = S.kv_len;
  S.qdrafts.clear();
  return TRI_OK;
}

int tri_get_state(tri_session* s, int seq, int* committed, int* kv_len, int32_t* tokens, int cap) {
  int rc = check_seq(s, seq);
  if (rc) return rc;
  const Seq& S = s->seqs[seq];
  if (committed) *committed = (int)S.tokens.size();
  if (kv_len) *kv_len = S.kv_len;
  if (tokens) {
    const int n = std::min<int>(cap, (int)S.tokens.size());
    for (int i = 0; i < n; ++i) tokens[i] = S.tokens[i];
  }
  return TRI_OK;
}

int tri_forward(tri_session* s, int n_rows, const int32_t* row_seq, const int32_t* row_tok, const int32_t* row_pos,
                const int32_t* row_hi, const int32_t* row_lora, float* logits, int32_t* out_tok, float* out_conf) {
  if (!s || !row_seq || !row_tok || !row_pos || !row_hi) return fail(TRI_EINVAL, "null argument");
  if (n_rows <= 0 || n_rows > s->max_rows) return fail(TRI_ECAPACITY, "n_rows %d outside [1, %d]", n_rows, s->max_rows);
  HostRows R;
  for (int i = 0; i < n_rows; ++i) {
    const int sq = row_seq[i];
    if (sq < 0 || sq >= s->max_batch) return fail(TRI_EINVAL, "row %d: bad seq", i);
    if (row_tok[i] < 0 || row_tok[i] > s->m->d.vocab) return fail(TRI_EINVAL, "row %d: bad token", i);
    if (row_pos[i] < 0 || row_hi[i] <= row_pos[i] || row_hi[i] > s->max_ctx)
      return fail(TRI_EINVAL, "row %d: need 0 <= pos < hi <= max_ctx", i);
    if (i > 0 && sq != row_seq[i - 1]) {
      for (int sl : R.slot_seq)
        if (sl == row_seq[i - 1]) return fail(TRI_EINVAL, "rows of a sequence must be contiguous");
      R.close_slot(row_seq[i - 1]);
    }
    R.add(row_tok[i], row_pos[i], row_hi[i], sq, row_lora ? (row_lora[i] != 0) : 0, 1);
  }
  for (int sl : R.slot_seq)
    if (sl == row_seq[n_rows - 1]) return fail(TRI_EINVAL, "rows of a sequence must be contiguous");
  R.close_slot(row_seq[n_rows - 1]);
  float* lg = logits ? logits : s->logits;
  int rc = stage_meta(s, 0, R, {}, {});
  if (!rc) rc = upload_meta(s, 0);
  if (!rc) rc = forward(s, 0, R, lg);
  if (!rc) rc = sample(s, 0, R, lg, 0.f, 0);
  if (!rc) rc = d2h_ints(s, s->o_out_tok, n_rows);
  if (!rc) rc = d2h_ints(s, s->o_status, 4);
  if (rc) return rc;
  HIPCHK(hipMemcpyAsync(s->hconf, s->dconf, (size_t)n_rows * 4, hipMemcpyDeviceToHost, s->st));
  HIPCHK(hipStreamSynchronize(s->st));
  rc = check_status(s, 0, "teacher-forced forward");
  if (rc) return rc;
  if (out_tok) memcpy(out_tok, s->hints + s->o_out_tok, (size_t)n_rows * 4);
  if (out_conf) memcpy(out_conf, s->hconf, (size_t)n_rows * 4);
  return TRI_OK;
}

int tri_forward_bytes(tri_session* s, int rows_per_seq, double* bytes) {
  if (!s || !bytes || rows_per_seq < 0) return fail(TRI_EINVAL, "bad argument");
  const tri_model_desc& d = s->m->d;
  const double esz = (double)s->m->esz;
  const double qd = (double)d.n_q_heads * d.head_dim, kd = (double)d.n_kv_heads * d.head_dim;
  double w = (double)d.d_model * (qd + 2 * kd) + qd * d.d_model + 3.0 * d.d_model * d.d_ffn;
  w *= d.n_layers * esz;
  w += (double)d.vocab * d.d_model * esz;       // lm_head
  w += (2.0 * d.n_layers + 1) * d.d_model * 4;  // norm gains
  double kv = 0, rows = 0;
  for (const Seq& S : s->seqs) {
    if (!S.active) continue;
    const double hi = (double)S.tokens.size() + rows_per_seq;
    kv += hi * kd * 2 * esz * d.n_layers;  // K and V read once per kv head
    rows += rows_per_seq;
  }
  const double logits = rows * d.vocab * 4.0 * 2;  // written once, read once
  *bytes = w + kv + logits;
  return TRI_OK;
}

// -------------------------------------------------------------- test hooks
int tri_set_trace(tri_session* s, int enabled) {
  if (!s) return fail(TRI_EINVAL, "null session");
  s->tracing = enabled != 0;
  s->trace.clear();
  return TRI_OK;
}

int tri_trace_count(tri_session* s, int* n) {
  if (!s || !n) return fail(TRI_EINVAL, "null argument");
  *n = (int)s->trace.size();
  return TRI_OK;
}

int tri_trace_get(tri_session* s, int i, int* n_rows, int32_t* seq, int32_t* tok, int32_t* pos, int32_t* hi,
                  int32_t* lora, float* logits, int cap_rows, int* has_logits) {
  if (!s || !n_rows) return fail(TRI_EINVAL, "null argument");
  if (i < 0 || i >= (int)s->trace.size()) return fail(TRI_EINVAL, "trace index %d out of range", i);
  const TraceRec& r = s->trace[i];
  const int n = (int)r.seq.size();
  *n_rows = n;
  if (has_logits) *has_logits = r.logits.empty() ? 0 : 1;
  if (cap_rows < n) return TRI_OK;
  if (seq) memcpy(seq, r.seq.data(), n * 4);
  if (tok) memcpy(tok, r.tok.data(), n * 4);
  if (pos) memcpy(pos, r.pos.data(), n * 4);
  if (hi) memcpy(hi, r.hi.data(), n * 4);
  if (lora) memcpy(lora, r.lora.data(), n * 4);
  if (logits && !r.logits.empty()) memcpy(logits, r.logits.data(), r.logits.size() * 4);
  return TRI_OK;
}

int tri_set_commit_schedule(tri_session* s, int seq, const int32_t* counts, int n) {
  int rc = check_seq(s, seq);
  if (rc) return rc;
  if (n < 0 || (n > 0 && !counts)) return fail(TRI_EINVAL, "bad commit schedule");
  for (int i = 0; i < n; ++i)
    if (counts[i] < 1) return fail(TRI_EINVAL, "commit count %d of the schedule is below 1", i);
  s->seqs[seq].sched.assign(counts, counts + n);
  return TRI_OK;
}

int tri_set_draft_override(tri_session* s, int seq, const int32_t* ref, int n_ref, int a_star) {
  int rc = check_seq(s, seq);
  if (rc) return rc;
  Seq& S = s->seqs[seq];
  if (a_star < 0) {
    S.a_star = -1;
    S.ref.clear();
    return TRI_OK;
  }
  if (!ref || n_ref <= 0) return fail(TRI_EINVAL, "override needs reference tokens");
  for (int i = 0; i < n_ref; ++i)
    if (ref[i] < 0 || ref[i] >= s->m->d.vocab) return fail(TRI_EINVAL, "reference token %d out of range", i);
  S.ref.assign(ref, ref + n_ref);
  S.a_star = a_star;
  return TRI_OK;
}

int tri_profile(tri_session* s, int kernel_class) {
  if (!s) return fail(TRI_EINVAL, "null session");
  if (kernel_class >= PROF_N) return fail(TRI_EINVAL, "bad kernel class");
  HIPCHK(hipStreamSynchronize(s->st));
  s->prof_class = kernel_class;
  s->ev_used = 0;
  return TRI_OK;
}

int tri_profile_read(tri_session* s, double* total_ms, int* launches) {
  if (!s || !total_ms || !launches) return fail(TRI_EINVAL, "null argument");
  HIPCHK(hipStreamSynchronize(s->st));
  double t = 0;
  for (size_t i = 0; i + 1 < s->ev_used; i += 2) {
    float ms = 0;
    HIPCHK(hipEventElapsedTime(&ms, s->ev[i], s->ev[i + 1]));
    t += ms;
  }
  *total_ms = t;
  *launches = (int)(s->ev_used / 2);
  return TRI_OK;
}

// -------------------------------------------------------- kernel-level ABI
int block_causal_attn_ws_bytes(int rows, int hq, int hd, int max_hi, int kv_split, size_t* bytes) {
  if (!bytes || rows < 0 || hq <= 0 || hd <= 0 || max_hi < 0 || kv_split < 0 || (kv_split % 64))
    return fail(TRI_EINVAL, "bad argument");
  *bytes = attn_ws_bytes(rows, hq, hd, max_hi, kv_split);
  return TRI_OK;
}

int block_causal_attn(const void* q, const void* k_cache, const void* v_cache, int n_seq, const int32_t* seq_start,
                      const int32_t* row_hi, int rows, int max_rows_per_seq, int max_hi, int hq, int hkv, int hd,
                      int ctx, float scale, int dtype, int kv_split, void* out, void* ws, size_t ws_bytes,
                      void* stream) {
  if (!q || !k_cache || !v_cache || !seq_start || !row_hi || !out) return fail(TRI_EINVAL, "null pointer");
  if (rows < 0 || n_seq <= 0 || hq <= 0 || hkv <= 0 || hq % hkv || max_rows_per_seq < 0 || max_hi < 0)
    return fail(TRI_EINVAL, "bad shape");
  if (ctx <= 0 || ctx % 64 || max_hi > ctx) return fail(TRI_EINVAL, "ctx must be a positive multiple of 64 >= max_hi");
  const bool v16 = dtype == TRI_BF16_V16;
  if (v16) dtype = TRI_BF16;
  if (dtype == TRI_BF16 ? hd != 128 : (dtype == TRI_F32 ? (hd > 128 || hd <= 0) : true))
    return fail(TRI_EINVAL, "unsupported dtype/head_dim");
  if (!(scale > 0)) return fail(TRI_EINVAL, "scale must be positive");
  if (kv_split == 0) kv_split = attn_pick_split_launch(max_hi, n_seq, max_rows_per_seq, hq, hkv);
  if (kv_split < 64 || kv_split % 64) return fail(TRI_EINVAL, "kv_split must be a positive multiple of 64");
  if (ws_bytes < attn_ws_bytes(rows, hq, hd, max_hi, kv_split) || (!ws && ws_bytes))
    return fail(TRI_ECAPACITY, "workspace too small");
  AttnLaunch a;
  a.q = q;
  a.kc = k_cache;
  a.vc = v_cache;
  a.seq_start = seq_start;
  a.slot_seq = nullptr;
  a.row_hi = row_hi;
  a.n_seq = n_seq;
  a.rows = rows;
  a.max_rows_per_seq = max_rows_per_seq;
  a.max_hi = max_hi;
  a.hq = hq;
  a.hkv = hkv;
  a.hd = hd;
  a.ctx = ctx;
  a.scale = scale;
  a.kv_split = kv_split;
  a.out = out;
  a.part = static_cast<float*>(ws);
  a.v_f16 = v16;
  HIPCHK(launch_attn(dtype, a, static_cast<hipStream_t>(stream)));
  return TRI_OK;
}

// ------------------------------------------------- allocation-free variant
// block_causal_attn without a workspace argument, for callers that cannot
// allocate device memory: the split partials live in this file-scope device
// array.  Every GPU the library runs on holds its own copy for the life of
// the process; host code uses the address hipGetSymbolAddress returns for the
// current device (kept per device), never the array's name.
constexpr size_t ATTN_SCRATCH_BYTES = (size_t)32 << 20;
static __device__ __align__(256) char attn_scratch[ATTN_SCRATCH_BYTES];

namespace {
constexpr int MAX_DEVICES = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[MAX_DEVICES] = {};

int scratch_for_current_device(void** out) {
  int dev = 0;
  HIPCHK(hipGetDevice(&dev));
  if (dev < 0 || dev >= MAX_DEVICES) return fail(TRI_EINVAL, "device %d beyond the %d the library tracks", dev, MAX_DEVICES);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    HIPCHK(hipGetSymbolAddress(&p, HIP_SYMBOL(attn_scratch)));
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return TRI_OK;
}
}  // namespace

int block_causal_attn_noalloc(const void* q, const void* k_cache, const void* v_cache, int n_seq,
                              const int32_t* seq_start, const int32_t* row_hi, int rows, int max_rows_per_seq,
                              int max_hi, int hq, int hkv, int hd, int ctx, float scale, int dtype, int kv_split,
                              void* out, void* stream) {
  if (rows < 0 || hq <= 0 || hd <= 0 || max_hi < 0 || kv_split < 0 || kv_split % 64) return fail(TRI_EINVAL, "bad shape");
  const int split = kv_split == 0 && hkv > 0 ? attn_pick_split_launch(max_hi, n_seq, max_rows_per_seq, hq, hkv) : kv_split;
  const size_t need = attn_ws_bytes(rows, hq, hd, max_hi, split);
  if (need > ATTN_SCRATCH_BYTES)
    return fail(TRI_ECAPACITY, "split partials need %zu bytes, the static scratch holds %zu (fewer rows or longer kv_split)",
                need, ATTN_SCRATCH_BYTES);
  void* ws = nullptr;
  int rc = scratch_for_current_device(&ws);
  if (rc) return rc;
  return block_causal_attn(q, k_cache, v_cache, n_seq, seq_start, row_hi, rows, max_rows_per_seq, max_hi, hq, hkv, hd,
                           ctx, scale, dtype, split, out, ws, ATTN_SCRATCH_BYTES, stream);
}

int sample_commit_ws_bytes(int rows, int vocab, size_t* bytes) {
  if (!bytes || rows < 0 || vocab <= 0) return fail(TRI_EINVAL, "bad argument");
  *bytes = vocab_ws_bytes(rows, vocab);
  return TRI_OK;
}

int sample_commit(const float* logits, int rows, int vocab, const int32_t* row_kind, const int32_t* block_start,
                  int n_blocks, float threshold, int32_t* out_tok, float* out_conf, int32_t* out_commit,
                  int32_t* out_status, void* ws, size_t ws_bytes, void* stream) {
  if (!logits || !row_kind || !out_tok || !out_conf || !out_commit || !out_status || !ws)
    return fail(TRI_EINVAL, "null pointer");
  if (rows <= 0 || vocab <= 0 || n_blocks < 0 || (n_blocks > 0 && !block_start)) return fail(TRI_EINVAL, "bad shape");
  if (!(threshold >= 0.f && threshold <= 1.f)) return fail(TRI_EINVAL, "threshold must be in [0, 1]");
  if (ws_bytes < vocab_ws_bytes(rows, vocab)) return fail(TRI_ECAPACITY, "workspace too small");
  HIPCHK(launch_sample_commit(logits, rows, vocab, row_kind, block_start, n_blocks, threshold, out_tok, out_conf,
                              out_commit, out_status, ws, static_cast<hipStream_t>(stream)));
  return TRI_OK;
}

int verify_accept(const int32_t* draft, const int32_t* ar_tok, int batch, int k, int32_t* accept_len,
                  int32_t* committed, int32_t* kv_len, void* stream) {
  if (!draft || !ar_tok || !accept_len || !committed) return fail(TRI_EINVAL, "null pointer");
  if (batch <= 0 || k < 0) return fail(TRI_EINVAL, "bad shape");
  HIPCHK(launch_verify_accept(draft, ar_tok, batch, k, accept_len, committed, kv_len, static_cast<hipStream_t>(stream)));
  return TRI_OK;
}

}  // extern "C"
