// Host checks of launch plans.
// GEMM: for every projection plan the library builds for the named model
// shapes, and row counts covering the decode kernel (1..64) and the large-M
// kernel's forms (tall and square, one slot and chained), the highest packed
// weight element a launch reads must lie inside the packed matrix.
// Attention splits: every split the session rule or the per-launch model picks
// is a multiple of 64 keys in [128, 4096], and a long-context session (8K keys
// or more) keeps a full-capacity launch of 33-row blocks within one round of
// 256 workgroups whenever the rule's bound allows it.
// Prints one line per check group and exits non-zero on a violation.
#include <cstdio>
#include <cstdlib>
#include <algorithm>
#include <vector>

#include "tri_common.h"

using namespace tri;

struct Shape {
  const char* name;
  int d, hq, hkv, hd, ffn, vocab, lora;
};

int main() {
  const Shape shapes[] = {{"8b-class", 4096, 32, 8, 128, 12288, 151936, 0},
                          {"14b-class", 5120, 40, 8, 128, 17408, 151936, 128},
                          {"small-bf16", 512, 4, 2, 128, 1024, 1000, 128},
                          {"odd-bf16", 640, 5, 1, 128, 1728, 777, 64}};
  const int rows[] = {1,   2,   3,   15,  16,  17,  31,  32,  33,  47,  48,  63,   64,   65,   66,   96,
                      127, 128, 129, 200, 255, 256, 257, 300, 511, 512, 600, 1024, 1122, 2112, 4096, 8192};
  int bad = 0;
  for (const Shape& s : shapes) {
    const int qd = s.hq * s.hd, kd = s.hkv * s.hd;
    struct P {
      const char* n;
      int N, K;
      bool unsplit;
    } proj[] = {{"qkv", qd + 2 * kd, s.d, false}, {"o", s.d, qd, false},     {"gate/up", 2 * s.ffn, s.d, false},
                {"down", s.d, s.ffn, false},       {"lm_head", s.vocab, s.d, true}, {"lora_a", s.lora, qd, false},
                {"lora_b", s.d, s.lora, false}};
    long checks = 0;
    for (const P& p : proj) {
      if (p.N <= 0 || p.K <= 0) continue;
      const GemmPlan plan = gemm_plan(p.N, p.K, TRI_BF16, p.unsplit);
      const size_t elems = gemm_packed_bytes(plan, p.N, p.K, TRI_BF16) / 2;
      if (plan.Ks % (plan.nch * 256)) {
        printf("%s %s: stages per pass (%d) do not divide the split (%d k)\n", s.name, p.n, plan.nch, plan.Ks);
        ++bad;
      }
      for (int M : rows)
        for (int inv = 0; inv < 2; ++inv) {
          const size_t reach = gemm_w_reach(TRI_BF16, plan, M, p.N, p.K, inv != 0);
          ++checks;
          if (reach > elems || reach == 0) {
            printf("%s %s M=%d invariant=%d: reads up to element %zu of %zu\n", s.name, p.n, M, inv, reach, elems);
            ++bad;
          }
        }
    }
    printf("%s: %ld launches checked\n", s.name, checks);
  }
  long splits = 0;
  const int heads[][2] = {{32, 8}, {40, 8}, {4, 2}, {5, 1}, {64, 8}};
  for (const auto& h : heads) {
    const int hq = h[0], hkv = h[1], G = hq / hkv;
    for (int ctx = 64; ctx <= 131072; ctx += ctx < 4096 ? 64 : 1024)
      for (int n_seq : {1, 2, 8, 16}) {
        const int sp = attn_pick_split(ctx, n_seq, hq, hkv);
        ++splits;
        if (sp % 64 || sp < 128 || sp > 4096) {
          printf("session split %d for ctx %d, %d sequences, %dq/%dkv\n", sp, ctx, n_seq, hq, hkv);
          ++bad;
        }
        if (n_seq == 1 && ctx >= 8192) {
          const int qtiles = (33 * G + 15) / 16;
          const int per_wg = qtiles >= 8 ? 8 : 4;  // query tiles per workgroup beyond 4K keys
          const long wgs = (long)((ctx + sp - 1) / sp) * ((qtiles + per_wg - 1) / per_wg) * hkv;
          int pow2 = 128;
          while (pow2 < 2048 && 2.0 * pow2 <= ctx / 16.0) pow2 *= 2;
          const long per_split = (long)((qtiles + per_wg - 1) / per_wg) * hkv;
          const long ns_max = 256 / per_split;
          const bool fits = ns_max >= 1 && ((ctx + ns_max - 1) / ns_max + 63) / 64 * 64 <= 2 * pow2;
          if (fits && wgs > 256) {
            printf("session split %d for ctx %d, %dq/%dkv: %ld workgroups at capacity\n", sp, ctx, hq, hkv, wgs);
            ++bad;
          }
        }
        const int sl = attn_pick_split_launch(ctx, n_seq, 32, hq, hkv);
        if (sl % 64 || sl < 128 || sl > 4096) {
          printf("launch split %d for %d keys, %d sequences, %dq/%dkv\n", sl, ctx, n_seq, hq, hkv);
          ++bad;
        }
      }
  }
  printf("attention: %ld split choices checked\n", splits);
  // Compacted attention grid: for ragged slot layouts the table lists, slot
  // by slot, exactly the query groups g with g * (group size) < the slot's
  // query vectors (the groups the regular grid's workgroups find work in),
  // and uniform layouts keep the regular grid (0 entries).
  long tables = 0;
  unsigned rng = 12345u;
  auto next = [&](int mod) {
    rng = rng * 1103515245u + 12345u;
    return (int)((rng >> 8) % (unsigned)mod);
  };
  for (int trial = 0; trial < 4000; ++trial) {
    const int hkv = 8, G = (int[]){1, 2, 4, 5, 8}[trial % 5], hq = G * hkv;
    const int n = 2 + next(63), max_hi = (int[]){100, 600, 1600, 5000, 40000}[next(5)];
    const bool uniform = trial % 7 == 0;
    std::vector<int32_t> st(1, 0);
    const int r0 = 1 + next(33);
    for (int i = 0; i < n; ++i) st.push_back(st.back() + (uniform ? r0 : (next(4) == 0 ? 1 + next(64) : 1)));
    int maxr = 0;
    for (int i = 0; i < n; ++i) maxr = std::max(maxr, st[i + 1] - st[i]);
    const int qv = attn_group_vectors(maxr, G, max_hi);
    const int cap = st.back() + n;
    std::vector<int32_t> out(cap, -1);
    const int w = attn_work_table(st.data(), n, hq, hkv, max_hi, out.data(), cap);
    std::vector<int32_t> want;
    bool same = true;
    const int g0 = ((st[1] - st[0]) * G + qv - 1) / qv;
    for (int i = 0; i < n; ++i) {
      const int groups = ((st[i + 1] - st[i]) * G + qv - 1) / qv;
      same = same && groups == g0;
      for (int g = 0; g * qv < (st[i + 1] - st[i]) * G; ++g) want.push_back(i * 65536 + g);
    }
    ++tables;
    const bool ok = same ? w == 0 : (w == (int)want.size() && std::equal(want.begin(), want.end(), out.begin()));
    if (!ok || qv % 32 || qv < 32 || qv > 128) {
      printf("attention work table: trial %d, %d slots, G %d, max_hi %d: %d entries, expected %zu%s\n", trial, n, G,
             max_hi, w, same ? (size_t)0 : want.size(), same ? " (uniform)" : "");
      ++bad;
    }
  }
  printf("attention work tables: %ld layouts checked\n", tables);
  printf(bad ? "FAIL %d\n" : "OK\n", bad);
  return bad ? 1 : 0;
}
