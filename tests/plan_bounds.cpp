// Host check of the GEMM launches' weight reads: for every projection plan the
// library builds for the named model shapes, and row counts covering the
// decode kernel (1..64) and the large-M kernel's forms (tall and square, one
// slot and chained), the highest packed weight element a launch reads must lie
// inside the packed matrix.  Prints one line per shape and exits non-zero on
// a violation.
#include <cstdio>
#include <cstdlib>

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
  printf(bad ? "FAIL %d\n" : "OK\n", bad);
  return bad ? 1 : 0;
}
