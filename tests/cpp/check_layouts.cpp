// Host-side checks of the LDS carve-ups and the workspace plans (compiled with
// g++ by tests/test_plan_layouts.py; no GPU).  Prints one line per failure
// and "ok <n>" with the number of shapes checked.
#include <cstdio>
#include <initializer_list>

#include "../../fenwick_tree_hierarchical_amd/csrc/la_bwd_plan.hpp"

using namespace la;

static int fails = 0;
#define CHECK(cond, ...)                                   \
  do {                                                     \
    if (!(cond)) {                                         \
      ++fails;                                             \
      std::printf("FAIL %s: ", #cond);                     \
      std::printf(__VA_ARGS__);                            \
      std::printf("\n");                                   \
    }                                                      \
  } while (0)

static bool disjoint(int a0, int a1, int b0, int b1) { return a1 <= b0 || b1 <= a0; }

int main() {
  int n = 0;
  const int Cs[] = {16, 32, 64, 128}, Ds[] = {16, 32, 64, 128};
  for (int es : {2, 4})
    for (int C : Cs)
      for (int D : Ds)
        for (int L = 1; L <= kMaxLevels; ++L) {
          ++n;
          // forward output tile: Q, K|P, V, lambda, b2, e2 back to back
          const OutLds o = output_lds(C, D, es, L);
          const int kp = C * o.ld_row * es > C * o.ld_p * es ? C * o.ld_row * es : C * o.ld_p * es;
          CHECK(o.q + C * o.ld_row * es <= o.k, "C=%d D=%d es=%d L=%d", C, D, es, L);
          CHECK(o.k + kp <= o.v && o.v + C * o.ld_v * es <= o.lam, "C=%d D=%d es=%d L=%d", C, D, es, L);
          CHECK(o.lam + C * L * 4 <= o.b2 && o.b2 + C * 4 <= o.e2 && o.e2 + C * 4 <= o.total, "C=%d D=%d", C, D);
          CHECK((o.ld_row * es) % 16 == 0 && (o.ld_p * es) % 16 == 0, "row alignment C=%d D=%d es=%d", C, D, es);
          if (C > 64) continue;
          // backward, query side
          const BwdChunkLds q = bwd_chunk_lds(C, D, es, L, false);
          const int tile = C * q.ld_row * es, stile = C * q.ld_s * es;
          const int vt = q.g - q.v;
          CHECK(stile <= vt, "dS over V: C=%d D=%d es=%d", C, D, es);
          const int QB = C / 16, NW = bwd_waves(C);
          const int part_b = (QB * (QB + 1) / 2) * 16 * 4 + QB * 16 * 5 * 4;
          CHECK(q.part == q.q && part_b <= tile, "row sums over Q: C=%d D=%d es=%d", C, D, es);
          const int ninter = L - ilog2(C) - 1 > 0 ? L - ilog2(C) - 1 : 0;
          const int inter_b = NW * ninter * C * 4;
          if (q.inter == q.k) CHECK(inter_b <= q.g - q.k, "shares over K and dS: C=%d D=%d L=%d", C, D, L);
          else CHECK(q.inter >= q.b2 + C * 4 && q.inter + inter_b <= q.total, "own shares region: C=%d D=%d L=%d", C, D, L);
          CHECK(q.g + tile <= q.lam && q.lam + C * L * 4 <= q.b2 && q.b2 + C * 4 <= q.total, "C=%d D=%d L=%d", C, D, L);
          CHECK((q.ld_row * es) % 16 == 0 && (q.ld_s * es) % 16 == 0, "row alignment C=%d D=%d", C, D);
          // backward, key side: every region live at once is disjoint
          const BwdChunkLds k = bwd_chunk_lds(C, D, es, L, true);
          const int ends[][2] = {{k.q, k.q + tile}, {k.k, k.k + tile}, {k.v, k.v + tile}, {k.g, k.g + tile},
                                 {k.lam, k.lam + C * L * 4}, {k.b2, k.b2 + C * 4}, {k.s0, k.s0 + stile},
                                 {k.col, k.col + NW * C * 4}, {k.e2, k.e2 + C * 4}};
          for (int i = 0; i < 9; ++i) {
            CHECK(ends[i][1] <= k.total, "key side region %d past the end: C=%d D=%d L=%d", i, C, D, L);
            for (int j = i + 1; j < 9; ++j)
              CHECK(disjoint(ends[i][0], ends[i][1], ends[j][0], ends[j][1]), "key side %d/%d C=%d D=%d L=%d", i, j, C, D, L);
          }
        }
  // key-side node builder and the workspace plans
  for (int es : {2, 4})
    for (int C : {16, 32, 64})
      for (int D : Ds) {
        const int G = state_group(D);
        const RevLds r = rev_lds(C, D, es, G);
        CHECK(r.qt + D * r.ld_t * es <= r.gt && r.gt + D * r.ld_t * es <= r.b2 && r.b2 + G * C * 4 <= r.w &&
                  r.w + C * 4 <= r.total,
              "rev C=%d D=%d es=%d", C, D, es);
        for (long long T : {1LL, 15LL, 64LL, 1000LL, 4097LL, 16384LL, 131072LL}) {
          BwdPlan p;
          const int dt = es == 2 ? kBF16 : kF32;
          if (plan_bwd(2, 3, T, D, D, C, dt, levels_needed(T), &p) != kOK) continue;
          ++n;
          const FwdPlan& f = p.f;
          const size_t DD = (size_t)D * D;
          size_t prev = f.ws_bytes;
          if (f.n_chunks > 1) {
            CHECK(p.off_rnodes_in == prev && p.off_rnodes_in % 256 == 0, "T=%lld C=%d D=%d", T, C, D);
            CHECK(p.off_rnodes_in_t >= p.off_rnodes_in + f.BH * f.n_chunks * DD * f.es, "T=%lld", T);
            prev = p.off_rnodes_in_t + f.BH * f.n_chunks * DD * f.es;
          }
          if (f.n_groups > 1) {
            CHECK(p.JG == bit_length(f.n_groups - 1) && p.off_rpart >= prev, "T=%lld", T);
            CHECK(p.off_rnodes >= p.off_rpart + f.BH * f.n_groups * p.JG * DD * 4, "T=%lld", T);
            CHECK(p.off_rnodes_t >= p.off_rnodes + f.BH * f.n_groups * DD * f.es, "T=%lld", T);
            prev = p.off_rnodes_t + f.BH * f.n_groups * DD * f.es;
          }
          CHECK(p.off_dcol >= prev && p.off_dcol % 256 == 0, "T=%lld", T);
          CHECK(p.ws_bytes >= p.off_dcol + (size_t)f.BH * T * 4, "T=%lld", T);
          // every group level a key-side block can use has a share slot
          if (f.n_groups > 1) CHECK((1LL << (p.JG - 1)) < f.n_groups && (1LL << p.JG) >= f.n_groups, "T=%lld", T);
        }
      }
  std::printf("ok %d\n", n);
  return fails ? 1 : 0;
}
