// Host-side checks of the LDS carve-ups and the workspace plans (compiled with
// g++ by tests/test_plan_layouts.py; no GPU).  Prints one line per failure
// and "ok <n>" with the number of shapes checked.
#include <cstdio>
#include <initializer_list>

#include "../../fenwick_tree_hierarchical_amd/csrc/la_bwd_plan.hpp"
#include "../../fenwick_tree_hierarchical_amd/csrc/la_gdn_plan.hpp"

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
          // the late-V variant: V shares the Q tile, the rest back to back after
          // K|P; the plan picks it exactly where two workgroups fit per CU
          if (output_vlate_shape(C, D, es)) {
            const OutLds v = output_lds_vlate(C, D, es, L);
            CHECK(v.q == 0 && v.v == v.q && v.k == o.k && v.p == o.p && v.ld_v == o.ld_v, "late V C=%d D=%d L=%d", C, D, L);
            CHECK(C * v.ld_v * es <= v.k && v.k + kp <= v.lam, "late V C=%d D=%d L=%d", C, D, L);
            CHECK(v.lam + C * L * 4 <= v.b2 && v.b2 + C * 4 <= v.e2 && v.e2 + C * 4 <= v.total, "late V L=%d", L);
            FwdPlan fp;
            CHECK(plan_fwd(1, 2, 1000, D, D, C, es == 2 ? kBF16 : kF32, L >= levels_needed(1000) ? L : -1, &fp) == kOK,
                  "late V plan L=%d", L);
            if (L >= levels_needed(1000))
              CHECK((fp.lds_out_vlate > 0) == (2 * v.total <= kLdsLimit) && (fp.lds_out_vlate == 0 || fp.lds_out_vlate == v.total),
                    "late V choice L=%d", L);
          }
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
        // the staged and chunk-major key-side kernels: both row tiles, the gate
        // prefixes and the weights in order, two workgroups per CU where used
        if (es == 2 && rev_staged_fits(true, C, D, G)) {
          const RevStagedLds st = rev_staged_lds(C, D, G);
          const int rows = (G / 2) * C * 2 * D;
          CHECK(st.q == 0 && st.g == rows && st.b2 == 2 * rows && st.w == st.b2 + G * C * 4 &&
                    st.total == st.w + 2 * (G / 2) * C * 4 && 2 * st.total <= kLdsLimit,
                "staged rev C=%d D=%d", C, D);
          if (rev_cm_fits(true, C, D, G)) {
            int log2g = 0;
            for (int g = G; g > 1; g >>= 1) ++log2g;
            const RevStagedLds cm = rev_cm_lds(C, D, G);
            CHECK(cm.q == st.q && cm.g == st.g && cm.b2 == st.b2 && cm.w == st.w &&
                      cm.total == cm.w + (log2g + kRevGroupSlots) * (G / 2) * C * 4 && 2 * cm.total <= kLdsLimit,
                  "chunk-major rev C=%d D=%d", C, D);
          }
        }
        for (long long T : {1LL, 15LL, 64LL, 1000LL, 4097LL, 16384LL, 131072LL}) {
          BwdPlan p;
          const int dt = es == 2 ? kBF16 : kF32;
          if (plan_bwd(2, 3, T, D, D, C, dt, levels_needed(T), &p) != kOK) continue;
          ++n;
          const FwdPlan& f = p.f;
          const size_t DD = (size_t)D * D;
          size_t prev = f.ws_bytes;
          // the transposed nodes are kept only for the split key-side kernel
          const bool keep_t = p.lds_fused == 0;
          CHECK(p.rhalves == (rev_staged_fits(es == 2, C, D, f.G) ? 2 : 1), "T=%lld C=%d D=%d", T, C, D);
          if (f.n_chunks > 1) {
            CHECK(p.off_rnodes_in == prev && p.off_rnodes_in % 256 == 0, "T=%lld C=%d D=%d", T, C, D);
            prev = p.off_rnodes_in + f.BH * f.n_chunks * DD * f.es;
            if (keep_t) {
              CHECK(p.off_rnodes_in_t >= prev && p.off_rnodes_in_t % 256 == 0, "T=%lld", T);
              prev = p.off_rnodes_in_t + f.BH * f.n_chunks * DD * f.es;
            } else {
              CHECK(p.off_rnodes_in_t == 0, "T=%lld C=%d D=%d", T, C, D);
            }
          }
          if (f.n_groups > 1) {
            CHECK(p.JG == bit_length(f.n_groups - 1) && p.off_rpart >= prev, "T=%lld", T);
            CHECK(p.off_rnodes >= p.off_rpart + f.BH * f.n_groups * p.rhalves * p.JG * DD * 4, "T=%lld", T);
            prev = p.off_rnodes + f.BH * f.n_groups * DD * f.es;
            if (keep_t) {
              CHECK(p.off_rnodes_t >= prev && p.off_rnodes_t % 256 == 0, "T=%lld", T);
              prev = p.off_rnodes_t + f.BH * f.n_groups * DD * f.es;
            } else {
              CHECK(p.off_rnodes_t == 0, "T=%lld C=%d D=%d", T, C, D);
            }
          }
          // the workspace query (L unknown: planned for the most levels) covers this plan
          BwdPlan q;
          CHECK(plan_bwd(2, 3, T, D, D, C, dt, -1, &q) == kOK && q.ws_bytes >= p.ws_bytes, "T=%lld C=%d D=%d", T, C, D);
          CHECK(p.off_dcol >= prev && p.off_dcol % 256 == 0, "T=%lld", T);
          CHECK(p.ws_bytes >= p.off_dcol + (size_t)f.BH * T * 4, "T=%lld", T);
          // every group level a key-side block can use has a share slot
          if (f.n_groups > 1) CHECK((1LL << (p.JG - 1)) < f.n_groups && (1LL << p.JG) >= f.n_groups, "T=%lld", T);
        }
      }

  // Gated DeltaNet: LDS regions in order, 256-byte aligned, each large enough
  // for every tile placed in it, inside the limit; workspace regions ordered
  // and sized; the node levels cover every block a query chunk reads.
  for (int es : {2, 4})
    for (int C : {16, 32, 64})
      for (int D : {16, 32, 64}) {
        const int tCD = gdn_tile(C, D, es), tDC = gdn_tile(D, C, es), tCC = gdn_tile(C, C, es);
        const int fCC = gdn_tile(C, C, 4);
        const GdnPrepLds pl = gdn_prep_lds(C, D, es);
        const int sw = D * C * es;
        const int po[] = {pl.kr, pl.kt, pl.vst, pl.kbt, pl.g, pl.b2, pl.beta};
        for (int i = 0; i + 1 < 7; ++i) CHECK(po[i] % 256 == 0 && po[i] < po[i + 1], "gdn prep C=%d D=%d es=%d", C, D, es);
        CHECK(pl.kt - pl.kr >= tCD && pl.kt - pl.kr >= 16 * gdn_lde(C, 4) * 4 && pl.kt - pl.kr >= sw,
              "gdn prep K/X/U^T C=%d D=%d es=%d", C, D, es);
        CHECK(pl.vst - pl.kt >= sw && pl.kbt - pl.vst >= sw && pl.g - pl.kbt >= sw, "gdn prep swizzled C=%d D=%d", C, D);
        CHECK(pl.b2 - pl.g >= fCC, "gdn prep G/T C=%d", C);
        CHECK(pl.beta - pl.b2 >= C * 4 && pl.total - pl.beta >= C * 4, "gdn prep gates C=%d", C);
        CHECK(pl.total <= kLdsLimit, "gdn prep LDS %d C=%d D=%d es=%d", pl.total, C, D, es);
        CHECK(pl.total >= 3 * gdn_tile(D, D, es), "gdn prep merge staging C=%d D=%d es=%d", C, D, es);
        if (es == 2 && C == 64 && D == 64)
          CHECK(3 * pl.total <= kLdsLimit, "gdn prep: three workgroups per CU at the 16K shape (%d)", pl.total);
        (void)tDC;
        CHECK(gdn_tree_lds(D, es) >= D * gdn_lde(D, es) * es && gdn_tree_lds(D, es) <= kLdsLimit, "gdn tree D=%d", D);
        for (int L = 1; L <= kMaxLevels; ++L) {
          const GdnOutLds ol = gdn_out_lds(C, D, es, L);
          const int oo[] = {ol.q, ol.k, ol.v, ol.s, ol.lam, ol.b2, ol.beta, ol.total};
          for (int i = 0; i + 1 < 8; ++i) CHECK(oo[i] % 256 == 0 && oo[i] < oo[i + 1], "gdn out C=%d D=%d L=%d", C, D, L);
          CHECK(ol.k - ol.q >= tCD, "gdn out Q C=%d D=%d", C, D);
          CHECK(ol.v - ol.k >= tCD && ol.v - ol.k >= tCC, "gdn out K/Ahat C=%d D=%d es=%d", C, D, es);
          CHECK(ol.s - ol.v >= tCD && ol.s - ol.v >= tCC, "gdn out V/P C=%d D=%d es=%d", C, D, es);
          CHECK(ol.lam - ol.s >= tCC && ol.lam - ol.s >= tCD, "gdn out S/Qb C=%d D=%d es=%d", C, D, es);
          CHECK(ol.b2 - ol.lam >= C * L * es, "gdn out lambda C=%d L=%d", C, L);
          CHECK(ol.total <= kLdsLimit, "gdn out LDS %d C=%d D=%d es=%d L=%d", ol.total, C, D, es, L);
          if (es == 2 && C == 64 && D == 64 && L == 15)
            CHECK(4 * ol.total <= kLdsLimit, "gdn out: four workgroups per CU at the 16K shape (%d)", ol.total);
          ++n;
        }
        for (long long T : {1LL, 15LL, 16LL, 100LL, 1000LL, 4097LL, 16384LL}) {
          GdnPlan p;
          const int dt = es == 2 ? kBF16 : kF32;
          if (plan_gdn(2, 3, T, D, D, C, dt, levels_needed(T), &p) != kOK) {
            CHECK(false, "gdn plan rejected T=%lld C=%d D=%d", T, C, D);
            continue;
          }
          const size_t DD = (size_t)D * D;
          CHECK(p.off_tb == 0 && p.ws_bytes >= (size_t)p.BH * p.n_chunks * C * C * es, "gdn tb T=%lld", T);
          if (p.n_nodes > 0) {
            CHECK(p.off_pt % 256 == 0 && p.off_pt >= (size_t)p.BH * p.n_chunks * C * C * es, "gdn pt T=%lld", T);
            CHECK(p.off_psit % 256 == 0 && p.off_psit >= p.off_pt + p.n_nodes * DD * es, "gdn psit T=%lld", T);
            CHECK(p.off_gn % 256 == 0 && p.off_gn >= p.off_psit + p.n_nodes * DD * es, "gdn gn T=%lld", T);
            CHECK(p.ws_bytes >= p.off_gn + p.n_nodes * 4, "gdn ws T=%lld", T);
          }
          // every block (m, x) a query chunk c reads, x = (c >> m) - 1 for a set
          // bit m of c, lies inside level m of the node array
          for (long long c = 0; c < p.n_chunks; ++c)
            for (int m = 0; m < 62 && (c >> m) != 0; ++m)
              if ((c >> m) & 1) {
                CHECK(m < p.n_tree && ((c >> m) - 1) < (p.n_full >> m), "gdn node T=%lld c=%lld m=%d", T, c, m);
                if (m + 1 < p.n_tree)
                  CHECK(p.lev_off[m] + p.BH * (p.n_full >> m) <= p.lev_off[m + 1], "gdn levels T=%lld", T);
              }
          ++n;
        }
      }
  std::printf("ok %d\n", n);
  return fails ? 1 : 0;
}
