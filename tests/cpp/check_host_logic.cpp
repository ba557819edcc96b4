// Host-side checks of the bucket enumeration and of the argument checks of
// the C ABI (compiled with g++ under the address and undefined-behaviour
// sanitizers by tests/test_plan_layouts.py; no GPU).  Prints one line per
// failure and "ok <n>" with the number of cases checked.
//
// Bucket enumeration: for chunks of 2^log2C tokens, a key token s in an
// earlier chunk than query token t sits at Fenwick level 1 + msb(t xor s)
// ("Log-Linear Attention", Italian summary, technical section 2, item 1);
// with whole chunks that is log2C + 1 + msb(ct xor cs).  The buckets the
// output kernel visits must cover every earlier chunk exactly once, each at
// that level, for every group size.
#include <cstdio>
#include <cstdint>
#include <initializer_list>
#include <vector>

#include "../../fenwick_tree_hierarchical_amd/csrc/la_levels.hpp"
#include "../../fenwick_tree_hierarchical_amd/csrc/la_validate.hpp"

using namespace la;

static int fails = 0;
static int64_t cases = 0;
#define CHECK(cond, ...)                   \
  do {                                     \
    ++cases;                               \
    if (!(cond)) {                         \
      if (++fails <= 50) {                 \
        std::printf("FAIL %s: ", #cond);   \
        std::printf(__VA_ARGS__);          \
        std::printf("\n");                 \
      }                                    \
    }                                      \
  } while (0)

// Most significant set bit of x > 0, by shifting (independent of the
// library's helpers).
static int msb(uint64_t x) {
  int m = -1;
  while (x) {
    x >>= 1;
    ++m;
  }
  return m;
}

static void check_enumeration() {
  for (int log2C = 4; log2C <= 7; ++log2C)
    for (int log2G = 0; log2G <= 3; ++log2G) {
      const int64_t n_chunks = 1100;  // spans 10 group levels at G = 1, a ragged top
      std::vector<int> seen(n_chunks);
      for (int64_t ct = 0; ct < n_chunks; ++ct) {
        // Pointwise: the enumerated level of every earlier chunk.
        for (int64_t cs = 0; cs < ct; ++cs) {
          const int want = log2C + 1 + msb((uint64_t)(ct ^ cs));
          const int got = enumerated_chunk_level(ct, cs, log2C, log2G);
          CHECK(got == want, "log2C=%d log2G=%d ct=%lld cs=%lld got %d want %d", log2C, log2G, (long long)ct,
                (long long)cs, got, want);
        }
        CHECK(enumerated_chunk_level(ct, ct, log2C, log2G) == -1, "own chunk ct=%lld", (long long)ct);
        CHECK(enumerated_chunk_level(ct, ct + 1, log2C, log2G) == -1, "later chunk ct=%lld", (long long)ct);
        // Partition: the buckets cover 0..ct-1 exactly once.
        for (int64_t c = 0; c < ct; ++c) seen[c] = 0;
        for (int j = 1; j <= log2G; ++j) {
          const BucketRef b = chunk_level_bucket(ct, j, log2C, log2G);
          if (!b.occupied) continue;
          CHECK(b.level == log2C + j, "chunk level ct=%lld j=%d", (long long)ct, j);
          for (int64_t c = b.last - (1ll << (j - 1)) + 1; c <= b.last; ++c) {
            CHECK(c >= 0 && c < ct, "chunk bucket out of range ct=%lld j=%d c=%lld", (long long)ct, j,
                  (long long)c);
            if (c >= 0 && c < ct) ++seen[c];
          }
        }
        for (int i = 1; i <= 62; ++i) {
          const BucketRef b = group_level_bucket(ct, i, log2C, log2G);
          if (!b.occupied) continue;
          CHECK(b.level == log2C + log2G + i, "group level ct=%lld i=%d", (long long)ct, i);
          const int64_t c0 = (b.last - (1ll << (i - 1)) + 1) << log2G, c1 = (b.last + 1) << log2G;
          for (int64_t c = c0; c < c1; ++c) {
            CHECK(c >= 0 && c < ct, "group bucket out of range ct=%lld i=%d c=%lld", (long long)ct, i,
                  (long long)c);
            if (c >= 0 && c < ct) ++seen[c];
          }
        }
        for (int64_t c = 0; c < ct; ++c)
          CHECK(seen[c] == 1, "log2C=%d log2G=%d ct=%lld chunk %lld covered %d times", log2C, log2G,
                (long long)ct, (long long)c, seen[c]);
      }
      // Far chunk indices (T near 2^40 tokens): pointwise only, sampled.
      for (int64_t ct : {int64_t(1) << 33, (int64_t(1) << 33) + 12345, (int64_t(1) << 34) - 1})
        for (int64_t cs : {int64_t(0), int64_t(1), ct / 3, ct - 9, ct - 1}) {
          const int want = log2C + 1 + msb((uint64_t)(ct ^ cs));
          CHECK(enumerated_chunk_level(ct, cs, log2C, log2G) == want, "far ct=%lld cs=%lld", (long long)ct,
                (long long)cs);
        }
    }
}

// Addresses that are never dereferenced: the checks only look at the values.
static const void* at(uintptr_t a) { return reinterpret_cast<const void*>(a); }
static const float* fat(uintptr_t a) { return reinterpret_cast<const float*>(a); }

static void check_validation() {
  // Forward: d = 64, C = 64, bf16, 2 heads of 4096 tokens.
  FwdPlan p{};
  CHECK(plan_fwd(1, 2, 4096, 64, 64, 64, kBF16, -1, &p) == kOK, "plan_fwd");
  const uintptr_t A = 0x100000;  // 256-byte aligned
  const void *q = at(A), *k = at(A + 0x1000), *v = at(A + 0x2000), *o = at(A + 0x3000), *ws = at(A + 0x4000);
  const float *la = fat(A + 0x5000), *lam = fat(A + 0x6000);
  CHECK(check_fwd_buffers(p, q, k, v, la, lam, o, ws, p.ws_bytes) == kOK, "fwd ok");
  CHECK(check_fwd_buffers(p, nullptr, k, v, la, lam, o, ws, p.ws_bytes) == kEINVAL, "fwd null q");
  CHECK(check_fwd_buffers(p, q, k, v, nullptr, lam, o, ws, p.ws_bytes) == kEINVAL, "fwd null log_a");
  CHECK(check_fwd_buffers(p, at(A + 8), k, v, la, lam, o, ws, p.ws_bytes) == kEALIGN, "fwd q align");
  CHECK(check_fwd_buffers(p, q, k, v, fat(A + 0x5002), lam, o, ws, p.ws_bytes) == kEALIGN, "fwd log_a align");
  CHECK(check_fwd_buffers(p, q, k, v, la, lam, o, ws, p.ws_bytes - 1) ==
            (p.ws_bytes > 0 ? kEWORKSPACE : kOK), "fwd small workspace");
  CHECK(check_fwd_buffers(p, q, k, v, la, lam, o, nullptr, p.ws_bytes) ==
            (p.ws_bytes > 0 ? kEWORKSPACE : kOK), "fwd null workspace");
  if (p.ws_bytes > 0)
    CHECK(check_fwd_buffers(p, q, k, v, la, lam, o, at(A + 0x4010), p.ws_bytes) == kEALIGN, "fwd ws align");

  // The state of a forward with an exported decode state.
  la_state st{};
  st.B = 1; st.H = 2; st.dk = 64; st.dv = 64; st.S = 13; st.t = 0;
  st.slots = const_cast<float*>(fat(A + 0x7000)); st.scale = const_cast<float*>(fat(A + 0x8000));
  CHECK(check_fwd_state(p, &st) == kOK, "state ok (13 slots for 4096 tokens)");
  st.S = 12;
  CHECK(check_fwd_state(p, &st) == kECAPACITY, "state 12 slots");
  st.S = 13; st.H = 3;
  CHECK(check_fwd_state(p, &st) == kESHAPE, "state heads");
  st.H = 2; st.slots = nullptr;
  CHECK(check_fwd_state(p, &st) == kEINVAL, "state null slots");
  st.slots = const_cast<float*>(fat(A + 0x7004));
  CHECK(check_fwd_state(p, &st) == kEALIGN, "state slot align");
  st.slots = const_cast<float*>(fat(A + 0x7000));

  // Backward.
  BwdPlan P{};
  CHECK(plan_bwd(1, 2, 4096, 64, 64, 64, kBF16, -1, &P) == kOK, "plan_bwd");
  const void *gq = at(A + 0x9000), *gk = at(A + 0xa000), *gv = at(A + 0xb000), *dout = at(A + 0xc000);
  const float *gla = fat(A + 0xd000), *glam = fat(A + 0xe000);
  CHECK(check_bwd_buffers(P, q, k, v, la, lam, dout, gq, gk, gv, gla, glam, ws, P.ws_bytes) == kOK, "bwd ok");
  CHECK(check_bwd_buffers(P, q, k, v, la, lam, dout, gq, gk, gv, gla, nullptr, ws, P.ws_bytes) == kEINVAL,
        "bwd null grad_lambda");
  CHECK(check_bwd_buffers(P, q, k, v, la, lam, dout, at(A + 0x9004), gk, gv, gla, glam, ws, P.ws_bytes) == kEALIGN,
        "bwd grad_q align");
  CHECK(check_bwd_buffers(P, q, k, v, la, lam, dout, gq, gk, gv, gla, glam, ws, P.ws_bytes - 1) == kEWORKSPACE,
        "bwd small workspace");

  // Gated DeltaNet.
  GdnPlan g{};
  CHECK(plan_gdn(1, 2, 4096, 64, 64, 64, kBF16, -1, &g) == kOK, "plan_gdn");
  const float* beta = fat(A + 0xf000);
  CHECK(check_gdn_buffers(g, q, k, v, la, beta, lam, o, ws, g.ws_bytes) == kOK, "gdn ok");
  CHECK(check_gdn_buffers(g, q, k, v, la, nullptr, lam, o, ws, g.ws_bytes) == kEINVAL, "gdn null beta");
  CHECK(check_gdn_buffers(g, q, k, v, la, fat(A + 0xf001), lam, o, ws, g.ws_bytes) == kEALIGN, "gdn beta align");
  CHECK(check_gdn_buffers(g, q, k, v, la, beta, lam, o, at(A + 0x4040), g.ws_bytes) == kEALIGN, "gdn ws align");

  // Decode: the merge at position t needs trailing_ones(t) + 1 slots and
  // bit_length(t) slots.
  int kstar = -1;
  st.t = 0;
  CHECK(check_decode(&st, q, k, v, la, lam, o, kBF16, &kstar) == kOK && kstar == 0, "decode t=0");
  st.t = (1 << 12) - 1;  // 12 trailing ones: the merge fills level 13
  CHECK(check_decode(&st, q, k, v, la, lam, o, kBF16, &kstar) == kOK && kstar == 12, "decode t=4095");
  st.t = (1 << 13) - 1;  // 13 trailing ones: level 14 does not exist
  CHECK(check_decode(&st, q, k, v, la, lam, o, kBF16, &kstar) == kECAPACITY, "decode t=8191");
  st.t = 1 << 13;  // bit length 14 > 13 slots
  CHECK(check_decode(&st, q, k, v, la, lam, o, kBF16, &kstar) == kECAPACITY, "decode t=8192");
  st.t = -1;
  CHECK(check_decode(&st, q, k, v, la, lam, o, kBF16, &kstar) == kEINVAL, "decode t<0");
  st.t = 5;
  CHECK(check_decode(&st, q, k, v, la, lam, o, 7, &kstar) == kEDTYPE, "decode dtype");
  CHECK(check_decode(nullptr, q, k, v, la, lam, o, kBF16, &kstar) == kEINVAL, "decode null state");
  CHECK(check_decode(&st, q, k, v, la, lam, nullptr, kBF16, &kstar) == kEINVAL, "decode null out");
  CHECK(check_decode(&st, q, k, v, la, lam, at(A + 0x3002), kBF16, &kstar) == kEALIGN, "decode out align");
  st.B = 0;  // nothing to step: tensors unchecked
  CHECK(check_decode(&st, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, kBF16, &kstar) == kOK,
        "decode empty batch");
}

int main() {
  check_enumeration();
  check_validation();
  if (fails) {
    std::printf("%d failures\n", fails);
    return 1;
  }
  std::printf("ok %lld\n", (long long)cases);
  return 0;
}
