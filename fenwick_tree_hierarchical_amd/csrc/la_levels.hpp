// The Fenwick buckets above a query chunk, as the forward's output kernel
// enumerates them ("Log-Linear Attention", Italian summary, technical
// section 2, item 1; Spanish summary, technical section 2, "Conceptos
// clave": a query sees its prefix cut into power-of-two buckets, the recent
// ones small and the old ones large).  With chunks of 2^log2C tokens and
// groups of 2^log2G chunks, a pair in different chunks sits at level
// log2C + 1 + msb(chunk_t xor chunk_s); the buckets of those levels are whole
// chunks (levels log2C + 1 .. log2C + log2G, inside the query's group) or
// whole groups (the levels above).  The level-table export walks the same
// enumeration for every pair in different chunks, so its byte-exact check
// covers the output kernel's bucket list; tests/cpp checks it against the
// closed form on the host for every group size.
//
// Pure C++17 (host and device).
#pragma once

#include <stdint.h>

#if defined(__HIPCC__)
#define LA_LV_HD __host__ __device__
#else
#define LA_LV_HD
#endif

namespace la {

struct BucketRef {
  bool occupied;   // the query chunk has a bucket at this level
  int64_t last;    // its last chunk (chunk levels) or last group (group levels)
  int level;       // Fenwick level of every pair in it
};

// Chunk level j (1 <= j <= log2G) above query chunk c: occupied when bit j-1
// of c's index inside its group is set; the bucket is the 2^(j-1) chunks
// ending at chunk `last`.
LA_LV_HD inline BucketRef chunk_level_bucket(int64_t c, int j, int log2C, int log2G) {
  const int64_t ci = c & ((1ll << log2G) - 1), c0 = c - ci;
  BucketRef b{false, 0, 0};
  if (j >= 1 && j <= log2G && ((ci >> (j - 1)) & 1)) {
    b.occupied = true;
    b.last = c0 + ((ci >> j) << j) + (1ll << (j - 1)) - 1;
    b.level = log2C + j;
  }
  return b;
}

// Group level i (1 <= i <= 62) above query chunk c: occupied when bit i-1 of
// the group index g = c >> log2G is set; the bucket is the 2^(i-1) groups
// ending at group `last`.
LA_LV_HD inline BucketRef group_level_bucket(int64_t c, int i, int log2C, int log2G) {
  const int64_t g = c >> log2G;
  BucketRef b{false, 0, 0};
  if (i >= 1 && i <= 62 && ((g >> (i - 1)) & 1)) {
    b.occupied = true;
    b.last = ((g >> i) << i) + (1ll << (i - 1)) - 1;
    b.level = log2C + log2G + i;
  }
  return b;
}

// Level of the bucket of query chunk ct that holds key chunk cs < ct, found
// by walking the enumeration; -1 when none holds it.
LA_LV_HD inline int enumerated_chunk_level(int64_t ct, int64_t cs, int log2C, int log2G) {
  for (int j = 1; j <= log2G; ++j) {
    const BucketRef b = chunk_level_bucket(ct, j, log2C, log2G);
    if (b.occupied && cs <= b.last && cs > b.last - (1ll << (j - 1))) return b.level;
  }
  for (int i = 1; i <= 62 && (ct >> log2G) >> (i - 1); ++i) {
    const BucketRef b = group_level_bucket(ct, i, log2C, log2G);
    if (!b.occupied) continue;
    const int64_t g0 = b.last - (1ll << (i - 1)) + 1;
    if (cs >= (g0 << log2G) && cs < ((b.last + 1) << log2G)) return b.level;
  }
  return -1;
}

}  // namespace la
