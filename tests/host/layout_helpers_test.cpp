// Host checks of helpers that the device code shares through layout.h. Built and run by
// tests/test_host_helpers.py with g++ (no GPU): exit status 0 when every check holds.
#include <cstdint>
#include <cstdio>
#include <initializer_list>

#include "layout.h"

static int failures = 0;
#define CHECK(c)                                              \
  do {                                                        \
    if (!(c)) {                                               \
      std::fprintf(stderr, "check failed: %s (line %d)\n", #c, __LINE__); \
      ++failures;                                             \
    }                                                         \
  } while (0)

int main() {
  using namespace amk;
  // buffer addresses: a low word with bit 31 set must not spill ones into the high word
  CHECK(address_from_words(0x00007fff, (int32_t)0x80001000u) == 0x00007fff80001000ull);
  CHECK(address_from_words(0x00000001, (int32_t)0xffffffffu) == 0x00000001ffffffffull);
  CHECK(address_from_words((int32_t)0x80000000u, 0) == 0x8000000000000000ull);
  CHECK(address_from_words(0, 0x12345678) == 0x12345678ull);
  for (uint64_t a : {0x0ull, 0x7ffff0001000ull, 0x7fff8000aa00ull, 0x1234ffffffffull}) {
    const int32_t hi = (int32_t)(uint32_t)(a >> 32), lo = (int32_t)(uint32_t)a;
    CHECK(address_from_words(hi, lo) == a);
  }
  // KV blocks partition [0, ctx) in order, for every block count
  for (int ctx = 1; ctx <= 300; ctx += 7)
    for (int nblk = 1; nblk <= 40; ++nblk) {
      int prev = 0;
      for (int b = 0; b < nblk; ++b) {
        int lo, hi;
        attn_block_range(ctx, nblk, b, &lo, &hi);
        CHECK(lo == prev && hi >= lo);
        prev = hi;
      }
      CHECK(prev == ctx);
    }
  // packed QKV rows map one to one onto the source rows of q, k and v
  const int nq = 8, nkv = 2, hd = 16;
  int seen[3][8 * 16] = {};
  for (int r = 0; r < qkv_rows(nq, nkv, hd); ++r) {
    const QkvRow q = qkv_decode(r, nq, nkv, hd);
    seen[q.kind][q.head * hd + q.dim]++;
    if (q.kind != KIND_V && (r % 2) == 0) {  // rotary rows come in pairs (j, j + hd / 2)
      const QkvRow p = qkv_decode(r + 1, nq, nkv, hd);
      CHECK(p.kind == q.kind && p.head == q.head && p.dim == q.dim + hd / 2);
    }
  }
  for (int i = 0; i < nq * hd; ++i) CHECK(seen[KIND_Q][i] == 1);
  for (int i = 0; i < nkv * hd; ++i) CHECK(seen[KIND_K][i] == 1 && seen[KIND_V][i] == 1);
  std::printf("%s\n", failures ? "FAILED" : "ok");
  return failures ? 1 : 0;
}
