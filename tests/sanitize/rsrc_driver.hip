// rsrc_driver.hip -- CPU pins (tests/test_host_sanitizers.py) of the GEMM
// kernel's buffer-resource range arithmetic (csrc/dg_rsrc.h), the code whose
// unclamped form once let an empty scale resource wrap to a 4 GB range and
// read near address zero.  Host code only; built with the host sanitizers.
#include <stdio.h>

#include "../../moe_grouped_gemm_x128_amd/csrc/dg_rsrc.h"

static int bad = 0;
#define CHECK(c)                                                     \
  do {                                                               \
    if (!(c)) {                                                      \
      fprintf(stderr, "check failed line %d: %s\n", __LINE__, #c);  \
      bad++;                                                         \
    }                                                                \
  } while (0)

int main() {
  using dg::base_moved;
  using dg::range_after;
  using dg::range_at_k;
  // moving inside the range keeps its end; reaching or passing it empties it
  CHECK(range_after(1000, 0, true) == 1000);
  CHECK(range_after(1000, 999, true) == 1);
  CHECK(range_after(1000, 1000, true) == 0);
  CHECK(range_after(1000, 1001, true) == 0);
  CHECK(range_after(1000, 0xffffffffu, true) == 0);
  CHECK(range_after(0, 0, true) == 0);
  CHECK(range_after(0, 128, true) == 0);  // an empty resource never wraps
  CHECK(range_after(1000, 5, false) == 0);
  // K offsets: empty stays empty at every K block, dead blocks read nothing
  for (uint32_t kb = 0; kb < 4096; ++kb) CHECK(range_at_k(0, kb * 128u, true) == 0);
  CHECK(range_at_k(7168 * 3, 128 * 55, false) == 0);
  // a resource of r >= 1 whole rows of L bytes, moved to K offsets below L,
  // keeps a positive range that ends where it did
  for (uint32_t rows = 1; rows <= 300; rows += 7)
    for (uint32_t blocks = 1; blocks <= 160; blocks += 9) {
      const uint32_t len = blocks * 128u, num = rows * len;
      for (uint32_t kb = 0; kb < blocks; ++kb) {
        const uint32_t r = range_at_k(num, kb * 128u, true);
        CHECK(r > 0 && r == num - kb * 128u && r == range_after(num, kb * 128u, true));
      }
    }
  // the 48-bit base carries into the high word and stays 48 bits wide
  uint32_t lo, hi;
  base_moved(0xffffff80u, 0x1234u, 0x100u, &lo, &hi);
  CHECK(lo == 0x80u && hi == 0x1235u);
  base_moved(0xffffffffu, 0xffffu, 1u, &lo, &hi);
  CHECK(lo == 0u && hi == 0u);
  base_moved(0x10u, 0x7u, 0u, &lo, &hi);
  CHECK(lo == 0x10u && hi == 0x7u);
  printf("bad=%d\n", bad);
  return bad != 0;
}
