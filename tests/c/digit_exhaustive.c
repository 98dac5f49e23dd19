/* Exhaustive check of the oracle's signed-digit split over all 2^32 words:
 * each digit lies in [-128, 127] and the digits reconstruct the word mod 2^32.
 * The reconstruction here is independent of the split's own code. */
#include <stdint.h>
#include <stdio.h>
#include "oracle.h"

int main(void) {
  uint64_t bad = 0, n = 0;
  int8_t s[4];
  for (uint64_t x = 0; x <= 0xFFFFFFFFull; ++x) {
    oracle_signed_digits((uint32_t)x, s);
    uint32_t y = 0;
    for (int j = 0; j < 4; ++j) {
      if (s[j] < -128 || s[j] > 127) ++bad;
      y += (uint32_t)((int32_t)s[j] * (int32_t)(1 << (8 * j)));  /* wraps mod 2^32 */
    }
    if (y != (uint32_t)x) {
      if (bad < 5) printf("mismatch at %08llx\n", (unsigned long long)x);
      ++bad;
    }
    ++n;
  }
  printf("checked %llu words, %llu bad\n", (unsigned long long)n, (unsigned long long)bad);
  return bad != 0;
}
