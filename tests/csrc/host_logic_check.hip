// Host-only checks of the launchers' integer and fp8 decisions (no GPU use):
//   div   - row / d by multiply-shift (div_magic_for) against integer division
//           for every d in [1, 4096] at rows spread over [0, 2^31), including
//           every multiple of d near the top and the rows around them;
//   clamp - for each fp8_max given on the command line (as a decimal), whether
//           the launchers clamp quotients before encoding (fp8_clamp_needed),
//           printed as "<fp8_max> <0|1>" for the caller to compare;
//   layout - for each line "G heads heads0 total_rows xs0 head_dim rope pos
//           max_pos" on stdin, the row kernel's pass layout (rows_layout),
//           printed as "<layout> <tok_shift>" (tok_shift -1 unless whole
//           tokens) for the caller to compare.
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "rnq_launch.h"

static int check_div() {
  long bad = 0, checked = 0;
  for (uint32_t d = 1; d <= 4096; ++d) {
    uint32_t magic, shift;
    rnq::div_magic_for(d, magic, shift);
    auto one = [&](uint64_t n) {
      if (n >= (1ull << 31)) return;
      const uint32_t got = (uint32_t)((n * magic) >> shift);
      checked++;
      if (got != n / d) {
        if (bad < 10) printf("div: d %u row %llu: %u != %llu\n", d, (unsigned long long)n, got, (unsigned long long)(n / d));
        bad++;
      }
    };
    for (uint64_t n = 0; n < 4 * d + 4; ++n) one(n);
    const uint64_t top = (1ull << 31) - 1;
    for (uint64_t k = 0; k < 64; ++k) {  // the last multiples of d below 2^31, +-1
      const uint64_t m = (top / d - k) * d;
      one(m - 1); one(m); one(m + 1);
    }
    for (uint64_t n = d; n < (1ull << 31); n = n * 3 + 7) { one(n - 1); one(n); one(n + 1); }
  }
  printf("div: %ld rows checked, %ld wrong\n", checked, bad);
  return bad == 0 ? 0 : 1;
}

int main(int argc, char** argv) {
  if (argc >= 2 && strcmp(argv[1], "div") == 0) return check_div();
  if (argc >= 2 && strcmp(argv[1], "clamp") == 0) {
    for (int i = 2; i < argc; ++i) {
      const float f = strtof(argv[i], nullptr);
      printf("%s %d\n", argv[i], rnq::fp8_clamp_needed(f) ? 1 : 0);
    }
    return 0;
  }
  if (argc >= 2 && strcmp(argv[1], "layout") == 0) {
    unsigned G, heads, heads0, rows, head_dim, rope, pos, max_pos;
    unsigned long long xs0;
    while (scanf("%u %u %u %u %llu %u %u %u %u", &G, &heads, &heads0, &rows, &xs0, &head_dim, &rope, &pos,
                 &max_pos) == 9) {
      uint32_t sh = 0xffffffffu;
      const int a = rnq::rows_layout(G, heads, heads0, rows, xs0, head_dim, rope, pos != 0, max_pos, &sh);
      printf("%d %d\n", a, a == rnq::ROWS_WHOLE_TOKENS ? (int)sh : -1);
    }
    return 0;
  }
  fprintf(stderr, "usage: host_logic_check div | clamp <fp8_max>... | layout < cases\n");
  return 2;
}
