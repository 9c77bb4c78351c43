// Host-only driver for the library's index map header (compiled with g++ by
// tests/test_abi_host.py; no GPU). Two modes:
//   fastdiv                      exhaustive/random check of FastDiv against '/'
//   table T H W wt wh ww st sh sw out.bin
//                                write the membership table token_of(window, slot)
//                                as int32, to be compared with the oracle's table.
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "index_map.hpp"

static int check_fastdiv() {
  uint64_t state = 0x9E3779B97F4A7C15ull;
  auto rnd = [&]() {
    state ^= state << 13; state ^= state >> 7; state ^= state << 17;
    return state;
  };
  // every divisor up to 4096 against every numerator up to 2^16, plus the top range
  for (uint32_t d = 1; d <= 4096; ++d) {
    const basa::FastDiv f = basa::make_fastdiv(d);
    for (uint32_t n = 0; n < (1u << 16); ++n)
      if (basa::fdiv(n, f) != n / d) { printf("FAIL d=%u n=%u\n", d, n); return 1; }
    for (uint32_t n = 0x7fffffffu - 4096; n != 0x80000000u; ++n)
      if (basa::fdiv(n, f) != n / d) { printf("FAIL d=%u n=%u\n", d, n); return 1; }
  }
  // random divisors and numerators over the whole 31-bit range
  for (int it = 0; it < 20000000; ++it) {
    uint32_t d = uint32_t(rnd() % 0x7fffffffu) + 1u;
    if (it & 1) d = uint32_t(rnd() % 70000u) + 1u;
    const uint32_t n = uint32_t(rnd() & 0x7fffffffu);
    if (basa::fdiv(n, basa::make_fastdiv(d)) != n / d) { printf("FAIL d=%u n=%u\n", d, n); return 1; }
  }
  // powers of two and their neighbours
  for (int s = 0; s < 31; ++s)
    for (int delta = -1; delta <= 1; ++delta) {
      const int64_t d64 = (int64_t(1) << s) + delta;
      if (d64 < 1 || d64 > 0x7fffffff) continue;
      const basa::FastDiv f = basa::make_fastdiv(uint32_t(d64));
      for (int it = 0; it < 100000; ++it) {
        const uint32_t n = uint32_t(rnd() & 0x7fffffffu);
        if (basa::fdiv(n, f) != n / uint32_t(d64)) { printf("FAIL d=%lld n=%u\n", (long long)d64, n); return 1; }
      }
    }
  printf("fastdiv ok\n");
  return 0;
}

int main(int argc, char** argv) {
  if (argc == 2 && !strcmp(argv[1], "fastdiv")) return check_fastdiv();
  if (argc == 12 && !strcmp(argv[1], "table")) {
    int a[9];
    for (int i = 0; i < 9; ++i) a[i] = atoi(argv[2 + i]);
    const int T = a[0], H = a[1], W = a[2], wt = a[3], wh = a[4], ww = a[5];
    auto red = [](int s, int n) { int r = s % n; return r < 0 ? r + n : r; };
    const basa::WinMap m = basa::make_winmap(T, H, W, wt, wh, ww, red(a[6], T), red(a[7], H), red(a[8], W));
    const int wtok = wt * wh * ww, nwin = T * H * W / wtok;
    FILE* f = fopen(argv[11], "wb");
    if (!f) return 2;
    for (int win = 0; win < nwin; ++win) {
      const basa::WinOrigin o = basa::window_origin(m, uint32_t(win));
      for (int l = 0; l < wtok; ++l) {
        const int32_t tok = basa::token_of(m, o, uint32_t(l));
        fwrite(&tok, 4, 1, f);
      }
    }
    fclose(f);
    return 0;
  }
  fprintf(stderr, "usage: fastdiv | table T H W wt wh ww st sh sw out.bin\n");
  return 2;
}
