// Host-only cross-check program: reads "seed c0 c1 c2 c3" lines and prints the
// four 32-bit words of rocRAND's Philox4x32-10 at counter (c0, c1, c2, c3)
// under key (seed mod 2^32, seed >> 32). rocRAND places the 64-bit offset/4 in
// counter words 0-1 and the subsequence in words 2-3, so the raw counter maps
// to subsequence = c2 | c3 << 32 and offset = 4 * (c0 | c1 << 32).
#include <rocrand/rocrand_philox4x32_10.h>
#include <cstdio>

int main() {
  unsigned long long seed;
  unsigned c0, c1, c2, c3;
  while (std::scanf("%llu %u %u %u %u", &seed, &c0, &c1, &c2, &c3) == 5) {
    rocrand_state_philox4x32_10 st;
    unsigned long long sub = (unsigned long long)c2 | ((unsigned long long)c3 << 32);
    unsigned long long off = 4ull * ((unsigned long long)c0 | ((unsigned long long)c1 << 32));
    rocrand_init(seed, sub, off, &st);
    uint4 r = rocrand4(&st);
    std::printf("%u %u %u %u\n", r.x, r.y, r.z, r.w);
  }
  return 0;
}
