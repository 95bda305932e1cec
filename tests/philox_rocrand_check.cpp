// Host-side cross-check of the oracle's Philox4x32-10 against rocRAND's
// open-source engine (header-only, compiled here from the ROCm headers).
// Reads lines "c0 c1 c2 c3 k0 k1" (hex words) from stdin and prints the four
// output words of one 10-round Philox4x32 call with that counter and key.
// rocRAND exposes the counter through (seed, subsequence, offset):
// key = seed, counter words 2-3 = subsequence, words 0-1 = offset / 4.
#include <rocrand/rocrand_kernel.h>
#include <cstdio>
int main() {
  unsigned c0,c1,c2,c3,k0,k1;
  while (scanf("%x %x %x %x %x %x", &c0,&c1,&c2,&c3,&k0,&k1) == 6) {
    unsigned long long seed = (unsigned long long)k0 | ((unsigned long long)k1 << 32);
    unsigned long long sub = (unsigned long long)c2 | ((unsigned long long)c3 << 32);
    unsigned long long off = 4ull * ((unsigned long long)c0 | ((unsigned long long)c1 << 32));
    rocrand_state_philox4x32_10 st;
    rocrand_init(seed, sub, off, &st);
    unsigned r0 = rocrand(&st), r1 = rocrand(&st), r2 = rocrand(&st), r3 = rocrand(&st);
    printf("%08x %08x %08x %08x\n", r0, r1, r2, r3);
  }
  return 0;
}
