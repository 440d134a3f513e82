// Host-side known-answer helper: prints rocRAND's Philox4x32-10 output for a given
// key (k0 k1) and counter (c0 c1 c2 c3), all hex.  Used only by the oracle pin tests.
#include <rocrand/rocrand_philox4x32_10.h>
#include <cstdio>
#include <cstdlib>
int main(int argc, char** argv){
  // args: key0 key1 c0 c1 c2 c3 (hex)
  unsigned v[6]; for (int i = 0; i < 6; ++i) v[i] = (unsigned)strtoul(argv[i+1], 0, 16);
  unsigned long long seed = (unsigned long long)v[0] | ((unsigned long long)v[1] << 32);
  unsigned long long sub = (unsigned long long)v[4] | ((unsigned long long)v[5] << 32);
  unsigned long long off = ((unsigned long long)v[2] | ((unsigned long long)v[3] << 32)) * 4ull;
  rocrand_device::philox4x32_10_engine e(seed, sub, off);
  for (int i = 0; i < 4; ++i) printf("%08x ", e.next());
  printf("\n"); return 0;
}
