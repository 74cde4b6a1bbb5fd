// Prints Philox4x32-10 output words from rocRAND's engine (host side) for
// counters (row, pos, 0, 0) under a 64-bit seed, one line per counter:
//   row pos w0 w1 w2 w3   (hex)
// Used only by the oracle's pin tests as an implementation independent of
// the oracle.  rocRAND's engine keys by the seed and advances its counter by
// offset/4 (low word first), so offset = 4 * (row + (pos << 32)) selects the
// counter (row, pos, 0, 0) in subsequence 0.
#include <rocrand/rocrand_philox4x32_10.h>
#include <cstdio>
#include <cstdlib>

int main(int argc, char** argv) {
    if (argc < 4) return 2;
    unsigned long long seed = strtoull(argv[1], nullptr, 0);
    int rows = atoi(argv[2]), pos = atoi(argv[3]);
    for (int r = 0; r < rows; ++r)
        for (int p = 0; p < pos; ++p) {
            unsigned long long off = 4ull * ((unsigned long long)r + ((unsigned long long)p << 32));
            rocrand_device::philox4x32_10_engine e(seed, 0, off);
            uint4 w = e.next4();
            printf("%d %d %08x %08x %08x %08x\n", r, p, w.x, w.y, w.z, w.w);
        }
    return 0;
}
