// Checks full_kv_block_range / full_q_block_range (the per-wave FULL block ranges the kernels
// use to skip the class test) against block_class itself, block by block, over square and
// rectangular lengths, causal / window / neither, and tile sizes from 1 to 128.
// Prints the number of blocks checked and of mismatches; exit status 1 on any mismatch.
#include <cstdio>

#include "block_class.h"

using namespace fa;

int main() {
    long n = 0, bad = 0;
    const int Ts[] = {1, 2, 5, 31, 32, 33, 64, 65, 100, 129, 257};
    const int bs[] = {1, 3, 16, 32, 64, 128};
    const int Ws[] = {0, 1, 2, 17, 64, 100, 300};
    for (int Tq : Ts)
        for (int Tk : Ts)
            for (int causal = 0; causal < 2; ++causal)
                for (int W : Ws)
                    for (int bq : bs)
                        for (int bk : bs) {
                            for (int r0 = 0; r0 < Tq + bq; r0 += bq) {
                                int lo, hi;
                                full_kv_block_range(Tq, Tk, r0, r0 + bq, bk, causal, W, lo, hi);
                                for (int j = 0; j * bk < Tk + bk; ++j, ++n) {
                                    const bool full = block_class(Tq, Tk, r0, r0 + bq, j * bk, j * bk + bk, causal, W) == kFull;
                                    if (full != (j >= lo && j < hi)) {
                                        if (bad++ < 10)
                                            std::printf("kv: Tq=%d Tk=%d causal=%d W=%d bq=%d bk=%d r0=%d j=%d\n",
                                                        Tq, Tk, causal, W, bq, bk, r0, j);
                                    }
                                }
                            }
                            for (int c0 = 0; c0 < Tk + bk; c0 += bk) {
                                int lo, hi;
                                full_q_block_range(Tq, Tk, c0, c0 + bk, bq, causal, W, lo, hi);
                                for (int i = 0; i * bq < Tq + bq; ++i, ++n) {
                                    const bool full = block_class(Tq, Tk, i * bq, i * bq + bq, c0, c0 + bk, causal, W) == kFull;
                                    if (full != (i >= lo && i < hi)) {
                                        if (bad++ < 10)
                                            std::printf("q: Tq=%d Tk=%d causal=%d W=%d bq=%d bk=%d c0=%d i=%d\n",
                                                        Tq, Tk, causal, W, bq, bk, c0, i);
                                    }
                                }
                            }
                        }
    std::printf("checked %ld mismatches %ld\n", n, bad);
    return bad != 0;
}
