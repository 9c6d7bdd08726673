// plan_driver.cpp -- drives the host-side planner over every workload shape
// and a grid of caller-made plans, for a build under AddressSanitizer and
// UndefinedBehaviorSanitizer (CPU only; no HIP call is made).  Prints a
// summary line; any sanitizer report aborts the process.
#include <stdio.h>
#include <string.h>

#include "skinny_gemm.h"

// Equal in every field but from_table (a completed caller plan is not the
// table's, by definition).
static int same(SkgPlan a, SkgPlan b) {
    a.from_table = b.from_table = 0;
    return memcmp(&a, &b, sizeof a) == 0;
}

int main() {
    const int dtypes[] = {SKG_DTYPE_BF16, SKG_DTYPE_FP8, SKG_DTYPE_FP8_MX};
    const int Ks[] = {2048, 2880, 4096, 6144, 7168, 8, 16, 32, 1040, 4112, 0, 7, 1 << 20};
    const int Ns[] = {128, 256, 384, 576, 2112, 4096, 1, 7, 65536, 0};
    const int cus[] = {1, 8, 80, 104, 256, 304};
    long planned = 0, failed = 0, mismatched = 0;
    // every workload shape (and edges) through the planner, then back
    // through plan completion, which must accept it unchanged
    for (int dt : dtypes)
        for (int K : Ks)
            for (int N : Ns)
                for (int M = 0; M <= 513; M += (M < 20 ? 1 : 7)) {
                    SkgPlan p;
                    memset(&p, 0xA5, sizeof p);
                    int rc = skinny_gemm_plan(M, N, K, dt, &p);
                    ++planned;
                    if (rc != SKG_OK) {
                        ++failed;
                        continue;
                    }
                    if (M == 0 || N == 0) continue;  // an empty call needs no plan
                    SkgPlan q = p;
                    if (skinny_gemm_plan_complete(M, N, K, dt, &q) != SKG_OK || !same(p, q))
                        ++mismatched;
                    for (int c : cus) {
                        SkgPlan r;
                        (void)skinny_gemm_plan_on(M, N, K, dt, c, &r);
                    }
                }
    // a grid of caller-made plans, valid and not, at a few shapes
    const int shapes[][3] = {{1, 256, 7168}, {16, 384, 7168}, {128, 4096, 7168}, {512, 4096, 7168},
                             {5, 100, 2056}, {300, 7, 4096}, {64, 2112, 2880}};
    const int kinds[] = {-1, 0, 1, 2, 3, 4};
    const int threads[] = {-64, 0, 63, 64, 192, 256, 1024, 2048};
    const int colss[] = {-1, 0, 1, 2, 3, 4, 5, 8, 16, 17};
    const int splitss[] = {-1, 0, 1, 2, 7, 64, 256, 257};
    const int depths[] = {-1, 0, 1, 2, 3, 4, 8, 16, 17};
    const int wms[] = {0, 1, 2, 3, 4};
    const int reduces[] = {-1, 0, 1, 2, 3};
    const int flagss[] = {0, 1, 2, 3};
    long tried = 0, accepted = 0;
    for (const auto &sh : shapes)
        for (int dt : dtypes)
            for (int kd : kinds)
                for (int t : threads)
                    for (int c : colss)
                        for (int s : splitss)
                            for (int d : depths)
                                for (int wm : wms)
                                    for (int rd : reduces)
                                        for (int fl : flagss) {
                                            SkgPlan p;
                                            memset(&p, 0, sizeof p);
                                            p.kind = kd;
                                            p.threads = t;
                                            p.cols = c;
                                            p.splits = s;
                                            p.depth = d;
                                            p.waves_m = wm;
                                            p.reduce = rd;
                                            p.flags = fl;
                                            ++tried;
                                            if (skinny_gemm_plan_complete(sh[0], sh[1], sh[2], dt,
                                                                          &p) == SKG_OK)
                                                ++accepted;
                                        }
    printf("planned %ld (rejected %ld, round-trip mismatches %ld); caller plans %ld (accepted %ld)\n",
           planned, failed, mismatched, tried, accepted);
    return mismatched != 0;
}
