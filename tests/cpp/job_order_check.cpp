// Host-side check of the attention-backward workgroup order (bwd_job in
// backward.hpp), run by tests/test_job_order.py: over many shapes, the order
// must issue every (group, sequence, job) exactly once, the dK/dV jobs in
// non-increasing order of work (rows walked), and the dQ jobs in order of
// decreasing end token up to one tile. Prints OK or the first failures.
#include "backward.hpp"

#include <cstdio>
#include <vector>

using namespace gqe;

static int bad = 0;
static void fail(const char* what, int T, int R, int Bt, int G, int s0, int kind, long L) {
    if (++bad <= 10) std::printf("%s: T=%d R=%d Bt=%d G=%d s0=%d kind=%d L=%ld\n", what, T, R, Bt, G, s0, kind, L);
}

int main() {
    for (int T : {1, 2, 37, 128, 200, 255, 256, 257, 1000, 2048, 32768, 262144 + 1037})
        for (int R : {1, 2, 4})
            for (int Bt : {1, 2, 3, 8})
                for (int G : {1, 2, 3, 8, 10})
                    for (int s0 : {-1, 0, 1, 7}) {
                        if (s0 >= G) continue;
                        RowSpace rs{};
                        rs.T = T;
                        rs.Bt = Bt;
                        rs.R = R;
                        rs.s0 = s0;
                        // 0: dK/dV (128 keys), 1: dK/dV (256 keys), 2: dQ (128 rows)
                        for (int cfg = 0; cfg < 3; ++cfg) {
                            const int kind = cfg < 2 ? 0 : 1;
                            const int64_t BS = cfg == 1 ? 256 : 128;
                            const int64_t n_r = kind == 0 ? (T + BS - 1) / BS : ((int64_t)T * R + BS - 1) / BS;
                            const int64_t n_x = kind == 0 ? n_r : ((int64_t)T * (R + 1) + BS - 1) / BS;
                            const int64_t stride = n_x > n_r ? n_x : n_r;
                            const int64_t tot = bwd_jobs(rs, G, n_r, n_x);
                            std::vector<int> seen((size_t)G * Bt * stride, 0);
                            int64_t prev = -1;
                            int64_t prev_tok = -1;
                            for (int64_t L = 0; L < tot; ++L) {
                                const BwdJob j = kind == 0 ? bwd_job(L, rs, G, n_r, DkdvSplit{T, BS, n_r, R})
                                                           : bwd_job(L, rs, G, n_r, DqSplit{n_r, n_x});
                                const int64_t lim = j.g == s0 ? n_x : n_r;
                                if (j.g < 0 || j.g >= G || j.b < 0 || j.b >= Bt || j.j < 0 || j.j >= lim) {
                                    fail("out of range", T, R, Bt, G, s0, kind, (long)L);
                                    continue;
                                }
                                seen[((size_t)j.g * Bt + j.b) * stride + j.j]++;
                                const int Rg = j.g == s0 ? R + 1 : R;
                                if (kind == 0) {
                                    const int64_t w = ((int64_t)T - j.j * BS) * Rg;   // rows from the tile's first key on
                                    if (prev >= 0 && w > prev) fail("dK/dV work increases", T, R, Bt, G, s0, kind, (long)L);
                                    prev = w;
                                } else {
                                    const int64_t qt = (lim - 1 - j.j);
                                    int64_t tok = (qt * BS + BS - 1) / Rg;
                                    if (tok > T - 1) tok = T - 1;
                                    if (prev_tok >= 0 && tok > prev_tok + BS) fail("dQ end token increases", T, R, Bt, G, s0, kind, (long)L);
                                    prev_tok = tok;
                                }
                            }
                            for (int g = 0; g < G; ++g)
                                for (int b = 0; b < Bt; ++b) {
                                    const int64_t lim = g == s0 ? n_x : n_r;
                                    for (int64_t jj = 0; jj < stride; ++jj)
                                        if (seen[((size_t)g * Bt + b) * stride + jj] != (jj < lim ? 1 : 0))
                                            fail("job not issued exactly once", T, R, Bt, G, s0, kind, (long)jj);
                                }
                        }
                    }
    if (bad) std::printf("FAIL %d\n", bad);
    else std::printf("OK\n");
    return bad != 0;
}
