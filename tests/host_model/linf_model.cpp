// linf_model.cpp -- test-only host build of the chessboard line step in
// exact_euclidean_distance_amd/csrc/linf_rmq.h: the same functions the
// chessboard kernels run (build_block, build_level, answer_run), in the same
// order, with plain arrays in place of LDS.  Not part of the library.
#include <stdint.h>

#include <vector>

#include "../../exact_euclidean_distance_amd/csrc/linf_rmq.h"

// g[j] for one line of L positions (-1: no source, else 0 .. 65534); writes
// h[q] and the attaining source j[q] (the line must hold a source).  Returns
// 0, or -1 for bad arguments.
extern "C" int model_linf_line(const int32_t* g, int L, int32_t* h, int32_t* jout) {
    if (L < 1 || L > 65535) return -1;
    std::vector<uint16_t> gs(edt::rmq_g_halves(L), 0);
    bool any = false;
    for (int j = 0; j < L; ++j) {
        if (g[j] > 65534) return -1;
        gs[edt::rmq_gi(j)] = g[j] < 0 ? edt::kRmqNoG : (uint16_t)g[j];
        any = any || g[j] >= 0;
    }
    if (!any) return -1;
    std::vector<uint32_t> words(edt::rmq_words(L));
    edt::RmqLine line(gs.data(), words.data(), L);
    for (int b = 0; b < line.nb; ++b) line.build_block(b);
    for (int k = 1; k < edt::rmq_levels(line.nb); ++k)
        for (int i = 0; i + (1 << k) <= line.nb; ++i) line.build_level(k, i);
    const uint32_t kall = line.line_min();
    if (kall == edt::kRmqNone) return -1;
    for (int q0 = 0; q0 < L; q0 += edt::kRmqBlock) {
        const int n = q0 + edt::kRmqBlock < L ? edt::kRmqBlock : L - q0;
        int hs[edt::kRmqBlock], js[edt::kRmqBlock];
        line.answer_run(q0, n, kall, hs, js);
        for (int t = 0; t < n; ++t) {
            h[q0 + t] = hs[t];
            jout[q0 + t] = js[t];
        }
    }
    return 0;
}
