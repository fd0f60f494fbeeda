// Host-side sizing of the prefill segment plan and of the backward workspace.
// Products saturate at SIZE_MAX: a shape whose buffers cannot exist reports a
// workspace of SIZE_MAX, which no caller can provide, instead of a wrapped
// small size.
#include <cstdint>
#include <initializer_list>

#include "kernels.h"

namespace liger {

namespace {

size_t sat_mul(std::initializer_list<size_t> fs) {
    size_t n = 1;
    for (const size_t f : fs)
        if (__builtin_mul_overflow(n, f, &n)) return SIZE_MAX;
    return n;
}

size_t sat_add(std::initializer_list<size_t> xs) {
    size_t n = 0;
    for (const size_t x : xs)
        if (__builtin_add_overflow(n, x, &n)) return SIZE_MAX;
    return n;
}

}  // namespace

PrefillPlan make_prefill_plan(int64_t B, int64_t T, int H_kv, int d, bool bf16, int64_t chunks_per_segment) {
    PrefillPlan pl;
    pl.n_chunks = (T + kChunk - 1) / kChunk;
    int64_t cps = chunks_per_segment;
    if (cps <= 0) {
        // One output workgroup per compute unit (each keeps its running state
        // resident in LDS when it fits, which beats two smaller ones per unit).
        const int64_t target = 256;
        const int64_t heads = B * H_kv;
        int64_t want_seg = (target + heads - 1) / heads;
        if (want_seg < 1) want_seg = 1;
        cps = (pl.n_chunks + want_seg - 1) / want_seg;
        if (cps < 2) cps = 2;
    }
    if (cps > pl.n_chunks) cps = pl.n_chunks;
    pl.cps = cps;
    pl.n_seg = (pl.n_chunks + cps - 1) / cps;
    pl.carry_floats = size_t(d) * d + d;
    pl.state_offset = sat_mul({size_t(B), size_t(H_kv), size_t(pl.n_seg - 1), pl.carry_floats});
    const size_t slots = sat_mul({size_t(B), size_t(H_kv), size_t(pl.n_seg), size_t(d) * d});
    // fp32 at d = 128: the output kernel also keeps each chunk's state operand
    // in global memory (same size as the state slots)
    // and, for a continuation, the 64 tokens before it as contiguous K and V
    // rows per (b, kv head) (the window halo of the first chunk)
    pl.op_offset = sat_add({pl.state_offset, slots});
    const bool hg = !bf16 && d == 128;
    const size_t ops = hg ? slots : 0;
    pl.halo_offset = sat_add({pl.op_offset, ops});
    const size_t halo = hg ? sat_mul({size_t(B), size_t(H_kv), 2 * 64, size_t(d)}) : 0;
    pl.workspace_bytes = sat_mul({sat_add({pl.halo_offset, halo}), sizeof(float)});
    return pl;
}

size_t backward_workspace_bytes(int64_t B, int64_t T, int H_kv, int H_q, int d) {
    if (T <= 0) return 0;
    const int64_t n = (T + 63) / 64;
    const size_t rec = size_t(d) * d + d;
    const size_t floats = sat_add({sat_mul({2, size_t(B), size_t(H_kv), size_t(n - 1), rec}),
                                   sat_mul({size_t(B), size_t(H_kv), size_t(T), size_t(d)}),
                                   sat_mul({size_t(B), size_t(H_kv), size_t(n), size_t(d)}),
                                   sat_mul({size_t(B), size_t(T), size_t(H_q), 2})});
    return sat_mul({floats, sizeof(float)});
}

}  // namespace liger
