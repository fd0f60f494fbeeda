// Internal launch interface between the C ABI (api.cpp) and the HIP kernels.
// Arguments arrive here already validated; these functions only configure
// and enqueue kernels on the given stream.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace liger {

struct DecodeArgs {
    const void* q;
    const void* k;
    const void* v;
    float* S;
    void* ring_k;
    void* ring_v;
    int64_t* pos;
    uint32_t* sync;
    void* o;
    int64_t N;
    int H_kv;
    int n_rep;
    int d;
    int window;
    int gate;   // 0 scalar mean, 1 vector avg-pool-4
    bool bf16;
    float alpha;
    void* stream;
    // meta-memory sink tokens [H_kv, n_sink, d] (none when n_sink == 0)
    const void* sink_k = nullptr;
    const void* sink_v = nullptr;
    int n_sink = 0;
};

struct RingFillArgs {
    const void* k;
    const void* v;
    void* ring_k;
    void* ring_v;
    int64_t* pos;
    uint32_t* sync;
    int64_t B;
    int64_t T;
    int H_kv;
    int d;
    int window;
    bool bf16;
    void* stream;
};

// Full causal softmax attention (bf16). q, o: [B, T, H_q, d]; k, v: [B, T, H_kv, d].
struct FullAttnArgs {
    const void* q;
    const void* k;
    const void* v;
    void* o;
    int64_t B;
    int64_t T;
    int H_q;
    int H_kv;
    int n_rep;
    int d;
    int ngroups;  // B x (query-head groups); set by the launcher
    void* stream;
};

// Segment plan of the chunked prefill: chunks of 64 tokens grouped into
// n_seg segments of cps chunks (the last segment may be shorter).
// Workspace: carry records (state entering each segment but the first, plus
// the segment's total log2 decay), then one private d*d fp32 slot per output
// workgroup that holds the running state between chunks.
struct PrefillPlan {
    int64_t n_chunks;        // ceil(T / 64)
    int64_t cps;             // chunks per segment
    int64_t n_seg;           // ceil(n_chunks / cps)
    size_t carry_floats;     // floats per carry record: d*d + d
    size_t state_offset;     // floats before the state slots: B * H_kv * (n_seg - 1) * carry_floats
    size_t op_offset;        // floats before the state-operand slots (fp32, d = 128): state_offset + slots
    size_t halo_offset;      // floats before the halo rows (fp32, d = 128): op_offset + operand slots
    size_t workspace_bytes;  // (halo_offset + [fp32, d = 128] B * H_kv * 2 * 64 * d) * 4
};

struct PrefillArgs {
    const void* q;
    const void* k;
    const void* v;
    void* o;
    float* S_T;
    float* workspace;
    int64_t B;
    int64_t T;
    int H_kv;
    int n_rep;
    int d;
    int window;
    int gate;
    bool bf16;
    float alpha;
    PrefillPlan plan;
    int stage_mask;  // 1 segment states, 2 carry scan, 4 outputs
    void* stream;
    // continuation (all null for a prefill from a zero state): the state and
    // KV ring (window = `window`) after pos[b] tokens
    const float* S0 = nullptr;
    const void* ring_k = nullptr;
    const void* ring_v = nullptr;
    const int64_t* pos = nullptr;
    // meta-memory sink tokens [H_kv, n_sink, d] prepended to every window
    // (none when n_sink == 0)
    const void* sink_k = nullptr;
    const void* sink_v = nullptr;
    int n_sink = 0;
};

constexpr int kChunk = 64;

PrefillPlan make_prefill_plan(int64_t B, int64_t T, int H_kv, int d, bool bf16, int64_t chunks_per_segment);

hipError_t launch_decode_step(const DecodeArgs& a);
hipError_t launch_ring_fill(const RingFillArgs& a);
// Continuation: the last min(T, window) new tokens go to slots (pos + t) mod
// window, older slots keep their tokens, then pos += T.
hipError_t launch_ring_append(const RingFillArgs& a);
hipError_t launch_prefill(const PrefillArgs& a);
hipError_t launch_full_attn(const FullAttnArgs& a);
// Carry records [B, H_kv, n_seg - 1, d*d + d] (state, log2 row decay) are
// replaced in place by the running states R_s = 2^(lg_s) (.) R_{s-1} + L_s, R_{-1} = 0.
hipError_t launch_carry_scan(float* carry, int64_t n_seg, int H_kv, int64_t B, int d, void* stream);

// Backward of the prefill (bf16 inputs, float32 gradients).
struct BackwardArgs {
    const void* q;
    const void* k;
    const void* v;
    const void* dO;
    float* dq;
    float* dk;
    float* dv;
    int64_t B;
    int64_t T;
    int H_kv;
    int n_rep;
    int d;
    int window;
    int gate;
    float alpha;
    float* workspace;
    void* stream;
};
size_t backward_workspace_bytes(int64_t B, int64_t T, int H_kv, int H_q, int d);
hipError_t launch_backward(const BackwardArgs& a);

}  // namespace liger
