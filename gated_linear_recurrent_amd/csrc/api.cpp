// C ABI of the Liger Attention library: argument validation, workspace
// sizing, launch configuration and HIP error mapping. Every check runs before
// the first HIP call, so an invalid call launches nothing.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdint>
#include <cstdio>
#include <initializer_list>
#include <mutex>
#include <string>

#include "kernels.h"
#include "liger_attn.h"

namespace {

thread_local std::string g_last_error;

liger_status fail(liger_status st, const std::string& msg) {
    g_last_error = msg;
    return st;
}

liger_status ok() {
    g_last_error.clear();
    return LIGER_OK;
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// Shared shape checks. `need_T` is false for decode (T is ignored there).
liger_status check_shape(const liger_shape* s, bool need_T) {
    if (!s) return fail(LIGER_E_INVALID_ARG, "shape is NULL");
    if (s->B < 1 || s->B > 65535) return fail(LIGER_E_INVALID_ARG, "B must be in 1..65535");
    if (need_T && (s->T < 1 || s->T > (int64_t(1) << 31)))
        return fail(LIGER_E_INVALID_ARG, "T must be in 1..2^31");
    if (s->H_kv < 1 || s->H_kv > 65535) return fail(LIGER_E_INVALID_ARG, "H_kv must be in 1..65535");
    if (s->H_q < 1 || s->H_q % s->H_kv != 0) return fail(LIGER_E_INVALID_ARG, "H_q must be a positive multiple of H_kv");
    if (s->dtype != LIGER_F32 && s->dtype != LIGER_BF16) return fail(LIGER_E_INVALID_ARG, "dtype must be LIGER_F32 or LIGER_BF16");
    if (s->d < 1) return fail(LIGER_E_INVALID_ARG, "d must be positive");
    if (s->d != 64 && s->d != 128) return fail(LIGER_E_UNSUPPORTED, "d must be 64 or 128");
    return LIGER_OK;
}

liger_status check_common(int32_t gate_mode, float alpha) {
    if (gate_mode != LIGER_GATE_SCALAR_MEAN && gate_mode != LIGER_GATE_VECTOR_AVGPOOL4)
        return fail(LIGER_E_INVALID_ARG, "gate_mode must be LIGER_GATE_SCALAR_MEAN or LIGER_GATE_VECTOR_AVGPOOL4");
    if (!(alpha >= 0.0f && alpha <= 1.0f)) return fail(LIGER_E_INVALID_ARG, "alpha must be in [0, 1]");
    return LIGER_OK;
}

liger_status check_ptr(const void* p, const char* name) {
    if (!p) return fail(LIGER_E_INVALID_ARG, std::string(name) + " is NULL");
    if (!aligned16(p)) return fail(LIGER_E_INVALID_ARG, std::string(name) + " is not 16-byte aligned");
    return LIGER_OK;
}

// Bytes of a [B, T, heads, d] tensor of `elem`-byte elements, saturating at
// SIZE_MAX (a size that large cannot be a real buffer).
size_t tensor_bytes(int64_t B, int64_t T, int64_t heads, int64_t d, size_t elem) {
    size_t n = elem;
    for (const int64_t f : {B, T, heads, d}) {
        if (__builtin_mul_overflow(n, static_cast<size_t>(f), &n)) return SIZE_MAX;
    }
    return n;
}

// True when the byte ranges [a, a + na) and [b, b + nb) share a byte.
bool overlaps(const void* a, size_t na, const void* b, size_t nb) {
    if (!a || !b || na == 0 || nb == 0) return false;  // absent optional buffer
    const uintptr_t x = reinterpret_cast<uintptr_t>(a), y = reinterpret_cast<uintptr_t>(b);
    return x < y ? y - x < na : x - y < nb;
}

// A shape whose buffers could not exist: some byte count saturated.
liger_status check_sizes(std::initializer_list<size_t> sizes) {
    for (const size_t n : sizes)
        if (n == SIZE_MAX) return fail(LIGER_E_INVALID_ARG, "shape too large: a buffer size overflows");
    return LIGER_OK;
}

struct Span {
    const void* p;
    size_t n;
    const char* name;
};

// Every output span must be disjoint from every input span and from the
// other outputs.
liger_status check_disjoint(std::initializer_list<Span> outs, std::initializer_list<Span> ins) {
    for (auto o = outs.begin(); o != outs.end(); ++o) {
        for (const Span& i : ins)
            if (overlaps(o->p, o->n, i.p, i.n))
                return fail(LIGER_E_INVALID_ARG, std::string(o->name) + " must not overlap " + i.name);
        for (auto o2 = o + 1; o2 != outs.end(); ++o2)
            if (overlaps(o->p, o->n, o2->p, o2->n))
                return fail(LIGER_E_INVALID_ARG, std::string(o->name) + " must not overlap " + o2->name);
    }
    return LIGER_OK;
}

liger_status map_hip(hipError_t e, const char* what) {
    if (e == hipSuccess) return ok();
    return fail(LIGER_E_HIP, std::string(what) + ": " + hipGetErrorString(e));
}

#define LIGER_TRY(expr)                    \
    do {                                   \
        liger_status st_ = (expr);         \
        if (st_ != LIGER_OK) return st_;   \
    } while (0)

// Sink tokens: NULL means none; otherwise 1..16 tokens with aligned k and v.
liger_status check_sinks(const liger_sinks* sk) {
    if (!sk) return ok();
    if (sk->n < 1 || sk->n > 16) return fail(LIGER_E_INVALID_ARG, "sinks->n must be in 1..16");
    LIGER_TRY(check_ptr(sk->k, "sinks->k"));
    LIGER_TRY(check_ptr(sk->v, "sinks->v"));
    return ok();
}

}  // namespace

// Scratch memory of liger_attn_prefill_noalloc (the prefill workspace: carried
// states and running-state slots), one copy on every GPU the library runs on,
// held until the process ends. Host code never uses this name as an address:
// it uses the per-device address from hipGetSymbolAddress below.
constexpr size_t kScratchBytes = size_t(32) << 20;
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

namespace {

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

// Device address of `scratch` on the current device, looked up once per
// device (with that device current) and kept.
liger_status scratch_address(void** out) {
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return map_hip(e, "hipGetDevice");
    if (dev < 0 || dev >= kMaxDevices) return fail(LIGER_E_UNSUPPORTED, "device index beyond the scratch table");
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {
        void* p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return map_hip(e, "hipGetSymbolAddress(scratch)");
        if (!p) return fail(LIGER_E_HIP, "hipGetSymbolAddress(scratch) returned NULL");
        g_scratch_ptr[dev] = p;
    }
    *out = g_scratch_ptr[dev];
    return ok();
}

}  // namespace

extern "C" {

const char* liger_last_error(void) { return g_last_error.c_str(); }

size_t liger_attn_prefill_workspace_size_ex(const liger_shape* shape, int32_t chunks_per_segment) {
    if (check_shape(shape, true) != LIGER_OK || chunks_per_segment < 0) return 0;
    const liger::PrefillPlan pl = liger::make_prefill_plan(shape->B, shape->T, shape->H_kv, shape->d,
                                                           shape->dtype == LIGER_BF16, chunks_per_segment);
    return pl.workspace_bytes == SIZE_MAX ? 0 : pl.workspace_bytes;
}

size_t liger_attn_prefill_workspace_size(const liger_shape* shape) {
    return liger_attn_prefill_workspace_size_ex(shape, 0);
}

}  // extern "C"

namespace {

// Checks of a prefill call that do not involve the workspace; fills `a`
// (everything but a.workspace).
liger_status prefill_validate(const void* q, const void* k, const void* v, const liger_sinks* sinks,
                              int32_t gate_mode, int32_t window, float alpha, const liger_shape* shape, void* o,
                              float* S_T, int32_t chunks_per_segment, int32_t stage_mask, void* stream,
                              liger::PrefillArgs& a) {
    if (stage_mask < 1 || stage_mask > 7) return fail(LIGER_E_INVALID_ARG, "stage_mask must be in 1..7");
    LIGER_TRY(check_sinks(sinks));
    LIGER_TRY(check_shape(shape, true));
    LIGER_TRY(check_common(gate_mode, alpha));
    if (window < 1 || window > 64) return fail(LIGER_E_INVALID_ARG, "window must be in 1..64");
    if (chunks_per_segment < 0) return fail(LIGER_E_INVALID_ARG, "chunks_per_segment must be >= 0");
    LIGER_TRY(check_ptr(q, "q"));
    LIGER_TRY(check_ptr(k, "k"));
    LIGER_TRY(check_ptr(v, "v"));
    LIGER_TRY(check_ptr(o, "o"));
    LIGER_TRY(check_ptr(S_T, "S_T"));
    const size_t es = shape->dtype == LIGER_BF16 ? 2 : 4;
    const size_t qb = tensor_bytes(shape->B, shape->T, shape->H_q, shape->d, es);
    const size_t kb = tensor_bytes(shape->B, shape->T, shape->H_kv, shape->d, es);
    const size_t sb = tensor_bytes(shape->B, shape->H_kv, shape->d, shape->d, 4);
    const size_t skb = sinks ? tensor_bytes(shape->H_kv, sinks->n, 1, shape->d, es) : 0;
    LIGER_TRY(check_sizes({qb, kb, sb, skb}));
    LIGER_TRY(check_disjoint({{o, qb, "o"}, {S_T, sb, "S_T"}},
                             {{q, qb, "q"}, {k, kb, "k"}, {v, kb, "v"},
                              {sinks ? sinks->k : nullptr, skb, "sinks->k"},
                              {sinks ? sinks->v : nullptr, skb, "sinks->v"}}));
    a.q = q;
    a.k = k;
    a.v = v;
    a.o = o;
    a.S_T = S_T;
    a.workspace = nullptr;
    a.B = shape->B;
    a.T = shape->T;
    a.H_kv = shape->H_kv;
    a.n_rep = shape->H_q / shape->H_kv;
    a.d = shape->d;
    a.window = window;
    a.gate = gate_mode;
    a.bf16 = shape->dtype == LIGER_BF16;
    a.alpha = alpha;
    a.plan = liger::make_prefill_plan(shape->B, shape->T, shape->H_kv, shape->d, shape->dtype == LIGER_BF16,
                                      chunks_per_segment);
    LIGER_TRY(check_sizes({a.plan.workspace_bytes}));
    a.stage_mask = stage_mask;
    a.stream = stream;
    if (sinks) {
        a.sink_k = sinks->k;
        a.sink_v = sinks->v;
        a.n_sink = sinks->n;
    }
    return LIGER_OK;
}

liger_status prefill_impl(const void* q, const void* k, const void* v, const liger_sinks* sinks, int32_t gate_mode,
                          int32_t window, float alpha, const liger_shape* shape, void* o, float* S_T,
                          void* workspace, size_t workspace_bytes, int32_t chunks_per_segment, int32_t stage_mask,
                          void* stream) {
    liger::PrefillArgs a;
    LIGER_TRY(prefill_validate(q, k, v, sinks, gate_mode, window, alpha, shape, o, S_T, chunks_per_segment,
                               stage_mask, stream, a));
    const liger::PrefillPlan& pl = a.plan;
    if (pl.workspace_bytes > 0) {
        if (!workspace) return fail(LIGER_E_WORKSPACE, "workspace is NULL but " + std::to_string(pl.workspace_bytes) + " bytes are needed");
        if (!aligned16(workspace)) return fail(LIGER_E_INVALID_ARG, "workspace is not 16-byte aligned");
        if (workspace_bytes < pl.workspace_bytes)
            return fail(LIGER_E_WORKSPACE, "workspace too small: " + std::to_string(workspace_bytes) + " < " +
                                               std::to_string(pl.workspace_bytes) + " bytes");
        const size_t es = shape->dtype == LIGER_BF16 ? 2 : 4;
        const size_t qb = tensor_bytes(shape->B, shape->T, shape->H_q, shape->d, es);
        const size_t kb = tensor_bytes(shape->B, shape->T, shape->H_kv, shape->d, es);
        const size_t sb = tensor_bytes(shape->B, shape->H_kv, shape->d, shape->d, 4);
        const size_t skb = sinks ? tensor_bytes(shape->H_kv, sinks->n, 1, shape->d, es) : 0;
        LIGER_TRY(check_disjoint({{workspace, pl.workspace_bytes, "workspace"}},
                                 {{q, qb, "q"}, {k, kb, "k"}, {v, kb, "v"}, {o, qb, "o"}, {S_T, sb, "S_T"},
                                  {sinks ? sinks->k : nullptr, skb, "sinks->k"},
                                  {sinks ? sinks->v : nullptr, skb, "sinks->v"}}));
    }
    a.workspace = static_cast<float*>(workspace);
    return map_hip(liger::launch_prefill(a), "prefill launch");
}

}  // namespace

extern "C" {

liger_status liger_attn_prefill_stages(const void* q, const void* k, const void* v, int32_t gate_mode,
                                       int32_t window, float alpha, const liger_shape* shape, void* o,
                                       float* S_T, void* workspace, size_t workspace_bytes,
                                       int32_t chunks_per_segment, int32_t stage_mask, void* stream) {
    return prefill_impl(q, k, v, nullptr, gate_mode, window, alpha, shape, o, S_T, workspace, workspace_bytes,
                        chunks_per_segment, stage_mask, stream);
}

liger_status liger_attn_prefill_sinks(const void* q, const void* k, const void* v, const liger_sinks* sinks,
                                      int32_t gate_mode, int32_t window, float alpha, const liger_shape* shape,
                                      void* o, float* S_T, void* workspace, size_t workspace_bytes, void* stream) {
    if (!sinks) return fail(LIGER_E_INVALID_ARG, "sinks is NULL");
    return prefill_impl(q, k, v, sinks, gate_mode, window, alpha, shape, o, S_T, workspace, workspace_bytes, 0, 7,
                        stream);
}

liger_status liger_attn_prefill_ex(const void* q, const void* k, const void* v, int32_t gate_mode,
                                   int32_t window, float alpha, const liger_shape* shape, void* o,
                                   float* S_T, void* workspace, size_t workspace_bytes,
                                   int32_t chunks_per_segment, void* stream) {
    return liger_attn_prefill_stages(q, k, v, gate_mode, window, alpha, shape, o, S_T, workspace,
                                     workspace_bytes, chunks_per_segment, 7, stream);
}

liger_status liger_attn_prefill(const void* q, const void* k, const void* v, int32_t gate_mode, int32_t window,
                                float alpha, const liger_shape* shape, void* o, float* S_T, void* workspace,
                                size_t workspace_bytes, void* stream) {
    return liger_attn_prefill_ex(q, k, v, gate_mode, window, alpha, shape, o, S_T, workspace, workspace_bytes, 0,
                                 stream);
}

size_t liger_attn_prefill_noalloc_max_workspace(void) { return kScratchBytes; }

liger_status liger_attn_prefill_noalloc(const void* q, const void* k, const void* v, int32_t gate_mode,
                                        int32_t window, float alpha, const liger_shape* shape, void* o, float* S_T,
                                        void* stream) {
    liger::PrefillArgs a;
    LIGER_TRY(prefill_validate(q, k, v, nullptr, gate_mode, window, alpha, shape, o, S_T, 0, 7, stream, a));
    if (a.plan.workspace_bytes > kScratchBytes)
        return fail(LIGER_E_WORKSPACE, "shape needs " + std::to_string(a.plan.workspace_bytes) +
                                           " bytes of scratch; liger_attn_prefill_noalloc holds " +
                                           std::to_string(kScratchBytes) + " (use liger_attn_prefill with a workspace)");
    void* ws = nullptr;
    LIGER_TRY(scratch_address(&ws));
    a.workspace = static_cast<float*>(ws);
    return map_hip(liger::launch_prefill(a), "prefill launch");
}

}  // extern "C"

namespace {

liger_status continue_impl(const void* q, const void* k, const void* v, const float* S0,
                           const liger_kv_ring* kv_ring, const liger_sinks* sinks, int32_t gate_mode, float alpha,
                           const liger_shape* shape, void* o, float* S_T, void* workspace, size_t workspace_bytes,
                           void* stream) {
    LIGER_TRY(check_shape(shape, true));
    LIGER_TRY(check_sinks(sinks));
    LIGER_TRY(check_common(gate_mode, alpha));
    if (!kv_ring) return fail(LIGER_E_INVALID_ARG, "kv_ring is NULL");
    const int32_t window = kv_ring->window;
    if (window < 1 || window > 64) return fail(LIGER_E_INVALID_ARG, "ring window must be in 1..64");
    LIGER_TRY(check_ptr(q, "q"));
    LIGER_TRY(check_ptr(k, "k"));
    LIGER_TRY(check_ptr(v, "v"));
    LIGER_TRY(check_ptr(S0, "S0"));
    LIGER_TRY(check_ptr(o, "o"));
    LIGER_TRY(check_ptr(S_T, "S_T"));
    LIGER_TRY(check_ptr(kv_ring->k, "kv_ring->k"));
    LIGER_TRY(check_ptr(kv_ring->v, "kv_ring->v"));
    if (!kv_ring->pos) return fail(LIGER_E_INVALID_ARG, "kv_ring->pos is NULL");
    if (!kv_ring->sync) return fail(LIGER_E_INVALID_ARG, "kv_ring->sync is NULL");
    const size_t es = shape->dtype == LIGER_BF16 ? 2 : 4;
    const size_t qb = tensor_bytes(shape->B, shape->T, shape->H_q, shape->d, es);
    const size_t kb = tensor_bytes(shape->B, shape->T, shape->H_kv, shape->d, es);
    const size_t sb = tensor_bytes(shape->B, shape->H_kv, shape->d, shape->d, 4);
    const size_t rb = tensor_bytes(shape->B, shape->H_kv, window, shape->d, es);
    const size_t pb = tensor_bytes(shape->B, 1, 1, 1, 8);
    const size_t cb = tensor_bytes(shape->B, 1, 1, 1, 4);
    const size_t skb = sinks ? tensor_bytes(shape->H_kv, sinks->n, 1, shape->d, es) : 0;
    LIGER_TRY(check_sizes({qb, kb, sb, rb, pb, cb, skb}));
    // written: o, S_T and the ring (k, v, pos, sync are updated in place)
    LIGER_TRY(check_disjoint({{o, qb, "o"}, {S_T, sb, "S_T"}, {kv_ring->k, rb, "kv_ring->k"},
                              {kv_ring->v, rb, "kv_ring->v"}, {kv_ring->pos, pb, "kv_ring->pos"},
                              {kv_ring->sync, cb, "kv_ring->sync"}},
                             {{q, qb, "q"}, {k, kb, "k"}, {v, kb, "v"}, {S0, sb, "S0"},
                              {sinks ? sinks->k : nullptr, skb, "sinks->k"},
                              {sinks ? sinks->v : nullptr, skb, "sinks->v"}}));
    const liger::PrefillPlan pl = liger::make_prefill_plan(shape->B, shape->T, shape->H_kv, shape->d,
                                                           shape->dtype == LIGER_BF16, 0);
    LIGER_TRY(check_sizes({pl.workspace_bytes}));
    if (pl.workspace_bytes > 0) {
        if (!workspace) return fail(LIGER_E_WORKSPACE, "workspace is NULL but " + std::to_string(pl.workspace_bytes) + " bytes are needed");
        if (!aligned16(workspace)) return fail(LIGER_E_INVALID_ARG, "workspace is not 16-byte aligned");
        if (workspace_bytes < pl.workspace_bytes)
            return fail(LIGER_E_WORKSPACE, "workspace too small: " + std::to_string(workspace_bytes) + " < " +
                                               std::to_string(pl.workspace_bytes) + " bytes");
        LIGER_TRY(check_disjoint({{workspace, pl.workspace_bytes, "workspace"}},
                                 {{q, qb, "q"}, {k, kb, "k"}, {v, kb, "v"}, {S0, sb, "S0"}, {o, qb, "o"},
                                  {S_T, sb, "S_T"}, {kv_ring->k, rb, "kv_ring->k"}, {kv_ring->v, rb, "kv_ring->v"},
                                  {kv_ring->pos, pb, "kv_ring->pos"}, {kv_ring->sync, cb, "kv_ring->sync"},
                                  {sinks ? sinks->k : nullptr, skb, "sinks->k"},
                                  {sinks ? sinks->v : nullptr, skb, "sinks->v"}}));
    }
    liger::PrefillArgs a;
    a.q = q;
    a.k = k;
    a.v = v;
    a.o = o;
    a.S_T = S_T;
    a.workspace = static_cast<float*>(workspace);
    a.B = shape->B;
    a.T = shape->T;
    a.H_kv = shape->H_kv;
    a.n_rep = shape->H_q / shape->H_kv;
    a.d = shape->d;
    a.window = window;
    a.gate = gate_mode;
    a.bf16 = shape->dtype == LIGER_BF16;
    a.alpha = alpha;
    a.plan = pl;
    a.stage_mask = 7;
    a.stream = stream;
    a.S0 = S0;
    a.ring_k = kv_ring->k;
    a.ring_v = kv_ring->v;
    a.pos = kv_ring->pos;
    if (sinks) {
        a.sink_k = sinks->k;
        a.sink_v = sinks->v;
        a.n_sink = sinks->n;
    }
    LIGER_TRY(map_hip(liger::launch_prefill(a), "prefill continuation launch"));
    liger::RingFillArgs r;
    r.k = k;
    r.v = v;
    r.ring_k = kv_ring->k;
    r.ring_v = kv_ring->v;
    r.pos = kv_ring->pos;
    r.sync = kv_ring->sync;
    r.B = shape->B;
    r.T = shape->T;
    r.H_kv = shape->H_kv;
    r.d = shape->d;
    r.window = window;
    r.bf16 = shape->dtype == LIGER_BF16;
    r.stream = stream;
    return map_hip(liger::launch_ring_append(r), "ring append launch");
}

}  // namespace

extern "C" {

liger_status liger_attn_prefill_continue(const void* q, const void* k, const void* v, const float* S0,
                                        const liger_kv_ring* kv_ring, int32_t gate_mode, float alpha,
                                        const liger_shape* shape, void* o, float* S_T, void* workspace,
                                        size_t workspace_bytes, void* stream) {
    return continue_impl(q, k, v, S0, kv_ring, nullptr, gate_mode, alpha, shape, o, S_T, workspace, workspace_bytes,
                         stream);
}

liger_status liger_attn_prefill_continue_sinks(const void* q, const void* k, const void* v, const float* S0,
                                              const liger_kv_ring* kv_ring, const liger_sinks* sinks,
                                              int32_t gate_mode, float alpha, const liger_shape* shape, void* o,
                                              float* S_T, void* workspace, size_t workspace_bytes, void* stream) {
    if (!sinks) return fail(LIGER_E_INVALID_ARG, "sinks is NULL");
    return continue_impl(q, k, v, S0, kv_ring, sinks, gate_mode, alpha, shape, o, S_T, workspace, workspace_bytes,
                         stream);
}

}  // extern "C"

namespace {

liger_status decode_impl(const void* q, const void* k, const void* v, float* S, const liger_kv_ring* kv_ring,
                         const liger_sinks* sinks, int32_t gate_mode, float alpha, const liger_shape* shape, void* o,
                         void* stream) {
    LIGER_TRY(check_shape(shape, false));
    LIGER_TRY(check_sinks(sinks));
    LIGER_TRY(check_common(gate_mode, alpha));
    if (!kv_ring) return fail(LIGER_E_INVALID_ARG, "kv_ring is NULL");
    if (kv_ring->window < 1 || kv_ring->window > 64) return fail(LIGER_E_INVALID_ARG, "ring window must be in 1..64");
    const int n_rep = shape->H_q / shape->H_kv;
    if (n_rep != 1 && n_rep != 2 && n_rep != 4 && n_rep != 8)
        return fail(LIGER_E_UNSUPPORTED, "decode is built for H_q / H_kv in {1, 2, 4, 8}");
    LIGER_TRY(check_ptr(q, "q"));
    LIGER_TRY(check_ptr(k, "k"));
    LIGER_TRY(check_ptr(v, "v"));
    LIGER_TRY(check_ptr(S, "S"));
    LIGER_TRY(check_ptr(o, "o"));
    LIGER_TRY(check_ptr(kv_ring->k, "kv_ring->k"));
    LIGER_TRY(check_ptr(kv_ring->v, "kv_ring->v"));
    if (!kv_ring->pos) return fail(LIGER_E_INVALID_ARG, "kv_ring->pos is NULL");
    if (!kv_ring->sync) return fail(LIGER_E_INVALID_ARG, "kv_ring->sync is NULL");
    {
        // written: o, and the decode state S, ring k/v, pos, sync (updated in place)
        const size_t es = shape->dtype == LIGER_BF16 ? 2 : 4;
        const size_t qb = tensor_bytes(shape->B, 1, shape->H_q, shape->d, es);
        const size_t kb = tensor_bytes(shape->B, 1, shape->H_kv, shape->d, es);
        const size_t sb = tensor_bytes(shape->B, shape->H_kv, shape->d, shape->d, 4);
        const size_t rb = tensor_bytes(shape->B, shape->H_kv, kv_ring->window, shape->d, es);
        const size_t pb = tensor_bytes(shape->B, 1, 1, 1, 8);
        const size_t cb = tensor_bytes(shape->B, 1, 1, 1, 4);
        const size_t skb = sinks ? tensor_bytes(shape->H_kv, sinks->n, 1, shape->d, es) : 0;
        LIGER_TRY(check_sizes({qb, kb, sb, rb, pb, cb, skb}));
        LIGER_TRY(check_disjoint({{o, qb, "o"}, {S, sb, "S"}, {kv_ring->k, rb, "kv_ring->k"},
                                  {kv_ring->v, rb, "kv_ring->v"}, {kv_ring->pos, pb, "kv_ring->pos"},
                                  {kv_ring->sync, cb, "kv_ring->sync"}},
                                 {{q, qb, "q"}, {k, kb, "k"}, {v, kb, "v"},
                                  {sinks ? sinks->k : nullptr, skb, "sinks->k"},
                                  {sinks ? sinks->v : nullptr, skb, "sinks->v"}}));
    }
    liger::DecodeArgs a;
    a.q = q;
    a.k = k;
    a.v = v;
    a.S = S;
    a.ring_k = kv_ring->k;
    a.ring_v = kv_ring->v;
    a.pos = kv_ring->pos;
    a.sync = kv_ring->sync;
    a.o = o;
    a.N = shape->B;
    a.H_kv = shape->H_kv;
    a.n_rep = n_rep;
    a.d = shape->d;
    a.window = kv_ring->window;
    a.gate = gate_mode;
    a.bf16 = shape->dtype == LIGER_BF16;
    a.alpha = alpha;
    a.stream = stream;
    if (sinks) {
        a.sink_k = sinks->k;
        a.sink_v = sinks->v;
        a.n_sink = sinks->n;
    }
    return map_hip(liger::launch_decode_step(a), "decode launch");
}

}  // namespace

extern "C" {

liger_status liger_attn_decode_step(const void* q, const void* k, const void* v, float* S,
                                    const liger_kv_ring* kv_ring, int32_t gate_mode, float alpha,
                                    const liger_shape* shape, void* o, void* stream) {
    return decode_impl(q, k, v, S, kv_ring, nullptr, gate_mode, alpha, shape, o, stream);
}

liger_status liger_attn_decode_step_sinks(const void* q, const void* k, const void* v, float* S,
                                          const liger_kv_ring* kv_ring, const liger_sinks* sinks, int32_t gate_mode,
                                          float alpha, const liger_shape* shape, void* o, void* stream) {
    if (!sinks) return fail(LIGER_E_INVALID_ARG, "sinks is NULL");
    return decode_impl(q, k, v, S, kv_ring, sinks, gate_mode, alpha, shape, o, stream);
}

liger_status liger_attn_full_causal(const void* q, const void* k, const void* v, const liger_shape* shape,
                                    void* o, void* stream) {
    LIGER_TRY(check_shape(shape, true));
    if (shape->dtype != LIGER_BF16) return fail(LIGER_E_UNSUPPORTED, "full causal attention is built for bf16 only");
    const int n_rep = shape->H_q / shape->H_kv;
    if (n_rep != 1 && n_rep != 2 && n_rep != 4 && n_rep != 8)
        return fail(LIGER_E_UNSUPPORTED, "full causal attention is built for H_q / H_kv in {1, 2, 4, 8}");
    if ((shape->T + 63) / 64 > 2147483647LL) return fail(LIGER_E_INVALID_ARG, "T too large");
    LIGER_TRY(check_ptr(q, "q"));
    LIGER_TRY(check_ptr(k, "k"));
    LIGER_TRY(check_ptr(v, "v"));
    LIGER_TRY(check_ptr(o, "o"));
    {
        const size_t qb = tensor_bytes(shape->B, shape->T, shape->H_q, shape->d, 2);
        const size_t kb = tensor_bytes(shape->B, shape->T, shape->H_kv, shape->d, 2);
        LIGER_TRY(check_sizes({qb, kb}));
        LIGER_TRY(check_disjoint({{o, qb, "o"}}, {{q, qb, "q"}, {k, kb, "k"}, {v, kb, "v"}}));
    }
    liger::FullAttnArgs a;
    a.q = q;
    a.k = k;
    a.v = v;
    a.o = o;
    a.B = shape->B;
    a.T = shape->T;
    a.H_q = shape->H_q;
    a.H_kv = shape->H_kv;
    a.n_rep = n_rep;
    a.d = shape->d;
    a.stream = stream;
    return map_hip(liger::launch_full_attn(a), "full attention launch");
}

size_t liger_attn_prefill_backward_workspace_size(const liger_shape* shape) {
    if (check_shape(shape, true) != LIGER_OK) return 0;
    const size_t n = liger::backward_workspace_bytes(shape->B, shape->T, shape->H_kv, shape->H_q, shape->d);
    return n == SIZE_MAX ? 0 : n;
}

liger_status liger_attn_prefill_backward(const void* q, const void* k, const void* v, const void* dO,
                                         int32_t gate_mode, int32_t window, float alpha,
                                         const liger_shape* shape, float* dq, float* dk, float* dv,
                                         void* workspace, size_t workspace_bytes, void* stream) {
    LIGER_TRY(check_shape(shape, true));
    LIGER_TRY(check_common(gate_mode, alpha));
    if (shape->dtype != LIGER_BF16) return fail(LIGER_E_UNSUPPORTED, "the backward is built for bf16 inputs only");
    if (window < 1 || window > 64) return fail(LIGER_E_INVALID_ARG, "window must be in 1..64");
    LIGER_TRY(check_ptr(q, "q"));
    LIGER_TRY(check_ptr(k, "k"));
    LIGER_TRY(check_ptr(v, "v"));
    LIGER_TRY(check_ptr(dO, "dO"));
    LIGER_TRY(check_ptr(dq, "dq"));
    LIGER_TRY(check_ptr(dk, "dk"));
    LIGER_TRY(check_ptr(dv, "dv"));
    const size_t need = liger::backward_workspace_bytes(shape->B, shape->T, shape->H_kv, shape->H_q, shape->d);
    LIGER_TRY(check_sizes({need}));
    if (workspace_bytes < need) return fail(LIGER_E_WORKSPACE, "workspace smaller than liger_attn_prefill_backward_workspace_size");
    if (need > 0) LIGER_TRY(check_ptr(workspace, "workspace"));
    {
        const size_t qb = tensor_bytes(shape->B, shape->T, shape->H_q, shape->d, 2);
        const size_t kb = tensor_bytes(shape->B, shape->T, shape->H_kv, shape->d, 2);
        const size_t gqb = tensor_bytes(shape->B, shape->T, shape->H_q, shape->d, 4);
        const size_t gkb = tensor_bytes(shape->B, shape->T, shape->H_kv, shape->d, 4);
        LIGER_TRY(check_sizes({qb, kb, gqb, gkb}));
        LIGER_TRY(check_disjoint({{dq, gqb, "dq"}, {dk, gkb, "dk"}, {dv, gkb, "dv"}, {workspace, need, "workspace"}},
                                 {{q, qb, "q"}, {k, kb, "k"}, {v, kb, "v"}, {dO, qb, "dO"}}));
    }
    liger::BackwardArgs a;
    a.q = q;
    a.k = k;
    a.v = v;
    a.dO = dO;
    a.dq = dq;
    a.dk = dk;
    a.dv = dv;
    a.B = shape->B;
    a.T = shape->T;
    a.H_kv = shape->H_kv;
    a.n_rep = shape->H_q / shape->H_kv;
    a.d = shape->d;
    a.window = window;
    a.gate = gate_mode;
    a.alpha = alpha;
    a.workspace = static_cast<float*>(workspace);
    a.stream = stream;
    return map_hip(liger::launch_backward(a), "backward launch");
}

liger_status liger_kv_ring_fill(const void* k, const void* v, const liger_shape* shape,
                                const liger_kv_ring* kv_ring, void* stream) {
    LIGER_TRY(check_shape(shape, true));
    if (!kv_ring) return fail(LIGER_E_INVALID_ARG, "kv_ring is NULL");
    if (kv_ring->window < 1 || kv_ring->window > 64) return fail(LIGER_E_INVALID_ARG, "ring window must be in 1..64");
    LIGER_TRY(check_ptr(k, "k"));
    LIGER_TRY(check_ptr(v, "v"));
    LIGER_TRY(check_ptr(kv_ring->k, "kv_ring->k"));
    LIGER_TRY(check_ptr(kv_ring->v, "kv_ring->v"));
    if (!kv_ring->pos) return fail(LIGER_E_INVALID_ARG, "kv_ring->pos is NULL");
    if (!kv_ring->sync) return fail(LIGER_E_INVALID_ARG, "kv_ring->sync is NULL");
    {
        const size_t es = shape->dtype == LIGER_BF16 ? 2 : 4;
        const size_t kb = tensor_bytes(shape->B, shape->T, shape->H_kv, shape->d, es);
        const size_t rb = tensor_bytes(shape->B, shape->H_kv, kv_ring->window, shape->d, es);
        const size_t pb = tensor_bytes(shape->B, 1, 1, 1, 8);
        const size_t cb = tensor_bytes(shape->B, 1, 1, 1, 4);
        LIGER_TRY(check_sizes({kb, rb, pb, cb}));
        LIGER_TRY(check_disjoint({{kv_ring->k, rb, "kv_ring->k"}, {kv_ring->v, rb, "kv_ring->v"},
                                  {kv_ring->pos, pb, "kv_ring->pos"}, {kv_ring->sync, cb, "kv_ring->sync"}},
                                 {{k, kb, "k"}, {v, kb, "v"}}));
    }
    liger::RingFillArgs a;
    a.k = k;
    a.v = v;
    a.ring_k = kv_ring->k;
    a.ring_v = kv_ring->v;
    a.pos = kv_ring->pos;
    a.sync = kv_ring->sync;
    a.B = shape->B;
    a.T = shape->T;
    a.H_kv = shape->H_kv;
    a.d = shape->d;
    a.window = kv_ring->window;
    a.bf16 = shape->dtype == LIGER_BF16;
    a.stream = stream;
    return map_hip(liger::launch_ring_fill(a), "ring fill launch");
}

}  // extern "C"
