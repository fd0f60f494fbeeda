// Liger Attention chunked prefill for gfx950.
//
// Math (paper-notes page "Liger: Linearizing Large Language Models to Gated
// Recurrent Structures": unified gated linear recurrence; Liger Attention):
//   S_t = G_t (.) S_{t-1} + phi(k_t)^T v_t ,  o_t = alpha phi(q_t) S_t + (1-alpha) SWA_t
// evaluated in 64-token chunks ("right-multiplication" order, linear in T).
// Within a chunk with inclusive log2 cumulative gate b_i (b_i <= 0, relative
// to the chunk start) and the state S entering the chunk:
//   o_grm,i = sum_{j<=i} sum_c phiq_i[c] phik_j[c] 2^(b_i[c]-b_j[c]) v_j
//           + (phiq_i (.) 2^(b_i)) S
//   S_end   = diag(2^(b_last)) S + sum_j (phik_j (.) 2^(b_last - b_j))^T v_j
// Scalar gate: the decay 2^(b_i - b_j) is a per-(i, j) scalar applied to the
// MFMA result (always bounded by 1). Vector gate: the decay varies with the
// contracted channel, so it is split around a per-channel reference m (the
// cumulative gate at the chunk's middle token): query operand
// phiq (.) 2^(b_i - m), key operand phik (.) 2^(m - b_j), state operand
// diag(2^m) S. A channel whose factors could exceed 2^96 ("bad") is left out
// of the MFMA and added exactly in fp32 instead.
// The sliding window (w <= 64 keys, self included, scale 1/sqrt(d)) reuses
// the same K/V tiles: the current chunk plus the previous one.
//
// Three kernels (sequence parallelism over segments of `cps` chunks):
//   P1 segment_state_*_kernel: local end state L_s (from zero) and total log2
//                             decay of every segment but the last
//   P2 carry_scan_kernel    : S_in[s+1] = 2^(lg_s) (.) S_in[s] + L_s, in place
//   P3 prefill_output_kernel: per segment, walks its chunks from S_in[s],
//                             computes o, and (last segment) writes S_T
#include <type_traits>

#include "device_common.h"
#include "kernels.h"

namespace liger {

constexpr int kPThreads = 512;
constexpr int kPWaves = kPThreads / 64;
constexpr float kEmax2 = 96.0f;  // largest log2 factor admitted to the MFMA path

// The lane index as a value the compiler cannot move: code derived from it
// stays where it is written (a rare path inside a loop is not hoisted).
__device__ __forceinline__ int opaque_lane(int lane) {
    asm volatile("" : "+v"(lane));
    return lane;
}

// Thread index hidden from loop-invariant code motion: values derived from it
// are recomputed where they are used instead of being held in registers
// across the whole chunk loop.
__device__ __forceinline__ int ltid() {
    int t = static_cast<int>(threadIdx.x);
    asm volatile("" : "+v"(t));
    return t;
}

// ------------------------------------------------------------- LDS layout
template <typename T, int D, int GATE, bool FULL>
struct Layout {
    static constexpr int E = sizeof(T);
    static constexpr int PAD = 16 / E;
    static constexpr int DP = D + PAD;   // pitch of token-major [64][D] tiles
    static constexpr int JP = 64 + PAD;  // pitch of channel-major [D][64] tiles
    static constexpr int FP = D + 4;     // pitch of the fp32 gate-factor tile
    // fp32 at d = 128 ("global halo"): the output kernel keeps only the current
    // chunk's K/V in LDS; the previous chunk's keys and values (the window
    // halo) and the state operand are read from global memory.
    static constexpr bool HG = FULL && E == 4 && D == 128;
    static constexpr int NSLOT = FULL && !HG ? 2 : 1;
    static constexpr int KB_ELEMS = (64 * DP > D * JP) ? 64 * DP : D * JP;
    // bf16 keeps V token-major ([64][VP], rows 8 banks apart) and reads it with
    // transposing loads; fp32 stores V^T ([D][JP], keys at key_pos).
    static constexpr bool VNAT = (E == 2);
    static constexpr int VP = D + 16;
    static constexpr int V_ELEMS = VNAT ? 64 * VP : D * JP;

    static constexpr int SP = D + 4;     // pitch of the resident fp32 state [D][SP]

    static constexpr size_t K_OFF = 0;                                        // raw K [slot][64][DP]
    static constexpr size_t VT_OFF = K_OFF + size_t(NSLOT) * 64 * DP * E;     // V [slot][V_ELEMS]
    static constexpr size_t KB_OFF = VT_OFF + size_t(NSLOT) * V_ELEMS * E;    // K~ (state^T or intra)
    static constexpr size_t ST_OFF = KB_OFF + size_t(KB_ELEMS) * E;           // state region
    // small persistent arrays: kmax[64] kinv[64] b2s[64] b2e[64] dec[D] mref[D]
    // emref[D] blast[D] badlist[D] badmask[D/32] nbad, exact
    static constexpr size_t SMALL_WORDS = 64 * 4 + D * 5 + D / 32 + 4;
    static constexpr size_t F_BYTES = (FULL && GATE) ? size_t(64) * FP * 4 : 0;
    static constexpr size_t TMP_FLOATS = size_t(kPThreads) + 3 * D;
    // Output kernels keep the running state in LDS as fp32 S^T [D][SP] when
    // everything fits ("resident state"); otherwise the state region holds the
    // operand-type copy S'^T [D][DP] and the fp32 state lives in registers and
    // a per-workgroup global slot between chunks.
    static constexpr size_t S32_BYTES = size_t(D) * SP * 4;
    static constexpr size_t BUDGET = 160 * 1024;  // one output workgroup per compute unit
    static constexpr bool SLDS = FULL && !HG && (ST_OFF + S32_BYTES + F_BYTES + SMALL_WORDS * 4 <= BUDGET) &&
                                 (size_t(KB_ELEMS) * E >= TMP_FLOATS * 4);
    static constexpr size_t ST_BYTES = (!FULL || HG) ? 0 : SLDS ? S32_BYTES : size_t(D) * DP * E;
    static constexpr size_t F_OFF = ST_OFF + ST_BYTES;                        // fp32 [64][FP]
    static constexpr size_t TMP_OFF = F_OFF + F_BYTES;                        // gate-scan scratch
    // The scan scratch (part sums, raw references) shares a region that is
    // idle during the gate scan: K~ (resident state: K~ is written after the
    // scan), S'^T (other output kernels: free until the state phase), else
    // it has its own.
    static constexpr int TMP_WHERE = SLDS ? 1 : (FULL && ST_BYTES >= TMP_FLOATS * 4) ? 2 : 0;
    static constexpr size_t SMALL_OFF = TMP_WHERE ? TMP_OFF : TMP_OFF + TMP_FLOATS * 4;
    static constexpr size_t TOTAL = SMALL_OFF + SMALL_WORDS * 4;
    static_assert(TOTAL <= BUDGET, "LDS budget of a gfx950 workgroup exceeded");
};

template <typename T, int D, int GATE, bool FULL>
struct Smem {
    typedef Layout<T, D, GATE, FULL> L;
    T* K;      // [NSLOT][64][DP]
    T* Vt;     // [NSLOT][V_ELEMS]: [64][VP] (bf16) or [D][JP] (fp32)
    T* Kb;     // [D][JP] (K~ state, transposed) then [64][DP] (K~ intra)
    T* St;     // [D][DP] (no resident state)
    float* S32;   // [D][SP] resident fp32 state, S32[dv][dk] = S[dk][dv]
    float* F;  // [64][FP]
    float* part;  // [kPThreads]
    float* m2raw; // [D]
    float* bl2;   // [D]
    float* b0;    // [D]
    float* kmax;  // [64]
    float* kinv;  // [64]
    float* b2s;   // [64] scalar-gate cumulative log2 gate
    float* b2e;   // [64] scalar-gate log2 gate per token (the scan's input)
    float* dec;   // [D] 2^(b_last) per d_k row
    float* mref;  // [D] log2 reference per channel (0 for bad channels)
    float* emref; // [D] 2^mref
    float* blast; // [D] log2 decay of the whole chunk per channel
    int* badlist; // [D]
    uint32_t* badmask;  // [D/32]
    int* nbad;
    int* exact;  // scalar gate: this chunk's decay range needs the exact per-pair path

    __device__ explicit Smem(char* base) {
        K = reinterpret_cast<T*>(base + L::K_OFF);
        Vt = reinterpret_cast<T*>(base + L::VT_OFF);
        Kb = reinterpret_cast<T*>(base + L::KB_OFF);
        St = reinterpret_cast<T*>(base + L::ST_OFF);
        S32 = reinterpret_cast<float*>(base + L::ST_OFF);
        F = reinterpret_cast<float*>(base + L::F_OFF);
        float* tmp = reinterpret_cast<float*>(
            base + (L::TMP_WHERE == 1 ? L::KB_OFF : L::TMP_WHERE == 2 ? L::ST_OFF : L::TMP_OFF));
        part = tmp;
        m2raw = tmp + kPThreads;
        bl2 = m2raw + D;
        b0 = bl2 + D;
        float* sm = reinterpret_cast<float*>(base + L::SMALL_OFF);
        kmax = sm;
        kinv = sm + 64;
        b2s = sm + 128;
        b2e = sm + 192;
        dec = sm + 256;
        mref = dec + D;
        emref = mref + D;
        blast = emref + D;
        badlist = reinterpret_cast<int*>(blast + D);
        badmask = reinterpret_cast<uint32_t*>(badlist + D);
        nbad = reinterpret_cast<int*>(badmask + D / 32);
        exact = nbad + 1;
    }
};

struct PrefillParams {
    const void* q;
    const void* k;
    const void* v;
    void* o;
    float* S_T;
    float* carry;
    float* state_slots;
    float* op_slots;  // global halo: state operand [D][D] per output workgroup
    float* halo;      // global halo, continuation: K then V rows [64][D] per (b, kv head)
    int64_t T;
    int64_t n_chunks;
    int64_t cps;
    int64_t n_seg;
    int H_kv;
    int n_rep;
    int window;
    float alpha;
    // continuation: entering state [B, H_kv, d, d] and the KV ring
    // [B, H_kv, window, d] after pos[b] tokens (null for a zero state)
    const float* S0;
    const void* ring_k;
    const void* ring_v;
    const int64_t* pos;
    // meta-memory sink tokens [H_kv, n_sink, d] (output kernel, SINK = true)
    const void* sink_k;
    const void* sink_v;
    int n_sink;
    // global halo (fp32, d = 128) only: the output kernel computes the
    // segment-state records instead of outputs (no segment-state kernel is
    // built for that tile shape)
    int rec_mode;
};

// ------------------------------------------------------------ chunk loading
// K rows go to LDS as they are; V is written transposed (V^T[c][key_pos(j)]),
// two keys per 32-bit (bf16) or 64-bit (fp32) store so that the lanes of a
// wave write one contiguous row segment. Rows past the end are zero.
// The global loads (issue) and the LDS stores (commit) are separate steps so
// that other loads can be issued in between.
template <typename T, int D>
struct ChunkRegs {
    static constexpr int VPL = 16 / sizeof(T);
    static constexpr int PPR = D / VPL;                                  // 16-byte pieces per row
    static constexpr int NK = (64 * PPR + kPThreads - 1) / kPThreads;    // K pieces per thread
    static constexpr bool VNAT = sizeof(T) == 2;
    static constexpr int NV = VNAT ? 1 : (32 * PPR + kPThreads - 1) / kPThreads;  // V row pairs per thread (fp32)
    uint4 k[NK];
    uint4 v[VNAT ? NK : 1];  // bf16: V pieces, same mapping as K
    uint4 v0[NV], v1[NV];
};

template <typename T, int D>
__device__ __forceinline__ void load_chunk_issue(ChunkRegs<T, D>& cr, const T* kbase, const T* vbase,
                                                 int64_t row_stride, int64_t t0, int nvalid) {
    typedef ChunkRegs<T, D> CR;
    const int tid = ltid();
#pragma unroll
    for (int n = 0; n < CR::NK; ++n) {
        const int idx = tid + n * kPThreads;
        const int j = idx / CR::PPR;
        const int c0 = (idx % CR::PPR) * CR::VPL;
        cr.k[n] = make_uint4(0, 0, 0, 0);
        if (idx < 64 * CR::PPR && j < nvalid)
            cr.k[n] = *reinterpret_cast<const uint4*>(kbase + (t0 + j) * row_stride + c0);
    }
    if constexpr (CR::VNAT) {
#pragma unroll
        for (int n = 0; n < CR::NK; ++n) {
            const int idx = tid + n * kPThreads;
            const int j = idx / CR::PPR;
            const int c0 = (idx % CR::PPR) * CR::VPL;
            cr.v[n] = make_uint4(0, 0, 0, 0);
            if (idx < 64 * CR::PPR && j < nvalid)
                cr.v[n] = *reinterpret_cast<const uint4*>(vbase + (t0 + j) * row_stride + c0);
        }
        return;
    }
#pragma unroll
    for (int n = 0; n < CR::NV; ++n) {
        const int idx = tid + n * kPThreads;
        const int j0 = 2 * (idx & 31);
        const int c0 = (idx >> 5) * CR::VPL;
        cr.v0[n] = make_uint4(0, 0, 0, 0);
        cr.v1[n] = make_uint4(0, 0, 0, 0);
        if (idx < 32 * CR::PPR) {
            if (j0 < nvalid) cr.v0[n] = *reinterpret_cast<const uint4*>(vbase + (t0 + j0) * row_stride + c0);
            if (j0 + 1 < nvalid) cr.v1[n] = *reinterpret_cast<const uint4*>(vbase + (t0 + j0 + 1) * row_stride + c0);
        }
    }
}

// The 64 tokens before a continuation as a chunk: row j is token pos - 64 + j,
// read from ring slot (pos - 64 + j) mod window when it is among the npv
// (= min(pos, window)) tokens the ring holds, zero otherwise. Same register
// mapping as load_chunk_issue.
template <typename T, int D>
__device__ __forceinline__ void load_ring_issue(ChunkRegs<T, D>& cr, const T* rk, const T* rv, int64_t pos,
                                                int window, int npv) {
    typedef ChunkRegs<T, D> CR;
    const int tid = ltid();
    auto row_of = [&](int j) -> int64_t {  // ring row of chunk row j, or -1
        if (j < 64 - npv) return -1;
        return (pos - 64 + j) % window;  // pos - 64 + j >= pos - npv >= 0
    };
#pragma unroll
    for (int n = 0; n < CR::NK; ++n) {
        const int idx = tid + n * kPThreads;
        const int j = idx / CR::PPR;
        const int c0 = (idx % CR::PPR) * CR::VPL;
        cr.k[n] = make_uint4(0, 0, 0, 0);
        const int64_t rr = idx < 64 * CR::PPR ? row_of(j) : -1;
        if (rr >= 0) cr.k[n] = *reinterpret_cast<const uint4*>(rk + rr * D + c0);
        if constexpr (CR::VNAT) {
            cr.v[n] = make_uint4(0, 0, 0, 0);
            if (rr >= 0) cr.v[n] = *reinterpret_cast<const uint4*>(rv + rr * D + c0);
        }
    }
    if constexpr (!CR::VNAT) {
#pragma unroll
        for (int n = 0; n < CR::NV; ++n) {
            const int idx = tid + n * kPThreads;
            const int j0 = 2 * (idx & 31);
            const int c0 = (idx >> 5) * CR::VPL;
            cr.v0[n] = make_uint4(0, 0, 0, 0);
            cr.v1[n] = make_uint4(0, 0, 0, 0);
            if (idx < 32 * CR::PPR) {
                const int64_t r0 = row_of(j0), r1 = row_of(j0 + 1);
                if (r0 >= 0) cr.v0[n] = *reinterpret_cast<const uint4*>(rv + r0 * D + c0);
                if (r1 >= 0) cr.v1[n] = *reinterpret_cast<const uint4*>(rv + r1 * D + c0);
            }
        }
    }
}

template <typename T, int D, int GATE, bool FULL>
__device__ __forceinline__ void load_chunk_commit(const Smem<T, D, GATE, FULL>& sm, int slot, const ChunkRegs<T, D>& cr) {
    typedef Layout<T, D, GATE, FULL> L;
    typedef ChunkRegs<T, D> CR;
    T* Ks = sm.K + slot * 64 * L::DP;
    T* Vts = sm.Vt + slot * L::V_ELEMS;
    const int tid = ltid();
#pragma unroll
    for (int n = 0; n < CR::NK; ++n) {
        const int idx = tid + n * kPThreads;
        if (idx < 64 * CR::PPR)
            *reinterpret_cast<uint4*>(Ks + (idx / CR::PPR) * L::DP + (idx % CR::PPR) * CR::VPL) = cr.k[n];
    }
    if constexpr (CR::VNAT) {
#pragma unroll
        for (int n = 0; n < CR::NK; ++n) {
            const int idx = tid + n * kPThreads;
            if (idx < 64 * CR::PPR)
                *reinterpret_cast<uint4*>(Vts + (idx / CR::PPR) * L::VP + (idx % CR::PPR) * CR::VPL) = cr.v[n];
        }
        return;
    }
#pragma unroll
    for (int n = 0; n < CR::NV; ++n) {
        const int idx = tid + n * kPThreads;
        if (idx >= 32 * CR::PPR) continue;
        const int j0 = 2 * (idx & 31);
        const int c0 = (idx >> 5) * CR::VPL;
        const T* e0 = reinterpret_cast<const T*>(&cr.v0[n]);
        const T* e1 = reinterpret_cast<const T*>(&cr.v1[n]);
        T* dst = Vts + c0 * L::JP + key_pos(j0);
#pragma unroll
        for (int e = 0; e < CR::VPL; ++e) {
            if constexpr (sizeof(T) == 2) {
                *reinterpret_cast<uint32_t*>(dst + e * L::JP) =
                    static_cast<uint32_t>(e0[e]) | (static_cast<uint32_t>(e1[e]) << 16);
            } else {
                *reinterpret_cast<float2*>(dst + e * L::JP) = make_float2(e0[e], e1[e]);
            }
        }
    }
}

template <typename T, int D, int GATE, bool FULL>
__device__ __forceinline__ void load_chunk(const Smem<T, D, GATE, FULL>& sm, int slot,
                                           const T* kbase, const T* vbase, int64_t row_stride,
                                           int64_t t0, int nvalid) {
    ChunkRegs<T, D> cr;
    load_chunk_issue<T, D>(cr, kbase, vbase, row_stride, t0, nvalid);
    load_chunk_commit(sm, slot, cr);
}

template <typename T, int D, int GATE, bool FULL>
__device__ __forceinline__ void zero_slot(const Smem<T, D, GATE, FULL>& sm, int slot) {
    typedef Layout<T, D, GATE, FULL> L;
    uint32_t* kz = reinterpret_cast<uint32_t*>(sm.K + slot * 64 * L::DP);
    for (int i = ltid(); i < 64 * L::DP * int(sizeof(T)) / 4; i += kPThreads) kz[i] = 0u;
    uint32_t* vz = reinterpret_cast<uint32_t*>(sm.Vt + slot * L::V_ELEMS);
    for (int i = ltid(); i < L::V_ELEMS * int(sizeof(T)) / 4; i += kPThreads) vz[i] = 0u;
}

// ------------------------------------------------------- per-chunk gate work
// B1: softmax statistics of every key row (max, 1/sum) and, for the scalar
// gate, ell2_j = log2 sigmoid(mean_c k_j[c]). Eight lanes share a row (DPP
// reductions); rows past the end get 1/sum = 0 so phi(k) vanishes there, and
// ell2 = 0.
template <typename T, int D, int GATE, bool FULL>
__device__ __forceinline__ void key_row_stats(const Smem<T, D, GATE, FULL>& sm, int slot, int nvalid) {
    typedef Layout<T, D, GATE, FULL> L;
    static_assert(kPThreads == 64 * 8, "eight lanes per key row");
    constexpr int VPL = 16 / sizeof(T);
    constexpr int NLD = D / (8 * VPL);  // 16-byte loads per lane
    const int tid = ltid();
    const int j = tid >> 3, part = tid & 7;
    const T* row = sm.K + slot * 64 * L::DP + j * L::DP + part * VPL;
    float x[NLD * VPL];
#pragma unroll
    for (int q = 0; q < NLD; ++q) {
        const uint4 u = *reinterpret_cast<const uint4*>(row + q * 8 * VPL);
        const T* e = reinterpret_cast<const T*>(&u);
#pragma unroll
        for (int i = 0; i < VPL; ++i) x[q * VPL + i] = to_f32(e[i]);
    }
    float mx = -INFINITY, sraw = 0.f;
#pragma unroll
    for (int i = 0; i < NLD * VPL; ++i) {
        mx = fmaxf(mx, x[i]);
        sraw += x[i];
    }
    mx = group8_max(mx);
    float se = 0.f;
#pragma unroll
    for (int i = 0; i < NLD * VPL; ++i) se += fast_exp2((x[i] - mx) * kLog2e);
    se = group8_sum(se);
    if (GATE == 0) sraw = group8_sum(sraw);
    if (part == 0) {
        const bool ok = j < nvalid;
        sm.kmax[j] = mx;
        sm.kinv[j] = ok ? fast_rcp(se) : 0.0f;
        if (GATE == 0) sm.b2e[j] = ok ? log2_sigmoid(sraw * (1.0f / D)) : 0.0f;
    }
}

// Vector gate, part 1: thread (c, part) owns channel c and TPT consecutive
// tokens. x_j[c] = mean of k_j over the in-range channels c-1..c+2; ell2 =
// log2 sigmoid(x); b2 = inclusive prefix over the chunk. Leaves the raw
// reference (token min(31, n-1)), the last value and the first value per
// channel in LDS.
template <typename T, int D, int GATE, bool FULL, int TPT>
__device__ __forceinline__ void vector_gate_scan(const Smem<T, D, GATE, FULL>& sm, int slot,
                                                 int nvalid, float (&b2)[TPT]) {
    typedef Layout<T, D, GATE, FULL> L;
    constexpr int NPART = kPThreads / D;
    const int c = ltid() % D;
    const int part = ltid() / D;
    const T* Ks = sm.K + slot * 64 * L::DP;
    int cnt = 0;
    float xs[TPT];
#pragma unroll
    for (int jj = 0; jj < TPT; ++jj) xs[jj] = pool4_taps<D>(Ks + (part * TPT + jj) * L::DP, c, cnt);
    const float inv_cnt = 1.0f / static_cast<float>(cnt);
    float run = 0.f;
#pragma unroll
    for (int jj = 0; jj < TPT; ++jj) {
        const float l = log2_sigmoid(xs[jj] * inv_cnt);
        run += part * TPT + jj < nvalid ? l : 0.0f;
        b2[jj] = run;
    }
    sm.part[part * D + c] = run;
    lds_barrier();
    float off = 0.f;
#pragma unroll
    for (int p = 0; p < NPART - 1; ++p) {
        const float s = sm.part[p * D + c];
        off += p < part ? s : 0.0f;
    }
    const int ref = nvalid - 1 < 31 ? nvalid - 1 : 31;
    const int last = nvalid - 1;
#pragma unroll
    for (int jj = 0; jj < TPT; ++jj) {
        b2[jj] += off;
        const int j = part * TPT + jj;
        if (j == ref) sm.m2raw[c] = b2[jj];
        if (j == last) sm.bl2[c] = b2[jj];
        if (j == 0) sm.b0[c] = b2[jj];
    }
}

// ------------------------------------------------------------ state update
template <int D>
struct StateTiles {
    static constexpr int NTT = D / 16;
    static constexpr int TPW = NTT * NTT / kPWaves;
    static_assert(TPW >= 1, "state tiles per wave");
    __device__ static __forceinline__ int rt(int wave, int u) { return (wave * TPW + u) / NTT; }
    __device__ static __forceinline__ int ct(int wave, int u) { return (wave * TPW + u) % NTT; }
};

// S <- diag(dec) S + sfac Kst^T V over the current chunk. The key operand is
// Kb as [D][JP] (transposed, keys at key_pos) or, with NAT, Kb as the
// token-major [64][DP] intra operand read with transposing loads.
// With RES the state is read from and written back to the resident LDS copy
// (acc returns the new state); otherwise it lives in acc.
template <typename T, int D, int GATE, bool FULL, bool RES = false, bool NAT = false>
__device__ __forceinline__ void state_advance(const Smem<T, D, GATE, FULL>& sm, int slot,
                                              f32x4_t (&acc)[StateTiles<D>::TPW], float sfac = 1.0f) {
    typedef Layout<T, D, GATE, FULL> L;
    typedef Mfma<T> M;
    typedef StateTiles<D> ST;
    static_assert(ST::NTT % ST::TPW == 0, "a wave's state tiles share one row tile");
    const int lane = ltid() & 63, wave = ltid() >> 6;
    const int col = lane & 15, g = lane >> 4;
    const T* Vts = sm.Vt + slot * L::V_ELEMS;
    const int rt = ST::rt(wave, 0);
    f32x4_t d[ST::TPW];
#pragma unroll
    for (int u = 0; u < ST::TPW; ++u) d[u] = zero4();
#pragma unroll
    for (int ks = 0; ks < 64 / M::KSTEP; ++ks) {
        typename M::frag a;
        if constexpr (NAT && sizeof(T) == 2) a = load_key_frag(sm.Kb, L::DP, M::KSTEP * ks, 16 * rt, lane);
        else if constexpr (NAT) a = sm.Kb[(M::KSTEP * ks + g) * L::DP + 16 * rt + col];
        else a = M::load(sm.Kb + (16 * rt + col) * L::JP + M::KSTEP * ks + M::KPL * g);
#pragma unroll
        for (int u = 0; u < ST::TPW; ++u) {
            const int t = ST::ct(wave, u);
            typename M::frag b;
            if constexpr (L::VNAT) b = load_key_frag(Vts, L::VP, M::KSTEP * ks, 16 * t, lane);
            else b = M::load(Vts + (16 * t + col) * L::JP + M::KSTEP * ks + M::KPL * g);
            d[u] = M::mma(a, b, d[u]);
        }
    }
    const int r0 = 16 * rt + 4 * g;
#pragma unroll
    for (int u = 0; u < ST::TPW; ++u) {
        const int t = ST::ct(wave, u);
        float* res = sm.S32 + (16 * t + col) * L::SP + r0;
        if constexpr (RES) {
            const float4 v = *reinterpret_cast<const float4*>(res);
            acc[u] = f32x4_t{v.x, v.y, v.z, v.w};
        }
#pragma unroll
        for (int r = 0; r < 4; ++r) acc[u][r] = sm.dec[r0 + r] * acc[u][r] + (NAT ? sfac * d[u][r] : d[u][r]);
        if constexpr (RES) *reinterpret_cast<float4*>(res) = make_float4(acc[u][0], acc[u][1], acc[u][2], acc[u][3]);
    }
}

// Resident state <- acc (tiles in accumulator order).
template <typename T, int D, int GATE, bool FULL>
__device__ __forceinline__ void put_resident(const Smem<T, D, GATE, FULL>& sm,
                                             const f32x4_t (&acc)[StateTiles<D>::TPW]) {
    typedef Layout<T, D, GATE, FULL> L;
    typedef StateTiles<D> ST;
    const int lane = ltid() & 63, wave = ltid() >> 6;
    const int col = lane & 15, g = lane >> 4;
#pragma unroll
    for (int u = 0; u < ST::TPW; ++u) {
        const int rt = ST::rt(wave, u), t = ST::ct(wave, u);
        *reinterpret_cast<float4*>(sm.S32 + (16 * t + col) * L::SP + 16 * rt + 4 * g) =
            make_float4(acc[u][0], acc[u][1], acc[u][2], acc[u][3]);
    }
}

// S'^T[dv][r] = S[r][dv] * 2^(mref[r]) in the operand type (state operand of
// the inter-chunk product).
template <typename T, int D, int GATE, bool FULL>
__device__ __forceinline__ void publish_state(const Smem<T, D, GATE, FULL>& sm,
                                              const f32x4_t (&acc)[StateTiles<D>::TPW]) {
    typedef Layout<T, D, GATE, FULL> L;
    typedef StateTiles<D> ST;
    const int lane = ltid() & 63, wave = ltid() >> 6;
    const int col = lane & 15, g = lane >> 4;
#pragma unroll
    for (int u = 0; u < ST::TPW; ++u) {
        const int rt = ST::rt(wave, u), t = ST::ct(wave, u);
        const int r0 = 16 * rt + 4 * g;
        float x[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) x[r] = GATE ? acc[u][r] * fast_exp2(sm.mref[r0 + r]) : acc[u][r];
        T* dst = sm.St + (16 * t + col) * L::DP + r0;
        if constexpr (sizeof(T) == 2) {
            *reinterpret_cast<uint2*>(dst) = make_uint2(pack_bf16x2(x[0], x[1]), pack_bf16x2(x[2], x[3]));
        } else {
            *reinterpret_cast<float4*>(dst) = make_float4(x[0], x[1], x[2], x[3]);
        }
    }
}

// The same operand in global memory as fp32 [D][D] (global halo): read back
// by the other waves of the workgroup after a barrier.
template <typename T, int D, int GATE, bool FULL>
__device__ __forceinline__ void publish_state_global(const Smem<T, D, GATE, FULL>& sm, float* dst,
                                                     const f32x4_t (&acc)[StateTiles<D>::TPW]) {
    typedef StateTiles<D> ST;
    const int lane = ltid() & 63, wave = ltid() >> 6;
    const int col = lane & 15, g = lane >> 4;
#pragma unroll
    for (int u = 0; u < ST::TPW; ++u) {
        const int rt = ST::rt(wave, u), t = ST::ct(wave, u);
        const int r0 = 16 * rt + 4 * g;
        float x[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) x[r] = GATE ? acc[u][r] * fast_exp2(sm.mref[r0 + r]) : acc[u][r];
        *reinterpret_cast<float4*>(dst + (16 * t + col) * D + r0) = make_float4(x[0], x[1], x[2], x[3]);
    }
}

template <int D>
__device__ __forceinline__ void store_state(float* dst, const f32x4_t (&acc)[StateTiles<D>::TPW]) {
    typedef StateTiles<D> ST;
    const int lane = ltid() & 63, wave = ltid() >> 6;
    const int col = lane & 15, g = lane >> 4;
#pragma unroll
    for (int u = 0; u < ST::TPW; ++u) {
        const int r0 = 16 * ST::rt(wave, u) + 4 * g;
        const int cc = 16 * ST::ct(wave, u) + col;
#pragma unroll
        for (int r = 0; r < 4; ++r) dst[(r0 + r) * D + cc] = acc[u][r];
    }
}

template <int D>
__device__ __forceinline__ void load_state(const float* src, f32x4_t (&acc)[StateTiles<D>::TPW]) {
    typedef StateTiles<D> ST;
    const int lane = ltid() & 63, wave = ltid() >> 6;
    const int col = lane & 15, g = lane >> 4;
#pragma unroll
    for (int u = 0; u < ST::TPW; ++u) {
        const int r0 = 16 * ST::rt(wave, u) + 4 * g;
        const int cc = 16 * ST::ct(wave, u) + col;
#pragma unroll
        for (int r = 0; r < 4; ++r) acc[u][r] = src ? src[(r0 + r) * D + cc] : 0.0f;
    }
}

// Private state slot of an output workgroup, in accumulator order: every
// lane moves one float4 per tile, so each access is a contiguous 1 KiB per wave.
template <int D>
__device__ __forceinline__ void load_slot(const float* slot, f32x4_t (&acc)[StateTiles<D>::TPW]) {
    typedef StateTiles<D> ST;
    const int tid = ltid();
    const int wave = tid >> 6, lane = tid & 63;
#pragma unroll
    for (int u = 0; u < ST::TPW; ++u) {
        const float4 v = *reinterpret_cast<const float4*>(slot + (size_t((wave * ST::TPW + u) * 64 + lane)) * 4);
        acc[u] = f32x4_t{v.x, v.y, v.z, v.w};
    }
}
template <int D>
__device__ __forceinline__ void store_slot(float* slot, const f32x4_t (&acc)[StateTiles<D>::TPW]) {
    typedef StateTiles<D> ST;
    const int tid = ltid();
    const int wave = tid >> 6, lane = tid & 63;
#pragma unroll
    for (int u = 0; u < ST::TPW; ++u)
        *reinterpret_cast<float4*>(slot + (size_t((wave * ST::TPW + u) * 64 + lane)) * 4) =
            make_float4(acc[u][0], acc[u][1], acc[u][2], acc[u][3]);
}

// -------------------------------------------- gate prep shared by P1 and P3
// gate_stats leaves in LDS: key row statistics, the cumulative gates, dec,
// mref, emref (vector), blast, badlist/badmask/nbad and F (output kernels,
// vector), and returns (through b2) the per-thread cumulative gates.
template <typename T, int D, int GATE, bool FULL, int TPT>
__device__ __forceinline__ void gate_stats(const Smem<T, D, GATE, FULL>& sm, int slot, int nvalid,
                                           float alpha, float (&b2)[TPT]) {
    typedef Layout<T, D, GATE, FULL> L;
    key_row_stats(sm, slot, nvalid);
    lds_barrier();
    if (GATE == 0) {
        // Every wave forms the inclusive prefix of the chunk's gates itself
        // (lane shifts and lane reads); wave 0 publishes it. With the resident
        // state, b2s is next read after the caller's barrier; gate_prep reads
        // it right away and keeps the barrier.
        const float pre = wave_prefix_sum(sm.b2e[ltid() & 63]);
        if (ltid() < 64) sm.b2s[ltid()] = pre;
        if constexpr (!(FULL && L::SLDS)) lds_barrier();
        const float bl = readlane_f(pre, nvalid - 1);
        // reference for the factorised intra-chunk decay: the middle token
        const float m = readlane_f(pre, nvalid - 1 < 31 ? nvalid - 1 : 31);
        const bool ex = fmaxf(readlane_f(pre, 0) - m, m - bl) > kEmax2;
        if (ltid() < D) {
            sm.dec[ltid()] = fast_exp2(bl);
            sm.mref[ltid()] = ex ? 0.0f : m;
            sm.blast[ltid()] = bl;
        }
        if (ltid() == 0) *sm.exact = ex ? 1 : 0;
    } else {
        vector_gate_scan<T, D, GATE, FULL, TPT>(sm, slot, nvalid, b2);
        lds_barrier();
        const int c = ltid() % D;
        const int part = ltid() / D;
        const float m2 = sm.m2raw[c];
        const float bl = sm.bl2[c];
        const bool bad = fmaxf(sm.b0[c] - m2, m2 - bl) > kEmax2;
        const float mref = bad ? 0.0f : m2;
        if (part == 0) {
            sm.mref[c] = mref;
            sm.emref[c] = fast_exp2(mref);
            sm.dec[c] = fast_exp2(bl);
            sm.blast[c] = bl;
            if (FULL && bad) {
                const int idx = atomicAdd(sm.nbad, 1);
                sm.badlist[idx] = c;
                atomicOr(&sm.badmask[c >> 5], 1u << (c & 31));
            }
        }
        if (FULL) {
#pragma unroll
            for (int jj = 0; jj < TPT; ++jj) {
                const int j = part * TPT + jj;
                sm.F[j * L::FP + c] = bad ? b2[jj] : alpha * fast_exp2(b2[jj] - mref);
            }
        }
    }
}

// Transposed state key operand Kb[c][key_pos(j)] = phik_j[c] 2^(b_last[c] - b_j[c])
// (b_last per channel from bl; the scalar gate reads its own scan).
template <typename T, int D, int GATE, bool FULL, int TPT>
__device__ __forceinline__ void state_key_operand(const Smem<T, D, GATE, FULL>& sm, int slot, int nvalid,
                                                  const float* bl, const float (&b2)[TPT]) {
    typedef Layout<T, D, GATE, FULL> L;
    const T* Ks = sm.K + slot * 64 * L::DP;
    if (GATE == 0) {
        const float blv = sm.b2s[nvalid - 1];
        constexpr int VPL = 16 / sizeof(T);
        for (int idx = ltid(); idx < 32 * (D / VPL); idx += kPThreads) {
            const int j0 = 2 * (idx & 31);
            const int c0 = (idx >> 5) * VPL;
            const uint4 u0 = *reinterpret_cast<const uint4*>(Ks + j0 * L::DP + c0);
            const uint4 u1 = *reinterpret_cast<const uint4*>(Ks + (j0 + 1) * L::DP + c0);
            const T* e0 = reinterpret_cast<const T*>(&u0);
            const T* e1 = reinterpret_cast<const T*>(&u1);
            const float m0 = sm.kmax[j0], m1 = sm.kmax[j0 + 1];
            const float f0 = blv - sm.b2s[j0], f1 = blv - sm.b2s[j0 + 1];
            const float s0 = sm.kinv[j0], s1 = sm.kinv[j0 + 1];
            T* dst = sm.Kb + c0 * L::JP + key_pos(j0);
#pragma unroll
            for (int e = 0; e < VPL; ++e) {
                const float a = s0 * fast_exp2((to_f32(e0[e]) - m0) * kLog2e + f0);
                const float b = s1 * fast_exp2((to_f32(e1[e]) - m1) * kLog2e + f1);
                if constexpr (sizeof(T) == 2) {
                    *reinterpret_cast<uint32_t*>(dst + e * L::JP) = pack_bf16x2(a, b);
                } else {
                    *reinterpret_cast<float2*>(dst + e * L::JP) = make_float2(a, b);
                }
            }
        }
    } else {
        const int c = ltid() % D;
        const int part = ltid() / D;
        const float blc = bl[c];
#pragma unroll
        for (int jj = 0; jj < TPT; ++jj) {
            const int j = part * TPT + jj;
            const float kv = to_f32(Ks[j * L::DP + c]);
            sm.Kb[c * L::JP + key_pos(j)] =
                from_f32<T>(sm.kinv[j] * fast_exp2((kv - sm.kmax[j]) * kLog2e + blc - b2[jj]));
        }
    }
}

// Both steps back to back (segment-state kernel and output kernels without a
// resident state); the vector gate reads b_last from the scan scratch.
template <typename T, int D, int GATE, bool FULL, int TPT>
__device__ __forceinline__ void gate_prep(const Smem<T, D, GATE, FULL>& sm, int slot, int nvalid,
                                          float alpha, float (&b2)[TPT]) {
    gate_stats<T, D, GATE, FULL, TPT>(sm, slot, nvalid, alpha, b2);
    state_key_operand<T, D, GATE, FULL, TPT>(sm, slot, nvalid, sm.bl2, b2);
}

// Scalar gate with the resident state: key row statistics, the chunk's gate
// prefix and the intra operand Kb[j][c] = phik_j[c] 2^(mref - b_j) in one
// phase with one barrier. Thread (j, part) keeps the exponentials of its
// pieces of key row j in registers for the operand, and takes b_j, the
// reference and the exact flag from its own wave's scan (every wave scans
// the same 64 gates), so nothing it writes to Kb depends on another wave's
// LDS stores after the barrier. Leaves in LDS what gate_stats leaves and the
// same operand as intra_key_operand.
template <typename T, int D>
__device__ __forceinline__ void scalar_gate_intra(const Smem<T, D, 0, true>& sm, int slot, int nvalid) {
    typedef Layout<T, D, 0, true> L;
    static_assert(kPThreads == 64 * 8, "eight lanes per key row");
    constexpr int VPL = 16 / sizeof(T);
    constexpr int NLD = D / (8 * VPL);  // pieces of VPL elements per lane: part * VPL + 8 VPL q
    const int tid = ltid();
    const int j = tid >> 3, part = tid & 7;
    const T* row = sm.K + slot * 64 * L::DP + j * L::DP + part * VPL;
    float x[NLD * VPL];
#pragma unroll
    for (int q = 0; q < NLD; ++q) {
        const uint4 u = *reinterpret_cast<const uint4*>(row + q * 8 * VPL);
        const T* e = reinterpret_cast<const T*>(&u);
#pragma unroll
        for (int i = 0; i < VPL; ++i) x[q * VPL + i] = to_f32(e[i]);
    }
    float mx = -INFINITY, sraw = 0.f;
#pragma unroll
    for (int i = 0; i < NLD * VPL; ++i) {
        mx = fmaxf(mx, x[i]);
        sraw += x[i];
    }
    mx = group8_max(mx);
    float se = 0.f;
#pragma unroll
    for (int i = 0; i < NLD * VPL; ++i) {
        x[i] = fast_exp2((x[i] - mx) * kLog2e);
        se += x[i];
    }
    se = group8_sum(se);
    sraw = group8_sum(sraw);
    const bool ok = j < nvalid;
    const float kinv = ok ? fast_rcp(se) : 0.0f;
    if (part == 0) {
        sm.kmax[j] = mx;
        sm.kinv[j] = kinv;
        sm.b2e[j] = ok ? log2_sigmoid(sraw * (1.0f / D)) : 0.0f;
    }
    __syncthreads();
    const float pre = wave_prefix_sum(sm.b2e[tid & 63]);
    if (tid < 64) sm.b2s[tid] = pre;
    const float bl = readlane_f(pre, nvalid - 1);
    // reference for the factorised intra-chunk decay: the middle token
    const float m = readlane_f(pre, nvalid - 1 < 31 ? nvalid - 1 : 31);
    const bool ex = fmaxf(readlane_f(pre, 0) - m, m - bl) > kEmax2;
    if (tid < D) {
        sm.dec[tid] = fast_exp2(bl);
        sm.mref[tid] = ex ? 0.0f : m;
        sm.blast[tid] = bl;
    }
    if (tid == 0) *sm.exact = ex ? 1 : 0;
    const float bj = __shfl(pre, j, 64);
    const float sc = kinv * (ex ? 1.0f : fast_exp2(m - bj));
    T* dst = sm.Kb + j * L::DP + part * VPL;
#pragma unroll
    for (int q = 0; q < NLD; ++q) {
        const float* y = x + q * VPL;
        if constexpr (sizeof(T) == 2) {
            *reinterpret_cast<uint4*>(dst + q * 8 * VPL) =
                make_uint4(pack_bf16x2(sc * y[0], sc * y[1]), pack_bf16x2(sc * y[2], sc * y[3]),
                           pack_bf16x2(sc * y[4], sc * y[5]), pack_bf16x2(sc * y[6], sc * y[7]));
        } else {
            *reinterpret_cast<float4*>(dst + q * 8 * VPL) = make_float4(sc * y[0], sc * y[1], sc * y[2], sc * y[3]);
        }
    }
}

// Intra operand Kb[j][c] = phik_j[c] 2^(mref[c] - b_j[c]) (vector, good
// channels), 0 (bad channels), phik_j[c] (scalar gate).
template <typename T, int D, int GATE, bool FULL, int TPT>
__device__ __forceinline__ void intra_key_operand(const Smem<T, D, GATE, FULL>& sm, int slot,
                                                  const float (&b2)[TPT]) {
    typedef Layout<T, D, GATE, FULL> L;
    const T* Ks = sm.K + slot * 64 * L::DP;
    if (GATE == 0) {
        constexpr int VPL = 16 / sizeof(T);
        for (int idx = ltid(); idx < 64 * (D / VPL); idx += kPThreads) {
            const int j = idx / (D / VPL);
            const int c0 = (idx % (D / VPL)) * VPL;
            const uint4 u = *reinterpret_cast<const uint4*>(Ks + j * L::DP + c0);
            const T* e = reinterpret_cast<const T*>(&u);
            const float m = sm.kmax[j];
            const float sc = sm.kinv[j] * (*sm.exact ? 1.0f : fast_exp2(sm.mref[0] - sm.b2s[j]));
            float y[VPL];
#pragma unroll
            for (int i = 0; i < VPL; ++i) y[i] = sc * fast_exp2((to_f32(e[i]) - m) * kLog2e);
            if constexpr (sizeof(T) == 2) {
                *reinterpret_cast<uint4*>(sm.Kb + j * L::DP + c0) =
                    make_uint4(pack_bf16x2(y[0], y[1]), pack_bf16x2(y[2], y[3]), pack_bf16x2(y[4], y[5]),
                               pack_bf16x2(y[6], y[7]));
            } else {
                *reinterpret_cast<float4*>(sm.Kb + j * L::DP + c0) = make_float4(y[0], y[1], y[2], y[3]);
            }
        }
    } else {
        const int c = ltid() % D;
        const int part = ltid() / D;
        const float mref = sm.mref[c];
        const bool bad = (sm.badmask[c >> 5] >> (c & 31)) & 1u;
#pragma unroll
        for (int jj = 0; jj < TPT; ++jj) {
            const int j = part * TPT + jj;
            const float kv = to_f32(Ks[j * L::DP + c]);
            const float val = bad ? 0.0f : sm.kinv[j] * fast_exp2((kv - sm.kmax[j]) * kLog2e + mref - b2[jj]);
            sm.Kb[j * L::DP + c] = from_f32<T>(val);
        }
    }
}

// ------------------------------------------------------------------ P1
// Local end state of a segment (from a zero state) and its total log2 decay:
//   L = sum_j (phik_j (.) 2^(b_end - b_j))^T v_j ,  lg = b_end
// over the segment's tokens, in blocks of up to TB tokens held in LDS
// token-major. Per block: key row statistics; the log2 gates and, per token,
// the sum of the gates after it (computed as suffix sums, so every factor is
// at most 1); the key operand phik_j (.) 2^(suffix after j); then one MFMA
// contraction over the block's tokens added to the running state rescaled by
// the block's decay. The vector gate (a log2 gate per channel) and the scalar
// gate (one per token) have a kernel each.
// Vector gate. The gate differs per channel, so each block needs a suffix
// sum per (token, channel): the lanes of a group share one 16-byte channel
// piece over a run of tokens (thread tid: piece tid / LPP, tokens
// TPL (tid % LPP) ..), the 4-tap pooled input comes from the piece and three
// neighbouring elements of the raw key row, and the suffix sums run over
// the lane group with DPP row shifts. Two barriers per block: the raw key
// tile, the value tile and the key operand alternate between two LDS
// buffers, and the operand has a buffer of its own, so it can be written
// while other lanes still read raw keys for their pooled inputs.
//   (a) each thread commits its raw key and value pieces, and forms the
//       softmax statistics of its key rows from its loaded registers (PPR
//       lanes per row); the next block's loads go into the same
//       registers;                                              barrier
//   (b) pooled gates, suffix sums over the group and the key operand
//       phik_j[c] 2^(gates after j in the block + later[c]), later = the
//       gates of the blocks after this one (blocks are taken from the
//       segment's end backwards, so the state is never rescaled);  barrier
//   (c) acc += Kop^T V, beside (a) of the next block.
// A segment is a whole number of chunks, so every block is a full chunk.
template <typename T, int D>
struct SegLayoutVector {
    static constexpr int E = sizeof(T);
    static constexpr int TB = kChunk;                  // tokens per block
    static constexpr int P = D + 16;                   // row pitch (elements) of the tiles
    static constexpr int VPL = 16 / E;                 // elements per 16-byte piece
    static constexpr int PPR = D / VPL;                // pieces per row
    static constexpr int NPT = TB * PPR / kPThreads;   // key (and value) pieces per thread
    static constexpr int TPL = TB * PPR / kPThreads;   // tokens per lane in the gate phase
    static constexpr int LPP = TB / TPL;               // lanes per channel piece in the gate phase
    static_assert(TB == 64 && NPT * kPThreads == TB * PPR, "block mapping");
    static_assert(PPR == 8 || PPR == 16, "a key row spans 8 or 16 lanes");
    static_assert(LPP == 32 || LPP == 64, "a piece spans half a wave or a whole wave");
    static constexpr size_t TILE = size_t(TB) * P * E;
    static constexpr size_t K_OFF = 0;         // raw keys, two buffers
    static constexpr size_t V_OFF = 2 * TILE;  // values, two buffers
    static constexpr size_t O_OFF = 4 * TILE;  // key operand, two buffers
    static constexpr size_t F_OFF = 6 * TILE;  // fp32: kmx[TB] kiv[TB]
    static constexpr size_t TOTAL = F_OFF + 2 * size_t(TB) * 4;
    static_assert(TOTAL <= 160 * 1024, "LDS budget of a gfx950 workgroup exceeded");
};

template <typename T, int D>
__global__ __launch_bounds__(kPThreads) void segment_state_vector_kernel(PrefillParams p) {
    typedef SegLayoutVector<T, D> SL;
    typedef Mfma<T> M;
    typedef StateTiles<D> ST;
    constexpr int RTW = ST::NTT >= 8 ? 2 : 1;  // state row tiles per wave
    constexpr int CTW = ST::TPW / RTW;          // state column tiles per wave
    static_assert(RTW * CTW == ST::TPW && (ST::NTT / RTW) * (ST::NTT / CTW) == kPWaves, "state tiling");
    static_assert(SL::TB % M::KSTEP == 0, "whole MFMA steps per block");
    constexpr int VPL = SL::VPL, TPL = SL::TPL, LPP = SL::LPP;
    __shared__ __align__(16) char smem[SL::TOTAL];
    float* kmx = reinterpret_cast<float*>(smem + SL::F_OFF);  // row max times log2 e
    float* kiv = kmx + SL::TB;                                 // 1 / row sum of exponentials

    const int s = blockIdx.x;
    const int h = blockIdx.y;
    const int64_t b = blockIdx.z;
    const int tid = threadIdx.x;
    const int lane = tid & 63, wave = tid >> 6;
    const int64_t tok0 = int64_t(s) * p.cps * kChunk;  // never the last segment: whole chunks
    const int nblk = int(p.cps);
    const int64_t blk_stride = int64_t(SL::TB) * p.H_kv * D;
    const T* kp[SL::NPT];
    const T* vp[SL::NPT];
#pragma unroll
    for (int n = 0; n < SL::NPT; ++n) {
        const int idx = tid + n * kPThreads;
        const int64_t off = ((b * p.T + tok0 + idx / SL::PPR) * p.H_kv + h) * D + (idx % SL::PPR) * VPL;
        kp[n] = static_cast<const T*>(p.k) + off;
        vp[n] = static_cast<const T*>(p.v) + off;
    }
    typedef unsigned u32x4 __attribute__((ext_vector_type(4)));  // a register quadruple, not a struct
    u32x4 kr[SL::NPT], vr[SL::NPT];
    auto issue = [&](int it) {  // the it-th block taken, counted from the segment's end
        const int64_t o = int64_t(nblk - 1 - it) * blk_stride;
#pragma unroll
        for (int n = 0; n < SL::NPT; ++n) {
            kr[n] = *reinterpret_cast<const u32x4*>(kp[n] + o);
            vr[n] = *reinterpret_cast<const u32x4*>(vp[n] + o);
        }
    };
    auto Kraw = [&](int buf) { return reinterpret_cast<T*>(smem + SL::K_OFF + buf * SL::TILE); };
    auto Vs = [&](int buf) { return reinterpret_cast<T*>(smem + SL::V_OFF + buf * SL::TILE); };
    auto Kop = [&](int buf) { return reinterpret_cast<T*>(smem + SL::O_OFF + buf * SL::TILE); };

    // (a) raw pieces to LDS; row statistics from the registers
    auto commit_stats = [&](int it, int buf) {
        float mxs[SL::NPT], ses[SL::NPT];
#pragma unroll
        for (int n = 0; n < SL::NPT; ++n) {
            const int idx = tid + n * kPThreads;
            const int o = (idx / SL::PPR) * SL::P + (idx % SL::PPR) * VPL;
            *reinterpret_cast<u32x4*>(Kraw(buf) + o) = kr[n];
            *reinterpret_cast<u32x4*>(Vs(buf) + o) = vr[n];
            const unsigned w[4] = {kr[n].x, kr[n].y, kr[n].z, kr[n].w};
            float x[VPL];
#pragma unroll
            for (int i = 0; i < VPL; ++i) {
                if constexpr (sizeof(T) == 2)  // element i is the low (even i) or high half of word i / 2
                    x[i] = __uint_as_float(i % 2 == 0 ? w[i / 2] << 16 : w[i / 2] & 0xffff0000u);
                else
                    x[i] = __uint_as_float(w[i]);
            }
            float mx = -INFINITY;
#pragma unroll
            for (int i = 0; i < VPL; ++i) mx = fmaxf(mx, x[i]);
            mx = group8_max(mx);
            if (SL::PPR == 16) mx = fmaxf(mx, dpp<kDppMirror>(mx));
            mx *= kLog2e;
            float se = 0.f;
#pragma unroll
            for (int i = 0; i < VPL; ++i) se += fast_exp2(fmaf(x[i], kLog2e, -mx));
            se = group8_sum(se);
            if (SL::PPR == 16) se += dpp<kDppMirror>(se);
            mxs[n] = mx;
            ses[n] = se;
        }
        if (it + 1 < nblk) issue(it + 1);
#pragma unroll
        for (int n = 0; n < SL::NPT; ++n) {
            const int idx = tid + n * kPThreads;
            if (idx % SL::PPR == 0) {
                kmx[idx / SL::PPR] = mxs[n];
                kiv[idx / SL::PPR] = fast_rcp(ses[n]);
            }
        }
    };

    // (b) pooled gates, suffix sums, key operand; later[] carries the
    // per-channel gates of the blocks already taken
    const int c0 = (tid / LPP) * VPL;
    const int l = tid % LPP;
    float later[VPL];
#pragma unroll
    for (int i = 0; i < VPL; ++i) later[i] = 0.0f;
    auto gate_operand = [&](int buf) {
        const T* Kr = Kraw(buf);
        float lg2[TPL][VPL];  // log2 gate per (token, channel)
#pragma unroll
        for (int t = 0; t < TPL; ++t) {
            const int j = TPL * l + t;
            const T* row = Kr + j * SL::P;
            const uint4 u = *reinterpret_cast<const uint4*>(row + c0);
            const T* pe = reinterpret_cast<const T*>(&u);
            float e[VPL + 3];  // channels c0 - 1 .. c0 + VPL + 1, zero outside the row
            e[0] = c0 > 0 ? to_f32(row[c0 - 1]) : 0.0f;
#pragma unroll
            for (int i = 0; i < VPL; ++i) e[i + 1] = to_f32(pe[i]);
            e[VPL + 1] = c0 + VPL < D ? to_f32(row[c0 + VPL]) : 0.0f;
            e[VPL + 2] = c0 + VPL < D ? to_f32(row[c0 + VPL + 1]) : 0.0f;
#pragma unroll
            for (int i = 0; i < VPL; ++i) {
                const int c = c0 + i;
                const float inv_cnt = (c == 0 || c == D - 2) ? (1.0f / 3.0f) : c == D - 1 ? 0.5f : 0.25f;
                const float x = (e[i] + e[i + 1]) + (e[i + 2] + e[i + 3]);
                lg2[t][i] = log2_sigmoid(x * inv_cnt);
            }
        }
        // the gates after each token: this lane's later tokens, then the
        // lanes after it (inclusive suffix over the group), then later blocks
        float after[VPL], tot[VPL];
#pragma unroll
        for (int i = 0; i < VPL; ++i) {
            float own = 0.f;
#pragma unroll
            for (int t = 0; t < TPL; ++t) own += lg2[t][i];
            const float incl = group_suffix_sum<LPP>(own);
            after[i] = incl - own + later[i];
            // the block's total: the group's first lane
            tot[i] = LPP == 64 ? readlane_f(incl, 0) : (lane < 32 ? readlane_f(incl, 0) : readlane_f(incl, 32));
        }
        T* Ko = Kop(buf);
#pragma unroll
        for (int t = TPL - 1; t >= 0; --t) {
            const int j = TPL * l + t;
            const uint4 u = *reinterpret_cast<const uint4*>(Kr + j * SL::P + c0);
            const T* pe = reinterpret_cast<const T*>(&u);
            const float m = kmx[j], sc = kiv[j];
            float y[VPL];
#pragma unroll
            for (int i = 0; i < VPL; ++i) {
                y[i] = sc * fast_exp2(fmaf(to_f32(pe[i]), kLog2e, after[i] - m));
                after[i] += lg2[t][i];
            }
            T* dst = Ko + j * SL::P + c0;
            if constexpr (sizeof(T) == 2) {
                *reinterpret_cast<uint4*>(dst) = make_uint4(pack_bf16x2(y[0], y[1]), pack_bf16x2(y[2], y[3]),
                                                            pack_bf16x2(y[4], y[5]), pack_bf16x2(y[6], y[7]));
            } else {
                *reinterpret_cast<float4*>(dst) = make_float4(y[0], y[1], y[2], y[3]);
            }
        }
#pragma unroll
        for (int i = 0; i < VPL; ++i) later[i] += tot[i];
    };

    // (c) acc += Kop^T V
    f32x4_t acc[ST::TPW];
#pragma unroll
    for (int u = 0; u < ST::TPW; ++u) acc[u] = zero4();
    const int col = lane & 15, g = lane >> 4;
    const int rt0 = (wave % (ST::NTT / RTW)) * RTW;
    const int ct0 = (wave / (ST::NTT / RTW)) * CTW;
    auto contract = [&](int buf) {
#pragma unroll
        for (int ks = 0; ks < SL::TB / M::KSTEP; ++ks) {
            typename M::frag af[RTW], bv[CTW];
#pragma unroll
            for (int a = 0; a < RTW; ++a) {
                if constexpr (sizeof(T) == 2) af[a] = load_key_frag(Kop(buf), SL::P, M::KSTEP * ks, 16 * (rt0 + a), lane);
                else af[a] = Kop(buf)[(M::KSTEP * ks + g) * SL::P + 16 * (rt0 + a) + col];
            }
#pragma unroll
            for (int tt = 0; tt < CTW; ++tt) {
                if constexpr (sizeof(T) == 2) bv[tt] = load_key_frag(Vs(buf), SL::P, M::KSTEP * ks, 16 * (ct0 + tt), lane);
                else bv[tt] = Vs(buf)[(M::KSTEP * ks + g) * SL::P + 16 * (ct0 + tt) + col];
            }
#pragma unroll
            for (int tt = 0; tt < CTW; ++tt)
#pragma unroll
                for (int a = 0; a < RTW; ++a) acc[a * CTW + tt] = M::mma(af[a], bv[tt], acc[a * CTW + tt]);
        }
    };

    issue(0);
    commit_stats(0, 0);
    for (int it = 0; it < nblk; ++it) {
        const int buf = it & 1;
        lds_barrier();  // this block's raw keys, values and row statistics are visible
        gate_operand(buf);
        lds_barrier();  // this block's key operand is visible
        if (it + 1 < nblk) {
            commit_stats(it + 1, buf ^ 1);
            contract(buf);
        } else {
            contract(buf);
        }
    }
    const size_t rec = size_t(D) * D + D;
    float* dst = p.carry + ((size_t(b) * p.H_kv + h) * size_t(p.n_seg - 1) + s) * rec;
#pragma unroll
    for (int a = 0; a < RTW; ++a)
#pragma unroll
        for (int tt = 0; tt < CTW; ++tt)
#pragma unroll
            for (int r = 0; r < 4; ++r)
                dst[(16 * (rt0 + a) + 4 * g + r) * D + 16 * (ct0 + tt) + col] = acc[a * CTW + tt][r];
    if (l == 0) {
#pragma unroll
        for (int i = 0; i < VPL; ++i) dst[size_t(D) * D + c0 + i] = later[i];
    }
}

// Scalar gate. Every channel of a token shares one log2 gate, so a block
// needs one gate and one suffix sum per token, and the kernel takes two
// barriers per block: the key operand and the value tile alternate between
// two LDS buffers, so nothing written for one block can overwrite what the
// contraction of the block before still reads. The blocks are taken from the
// segment's end backwards.
//   (a) from its loaded registers each thread commits its value pieces,
//       converts its key pieces (the next block's loads then go into the same
//       registers), forms the key-row softmax over the PPR lanes of the row and
//       the token's log2 gate, and publishes the gate;          barrier
//   (b) every wave forms the suffix sums of the block's gates itself (lane
//       shifts and lane reads, no further barrier) and writes the key operand
//       phik_j 2^(gates after j, in this block and the later ones);  barrier
//   (c) acc += Kop^T V, beside (a) of the next block.
// A segment is a whole number of chunks, so every block is a full chunk and
// no load needs a bounds test.
template <typename T, int D>
struct SegLayoutScalar {
    static constexpr int E = sizeof(T);
    static constexpr int TB = kChunk;                  // tokens per block, one per lane of the gate scan
    static constexpr int P = D + 16;                   // row pitch (elements) of the tiles
    static constexpr int VPL = 16 / E;                 // elements per 16-byte piece
    static constexpr int PPR = D / VPL;                // pieces per row
    static constexpr int NPT = TB * PPR / kPThreads;   // key (and value) pieces per thread
    static_assert(TB == 64 && NPT * kPThreads == TB * PPR, "block mapping");
    static_assert(PPR == 8 || PPR == 16, "a key row spans 8 or 16 lanes");
    static constexpr size_t TILE = size_t(TB) * P * E;
    static constexpr size_t K_OFF = 0;         // key operand, two buffers
    static constexpr size_t V_OFF = 2 * TILE;  // values, two buffers
    static constexpr size_t G_OFF = 4 * TILE;  // log2 gates, two buffers of TB floats
    static constexpr size_t TOTAL = G_OFF + 2 * size_t(TB) * 4;
    static_assert(TOTAL <= 160 * 1024, "LDS budget of a gfx950 workgroup exceeded");
};

template <typename T, int D>
__global__ __launch_bounds__(kPThreads) void segment_state_scalar_kernel(PrefillParams p) {
    typedef SegLayoutScalar<T, D> SL;
    typedef Mfma<T> M;
    typedef StateTiles<D> ST;
    constexpr int RTW = ST::NTT >= 8 ? 2 : 1;  // state row tiles per wave
    constexpr int CTW = ST::TPW / RTW;          // state column tiles per wave
    static_assert(RTW * CTW == ST::TPW && (ST::NTT / RTW) * (ST::NTT / CTW) == kPWaves, "state tiling");
    static_assert(SL::TB % M::KSTEP == 0, "whole MFMA steps per block");
    __shared__ __align__(16) char smem[SL::TOTAL];

    const int s = blockIdx.x;
    const int h = blockIdx.y;
    const int64_t b = blockIdx.z;
    const int tid = threadIdx.x;
    const int lane = tid & 63, wave = tid >> 6;
    const int64_t tok0 = int64_t(s) * p.cps * kChunk;  // never the last segment: whole chunks
    const int nblk = int(p.cps);                        // blocks of one chunk each
    const int64_t blk_stride = int64_t(SL::TB) * p.H_kv * D;  // elements between consecutive blocks
    // this thread's pieces of the segment's first block (token row idx / PPR, piece idx % PPR)
    const T* kp[SL::NPT];
    const T* vp[SL::NPT];
#pragma unroll
    for (int n = 0; n < SL::NPT; ++n) {
        const int idx = tid + n * kPThreads;
        const int64_t off = ((b * p.T + tok0 + idx / SL::PPR) * p.H_kv + h) * D + (idx % SL::PPR) * SL::VPL;
        kp[n] = static_cast<const T*>(p.k) + off;
        vp[n] = static_cast<const T*>(p.v) + off;
    }

    typedef unsigned u32x4 __attribute__((ext_vector_type(4)));  // a register quadruple, not a struct
    u32x4 kr[SL::NPT], vr[SL::NPT];
    auto issue = [&](int it) {  // the it-th block taken, counted from the segment's end
        const int64_t o = int64_t(nblk - 1 - it) * blk_stride;
#pragma unroll
        for (int n = 0; n < SL::NPT; ++n) {
            kr[n] = *reinterpret_cast<const u32x4*>(kp[n] + o);
            vr[n] = *reinterpret_cast<const u32x4*>(vp[n] + o);
        }
    };
    auto red_max = [](float v) {
        v = group8_max(v);
        if (SL::PPR == 16) v = fmaxf(v, dpp<kDppMirror>(v));
        return v;
    };
    auto red_sum = [](float v) {
        v = group8_sum(v);
        if (SL::PPR == 16) v += dpp<kDppMirror>(v);
        return v;
    };
    auto Kop = [&](int buf) { return reinterpret_cast<T*>(smem + SL::K_OFF + buf * SL::TILE); };
    auto Vs = [&](int buf) { return reinterpret_cast<T*>(smem + SL::V_OFF + buf * SL::TILE); };
    auto ell = [&](int buf) { return reinterpret_cast<float*>(smem + SL::G_OFF) + buf * SL::TB; };

    // (a) of a block whose loads are in kr/vr: values committed, key pieces
    // converted, the block after it issued into the same registers, key-row
    // statistics and the token gates (published to LDS)
    float ex[SL::NPT][SL::VPL];
    float kiv[SL::NPT];
    auto convert_commit = [&](int it, int buf) {
#pragma unroll
        for (int n = 0; n < SL::NPT; ++n) {
            const int idx = tid + n * kPThreads;
            *reinterpret_cast<u32x4*>(Vs(buf) + (idx / SL::PPR) * SL::P + (idx % SL::PPR) * SL::VPL) = vr[n];
            const unsigned w[4] = {kr[n].x, kr[n].y, kr[n].z, kr[n].w};
#pragma unroll
            for (int i = 0; i < SL::VPL; ++i) {
                if constexpr (sizeof(T) == 2)  // element i is the low (even i) or high half of word i / 2
                    ex[n][i] = __uint_as_float(i % 2 == 0 ? w[i / 2] << 16 : w[i / 2] & 0xffff0000u);
                else
                    ex[n][i] = __uint_as_float(w[i]);
            }
        }
        if (it + 1 < nblk) issue(it + 1);
    };
    auto stats = [&](int buf) {
#pragma unroll
        for (int n = 0; n < SL::NPT; ++n) {
            const int idx = tid + n * kPThreads;
            float mx = -INFINITY, sraw = 0.f;
#pragma unroll
            for (int i = 0; i < SL::VPL; ++i) {
                mx = fmaxf(mx, ex[n][i]);
                sraw += ex[n][i];
            }
            mx = red_max(mx) * kLog2e;
            float se = 0.f;
#pragma unroll
            for (int i = 0; i < SL::VPL; ++i) {
                ex[n][i] = fast_exp2(fmaf(ex[n][i], kLog2e, -mx));
                se += ex[n][i];
            }
            kiv[n] = fast_rcp(red_sum(se));
            sraw = red_sum(sraw);
            // every lane of the row stores the same value: no branch splits the region
            ell(buf)[idx / SL::PPR] = log2_sigmoid(sraw * (1.0f / D));
        }
    };
    // (b) suffix sums of the block's gates (each wave for itself), key operand
    // phik_j 2^(gates after j in the block + later), later = the gates of the
    // blocks after this one
    auto scan_operand = [&](int buf, float later) {
        const float incl = wave_suffix_sum(ell(buf)[lane]);  // sum of the gates of tokens >= lane
#pragma unroll
        for (int n = 0; n < SL::NPT; ++n) {
            const int idx = tid + n * kPThreads;
            const int j = idx / SL::PPR;
            float after = __shfl(incl, (j + 1) & 63, 64);  // the gates after token j
            if (j == SL::TB - 1) after = 0.0f;
            const float f = kiv[n] * fast_exp2(after + later);
            float y[SL::VPL];
#pragma unroll
            for (int i = 0; i < SL::VPL; ++i) y[i] = f * ex[n][i];
            T* e = Kop(buf) + j * SL::P + (idx % SL::PPR) * SL::VPL;
            if constexpr (sizeof(T) == 2) {
                *reinterpret_cast<uint4*>(e) = make_uint4(pack_bf16x2(y[0], y[1]), pack_bf16x2(y[2], y[3]),
                                                          pack_bf16x2(y[4], y[5]), pack_bf16x2(y[6], y[7]));
            } else {
                *reinterpret_cast<float4*>(e) = make_float4(y[0], y[1], y[2], y[3]);
            }
        }
        return readlane_f(incl, 0);  // the whole block
    };
    // (c) acc += Kop^T V; wave w owns row tiles rt0 .. rt0+RTW-1 and column
    // tiles ct0 .. ct0+CTW-1
    f32x4_t acc[ST::TPW];
#pragma unroll
    for (int u = 0; u < ST::TPW; ++u) acc[u] = zero4();
    const int col = lane & 15, g = lane >> 4;
    const int rt0 = (wave % (ST::NTT / RTW)) * RTW;
    const int ct0 = (wave / (ST::NTT / RTW)) * CTW;
    auto contract = [&](int buf) {
#pragma unroll
        for (int ks = 0; ks < SL::TB / M::KSTEP; ++ks) {
            typename M::frag af[RTW], bv[CTW];
#pragma unroll
            for (int a = 0; a < RTW; ++a) {
                if constexpr (sizeof(T) == 2) af[a] = load_key_frag(Kop(buf), SL::P, M::KSTEP * ks, 16 * (rt0 + a), lane);
                else af[a] = Kop(buf)[(M::KSTEP * ks + g) * SL::P + 16 * (rt0 + a) + col];
            }
#pragma unroll
            for (int tt = 0; tt < CTW; ++tt) {
                if constexpr (sizeof(T) == 2) bv[tt] = load_key_frag(Vs(buf), SL::P, M::KSTEP * ks, 16 * (ct0 + tt), lane);
                else bv[tt] = Vs(buf)[(M::KSTEP * ks + g) * SL::P + 16 * (ct0 + tt) + col];
            }
#pragma unroll
            for (int tt = 0; tt < CTW; ++tt)
#pragma unroll
                for (int a = 0; a < RTW; ++a) acc[a * CTW + tt] = M::mma(af[a], bv[tt], acc[a * CTW + tt]);
        }
    };

    // The blocks are taken last to first, so the decay of the blocks after a
    // block is already known when its key operand is formed and the running
    // state is never rescaled. Block n's contraction (LDS and MFMA work)
    // shares a region with the statistics of the block before it (VALU
    // work): the two use different buffers, and the block after that
    // overwrites block n's buffers only after the next first barrier.
    float lgs = 0.0f;  // log2 decay of the blocks taken so far (the same for every channel)
    issue(0);
    convert_commit(0, 0);
    stats(0);
    for (int it = 0; it < nblk; ++it) {
        const int buf = it & 1;
        lds_barrier();  // this block's gates and values are visible
        const float tot = scan_operand(buf, lgs);
        lds_barrier();  // this block's key operand is visible
        if (it + 1 < nblk) {
            convert_commit(it + 1, buf ^ 1);
            contract(buf);
            stats(buf ^ 1);
        } else {
            contract(buf);
        }
        lgs += tot;
    }
    const size_t rec = size_t(D) * D + D;
    float* dst = p.carry + ((size_t(b) * p.H_kv + h) * size_t(p.n_seg - 1) + s) * rec;
#pragma unroll
    for (int a = 0; a < RTW; ++a)
#pragma unroll
        for (int tt = 0; tt < CTW; ++tt)
#pragma unroll
            for (int r = 0; r < 4; ++r)
                dst[(16 * (rt0 + a) + 4 * g + r) * D + 16 * (ct0 + tt) + col] = acc[a * CTW + tt][r];
    if (tid < D) dst[size_t(D) * D + tid] = lgs;
}

// ------------------------------------------------------------------ P2
// One thread per state element. The decays of up to BATCH segment records
// come with one load per wave (lane u holds record u's, exponentiated once
// and read out with a lane read); the record elements are all loaded, in
// order, before the first multiply-add, so each step waits only for its own
// record while the stores of the steps before it drain.
template <int D>
__global__ __launch_bounds__(256) void carry_scan_kernel(float* __restrict__ carry, const float* __restrict__ S0,
                                                          int64_t n_seg, int H_kv) {
    constexpr int BATCH = 32;
    static_assert(D % 64 == 0, "a wave covers one row of the state, or half of it");
    const int e = blockIdx.x * 256 + threadIdx.x;  // D*D is a multiple of 256
    const int lane = threadIdx.x & 63;
    const int h = blockIdx.y;
    const int64_t b = blockIdx.z;
    const size_t rec = size_t(D) * D + D;
    float* base = carry + (size_t(b) * H_kv + h) * size_t(n_seg - 1) * rec;
    const int r = e / D;  // the same for every lane of a wave
    const int64_t last = n_seg - 2;
    float acc = S0 ? S0[(size_t(b) * H_kv + h) * D * D + e] : 0.f;
    for (int64_t s0 = 0; s0 < n_seg - 1; s0 += BATCH) {
        const int64_t sl = s0 + lane < last ? s0 + lane : last;
        const float dec = fast_exp2(base[sl * rec + size_t(D) * D + r]);  // lane u: record s0 + u
        float Ls[BATCH];
#pragma unroll
        for (int u = 0; u < BATCH; ++u) {
            const int64_t sr = s0 + u < last ? s0 + u : last;  // past the last record it is read again
            Ls[u] = base[sr * rec + e];
            __builtin_amdgcn_sched_barrier(0);  // issue order = record order
        }
#pragma unroll
        for (int u = 0; u < BATCH; ++u) {
            if (s0 + u < n_seg - 1) {
                acc = readlane_f(dec, u) * acc + Ls[u];
                base[(s0 + u) * rec + e] = acc;
            }
        }
    }
}

// ------------------------------------------------------------------ P3
template <typename T, int D, int GATE>
struct ItemCtx {
    const T* q;
    T* o;
    int64_t row0;      // b * T + t0 (token row of the chunk start)
    int H_q;
    int hq;
    int nvalid;
    int window;
    int npv;           // keys of the previous-chunk slot that exist (64, or fewer at the sequence start)
    float alpha;
    int cur;
    const T* sink_k;  // this key/value head's sink tokens [n_sink][D]
    const T* sink_v;
    int n_sink;
    // global halo (fp32, d = 128): the previous chunk's K and V rows in
    // global memory (row j at kprv[j * prv_stride]) and the state operand
    // S'^T [D][D] of this chunk
    const T* kprv;
    const T* vprv;
    int64_t prv_stride;
    const float* opg;
};

// One wave computes the outputs of 32 query rows (query tiles QA and QB of the
// chunk) of one query head over all of d_v. The pairs (0, 3) and (1, 2) have
// the same amount of intra-chunk work. Every LDS operand fragment it
// reads (key tiles, K~, S'^T, V^T) feeds both query tiles.
// Scores are kept per (query tile s, key tile kt) in the accumulator layout:
// lane (col, g) holds keys 16 kt + 4 g + r for query 16 I_s + col.
// The intra-chunk scores (keys of this chunk, j <= i) and the window weights
// (keys i-w < j <= i) multiply the same V rows, so they are added into one
// operand per key tile before the product with V.
// Raw query fragments of two query tiles: lane (col, g) holds row 16 I_s + col,
// elements KSTEP k + KPL g .. + KPL - 1. Rows past the end are zero.
template <typename T, int D>
struct QFrags {
    typename Mfma<T>::frag f[2][D / Mfma<T>::KSTEP];
};

// The output block a wave computes after the current one: the next item of
// this chunk, else the wave's first item of the next chunk. Its query
// fragments are loaded as soon as the current block's are no longer needed,
// so the load overlaps the rest of the current block and the chunk phases
// in between.
struct QNext {
    int64_t row0;  // b * T + t0 of that block's chunk
    int hq;
    int pair;      // 0: query tiles (0, 3), 1: (1, 2)
    int nvalid;
    bool any;      // false: this wave has no further block
};

// Next block of a wave that is on item `it` of chunk `c` (chunks end at c_end).
__device__ __forceinline__ QNext next_block(int it, int wave, int n_items, int n_rep, int h, int64_t b, int64_t T,
                                            int64_t c, int64_t c_end) {
    QNext nx;
    const bool same = it + kPWaves < n_items;
    const int itn = same ? it + kPWaves : wave;
    const int64_t cn = same ? c : c + 1;
    const int64_t tn = cn * kChunk;
    nx.any = cn < c_end;
    nx.row0 = b * T + tn;
    nx.nvalid = T - tn < kChunk ? int(T - tn) : kChunk;
    nx.hq = h * n_rep + itn % n_rep;
    nx.pair = itn / n_rep;
    return nx;
}

// UNCOND: rows past the end read row 0 of the chunk (always a token) and
// are zeroed where they are used, so the loads carry no branch: the compiler
// then counts them exactly, and waits on the vector memory counter for
// earlier loads do not also wait for these.
template <typename T, int D, bool UNCOND = false>
__device__ __forceinline__ void load_q_block(QFrags<T, D>& qf, const T* q, int64_t row0, int H_q, int hq, int qa,
                                             int qb, int nvalid, int lane) {
    typedef Mfma<T> M;
    const int col = lane & 15, g = lane >> 4;
#pragma unroll
    for (int s = 0; s < 2; ++s) {
        const int i = 16 * (s == 0 ? qa : qb) + col;
        const bool ok = i < nvalid;
        const T* qrow = q + ((row0 + (ok ? i : 0)) * H_q + hq) * D;
#pragma unroll
        for (int k = 0; k < D / M::KSTEP; ++k) {
            if constexpr (UNCOND) {
                static_assert(sizeof(T) == 2, "unconditional query loads are bf16 only");
                qf.f[s][k] = __builtin_bit_cast(typename M::frag,
                                                *reinterpret_cast<const uint4*>(qrow + M::KSTEP * k + M::KPL * g));
            } else if constexpr (sizeof(T) == 2) {
                const uint4 u = ok ? *reinterpret_cast<const uint4*>(qrow + M::KSTEP * k + M::KPL * g)
                                   : make_uint4(0, 0, 0, 0);
                qf.f[s][k] = __builtin_bit_cast(typename M::frag, u);
            } else {
                qf.f[s][k] = ok ? reinterpret_cast<const float*>(qrow)[M::KSTEP * k + g] : 0.0f;
            }
        }
    }
}

// Inter-chunk operand fragment read from the resident fp32 state: row dv,
// channels k0 .. k0 + KPL - 1, scaled by 2^mref (vector gate), packed to T.
template <typename T, int D, int GATE>
__device__ __forceinline__ typename Mfma<T>::frag resident_frag(const Smem<T, D, GATE, true>& sm, int dv, int k0) {
    typedef Layout<T, D, GATE, true> L;
    typedef Mfma<T> M;
    const float* src = sm.S32 + dv * L::SP + k0;
    float x[M::KPL];
    if constexpr (M::KPL == 8) {
        const float4 a = *reinterpret_cast<const float4*>(src);
        const float4 b = *reinterpret_cast<const float4*>(src + 4);
        x[0] = a.x; x[1] = a.y; x[2] = a.z; x[3] = a.w;
        x[4] = b.x; x[5] = b.y; x[6] = b.z; x[7] = b.w;
        if (GATE) {
            const float4 ea = *reinterpret_cast<const float4*>(sm.emref + k0);
            const float4 eb = *reinterpret_cast<const float4*>(sm.emref + k0 + 4);
            x[0] *= ea.x; x[1] *= ea.y; x[2] *= ea.z; x[3] *= ea.w;
            x[4] *= eb.x; x[5] *= eb.y; x[6] *= eb.z; x[7] *= eb.w;
        }
    } else {
        x[0] = GATE ? src[0] * sm.emref[k0] : src[0];
    }
    return M::pack(x);
}

template <typename T, int D, int GATE, int QA, int QB, bool SINK>
__device__ __forceinline__ void output_block(const Smem<T, D, GATE, true>& sm, const ItemCtx<T, D, GATE>& x,
                                             int lane, QFrags<T, D>& qin, const QNext& nx) {
    typedef Layout<T, D, GATE, true> L;
    typedef Mfma<T> M;
    typedef typename M::frag Frag;
    constexpr int KS = D / M::KSTEP;
    constexpr int KPL = M::KPL;
    constexpr int NT = D / 16;
    constexpr bool BF = sizeof(T) == 2;
    constexpr int QTS[2] = {QA, QB};    // query tiles of s = 0, 1 (relative to the chunk start)
    constexpr int KTMIN = (QA < QB ? QA : QB) - 4;  // key tiles KTMIN .. KTMAX
    constexpr int KTMAX = QA > QB ? QA : QB;
    constexpr int NKT = KTMAX - KTMIN + 1;
    constexpr int GMIN = (KTMIN - (KTMIN & 1)) / 2;  // aligned 32-key groups: key tiles 2G, 2G + 1
    constexpr int NG = KTMAX / 2 - GMIN + 1;
    // key tile kt is in query tile s's window range
    auto inr = [](int s, int kt) { return kt >= QTS[s] - 4 && kt <= QTS[s]; };
    const int col = lane & 15, g = lane >> 4;
    const int dl = col - 4 * g;         // i - j = 16 (I - kt) + dl - r inside a tile pair
    const T* Kcur = sm.K + x.cur * 64 * L::DP;
    const T* Kprv = sm.K + (L::NSLOT == 2 ? x.cur ^ 1 : 0) * 64 * L::DP;
    const T* Vcur = sm.Vt + x.cur * L::V_ELEMS;
    const T* Vprv = sm.Vt + (L::NSLOT == 2 ? x.cur ^ 1 : 0) * L::V_ELEMS;
    // row of the previous chunk's key tile kt (kt < 0): LDS, or global memory
    // with the global halo
    auto prev_krow = [&](int kt) -> const T* {
        if constexpr (L::HG) return x.kprv + (16 * kt + 64 + col) * x.prv_stride;
        else return Kprv + (16 * kt + 64 + col) * L::DP;
    };
    const int nbad = GATE ? *sm.nbad : 0;
    const bool exact = GATE ? false : (*sm.exact != 0);
    const bool full_window = x.window >= 64;

    int i_loc[2];
    bool row_ok[2];
#pragma unroll
    for (int s = 0; s < 2; ++s) {
        i_loc[s] = 16 * QTS[s] + col;
        row_ok[s] = i_loc[s] < x.nvalid;
    }
    // Per-lane values of the rare bad-channel paths, re-derived inside them
    // from a lane index the compiler cannot move, so that they are not
    // computed at the top of the block and kept live (or spilled) through it.
    struct RareLane {
        int il;       // query row of tile s
        bool ok;
        const T* qr;  // its raw query row
        int g;
    };
    auto rare_lane = [&](int s) -> RareLane {
        RareLane rl;
        const int lo = opaque_lane(lane);
        rl.il = 16 * QTS[s] + (lo & 15);
        rl.ok = rl.il < x.nvalid;
        rl.qr = x.q + ((x.row0 + (rl.ok ? rl.il : 0)) * x.H_q + x.hq) * D;
        rl.g = lo >> 4;
        return rl;
    };

    // ---- query rows: raw fragments (window operand). The recurrence operand
    // (built below) is e^(q - max) times the gate factor; the softmax
    // normaliser of phi(q) and alpha are applied to the products instead.
    Frag qr[2][KS], qt[2][KS];
    float qmax[2], qinv[2];
#pragma unroll
    for (int s = 0; s < 2; ++s)
#pragma unroll
        for (int k = 0; k < KS; ++k) {
            // without a resident state, bf16 query rows past the end arrive
            // unconditionally loaded (row 0) and are zeroed here
            if constexpr (L::SLDS || !BF) qr[s][k] = qin.f[s][k];
            else qr[s][k] = row_ok[s] ? qin.f[s][k] : M::zero();
        }
    auto qval = [&](int s, int k, int i) -> float {
        if constexpr (BF) {
            const uint4 u = __builtin_bit_cast(uint4, qr[s][k]);
            const uint32_t w = (i >> 1) == 0 ? u.x : (i >> 1) == 1 ? u.y : (i >> 1) == 2 ? u.z : u.w;
            return __uint_as_float((i & 1) ? (w & 0xffff0000u) : (w << 16));
        } else {
            return __builtin_bit_cast(float, qr[s][k]);
        }
    };
#pragma unroll
    for (int s = 0; s < 2; ++s) {
        float m = -INFINITY;
#pragma unroll
        for (int k = 0; k < KS; ++k)
#pragma unroll
            for (int i = 0; i < KPL; ++i) m = fmaxf(m, qval(s, k, i));
        qmax[s] = group4_max(m);
    }

    // ---- window scores over key tiles kt = KTMIN + u; query tile I uses
    // kt = I - 4 .. I. A key is valid when 0 <= i - j < window. With the full
    // 64-key window and a previous chunk (the common case, compiled on its
    // own) only the diagonal tile (kt = I) and the window's first tile
    // (kt = I - 4) are partial; otherwise tiles may be dead as a whole.
    // Maxima are taken on the raw products; the 1/sqrt(d) scale is applied
    // inside the exponent.
    float sc[2][NKT][4];
    float ss[2][4];  // sink tokens: lane (col, g) holds sinks 4 g + r of query col
    const float lscale = kLog2e * rsqrtf(static_cast<float>(D));
    auto window_scores = [&](auto fast_c) {
        constexpr bool FAST = decltype(fast_c)::value;
        float lmax[2] = {-INFINITY, -INFINITY};
        const unsigned w = FAST ? 64u : static_cast<unsigned>(x.window);
        // FAST (every tile in range is live): the next tile's key fragments
        // are requested before this tile's MFMAs
        Frag kbuf[2][KS];
        auto load_tile = [&](int kt, Frag* dst) {
            const T* krow = kt >= 0 ? Kcur + (16 * kt + col) * L::DP : prev_krow(kt);
#pragma unroll
            for (int k = 0; k < KS; ++k) dst[k] = M::load(krow + M::KSTEP * k + KPL * g);
        };
        if constexpr (FAST) load_tile(KTMIN, kbuf[0]);
#pragma unroll
        for (int u = 0; u < NKT; ++u) {
            const int kt = KTMIN + u;
            if constexpr (FAST) {
                if (u + 1 < NKT) load_tile(kt + 1, kbuf[(u + 1) & 1]);
            }
            bool live[2];
#pragma unroll
            for (int s = 0; s < 2; ++s)
                live[s] = inr(s, kt) &&
                          (FAST || ((kt >= 0 || x.npv > 0) && (16 * kt + 15 > 16 * QTS[s] - x.window)));
            if (live[0] || live[1]) {
                const T* krow = kt >= 0 ? Kcur + (16 * kt + col) * L::DP : prev_krow(kt);
                f32x4_t d4[2] = {zero4(), zero4()};
#pragma unroll
                for (int k = 0; k < KS; ++k) {
                    const Frag a = FAST ? kbuf[u & 1][k] : M::load(krow + M::KSTEP * k + KPL * g);
#pragma unroll
                    for (int s = 0; s < 2; ++s)
                        if (live[s]) d4[s] = M::mma(a, qr[s][k], d4[s]);
                }
#pragma unroll
                for (int s = 0; s < 2; ++s) {
                    if (!inr(s, kt)) continue;
                    if (!live[s]) {
#pragma unroll
                        for (int r = 0; r < 4; ++r) sc[s][u][r] = -INFINITY;
                        continue;
                    }
                    const int dt = 16 * (QTS[s] - kt);  // 16 (I - kt), compile-time
                    const bool before = !FAST && kt < 0 && x.npv < 64;  // keys before the sequence start
                    const bool partial = (kt == QTS[s] - 4) || (kt == QTS[s]) || !(FAST || full_window) || before;
#pragma unroll
                    for (int r = 0; r < 4; ++r) {
                        float v = d4[s][r];
                        if (partial)
                            v = (static_cast<unsigned>(dt + dl - r) < w && (!before || 16 * kt + 4 * g + r >= -x.npv))
                                    ? v : -INFINITY;
                        sc[s][u][r] = v;
                        lmax[s] = fmaxf(lmax[s], v);
                    }
                }
            } else if (!FAST) {
#pragma unroll
                for (int s = 0; s < 2; ++s)
                    if (inr(s, kt)) {
#pragma unroll
                        for (int r = 0; r < 4; ++r) sc[s][u][r] = -INFINITY;
                    }
            }
            __builtin_amdgcn_sched_barrier(0);  // at most two key tiles' fragments in flight
        }
        if constexpr (SINK) {
            // sink scores: the sink keys (rows past n_sink repeat the last one
            // and are masked) against both query tiles
            const T* srow = x.sink_k + (col < x.n_sink ? col : x.n_sink - 1) * D + KPL * g;
            f32x4_t d4[2] = {zero4(), zero4()};
#pragma unroll
            for (int k = 0; k < KS; ++k) {
                const Frag a = M::load(srow + M::KSTEP * k);
                d4[0] = M::mma(a, qr[0][k], d4[0]);
                d4[1] = M::mma(a, qr[1][k], d4[1]);
            }
#pragma unroll
            for (int s = 0; s < 2; ++s)
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const float v = 4 * g + r < x.n_sink ? d4[s][r] : -INFINITY;
                    ss[s][r] = v;
                    lmax[s] = fmaxf(lmax[s], v);
                }
        }
#pragma unroll
        for (int s = 0; s < 2; ++s) {
            const float m = group4_max(lmax[s]) * lscale;  // the diagonal key is always valid
            float sum = 0.f;
#pragma unroll
            for (int u = QTS[s] - 4 - KTMIN; u <= QTS[s] - KTMIN; ++u)
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const float e = fast_exp2(fmaf(sc[s][u][r], lscale, -m));  // exp2(-inf) = 0 for masked keys
                    sc[s][u][r] = e;
                    sum += e;
                }
            if constexpr (SINK) {
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const float e = fast_exp2(fmaf(ss[s][r], lscale, -m));
                    ss[s][r] = e;
                    sum += e;
                }
            }
            const float ps = (1.0f - x.alpha) * fast_rcp(group4_sum(sum));
#pragma unroll
            for (int u = QTS[s] - 4 - KTMIN; u <= QTS[s] - KTMIN; ++u)
#pragma unroll
                for (int r = 0; r < 4; ++r) sc[s][u][r] *= ps;
            if constexpr (SINK) {
#pragma unroll
                for (int r = 0; r < 4; ++r) ss[s][r] *= ps;
            }
        }
    };
    if (x.npv == 64 && full_window) window_scores(std::true_type{});
    else window_scores(std::false_type{});

    // recurrence operand (built after the window scores so qr can retire)
#pragma unroll
    for (int s = 0; s < 2; ++s) {
        float sum = 0.f;
        const float mq = qmax[s] * kLog2e;
#pragma unroll
        for (int k = 0; k < KS; ++k) {
            float tmp[KPL];
            float f[KPL];
            if (GATE) {
                const float* fr = sm.F + i_loc[s] * L::FP + M::KSTEP * k + KPL * g;
#pragma unroll
                for (int i = 0; i < KPL; i += 4) {
                    const float4 f4 = *reinterpret_cast<const float4*>(fr + i);
                    f[i] = f4.x;
                    if (i + 1 < KPL) f[i + 1] = f4.y;
                    if (i + 2 < KPL) f[i + 2] = f4.z;
                    if (i + 3 < KPL) f[i + 3] = f4.w;
                }
            }
#pragma unroll
            for (int i = 0; i < KPL; ++i) {
                const float e = fast_exp2(fmaf(qval(s, k, i), kLog2e, -mq));
                sum += e;
                if (GATE) {
                    const int ch = M::KSTEP * k + KPL * g + i;
                    float fi = f[i];
                    if (nbad && ((sm.badmask[ch >> 5] >> (ch & 31)) & 1u)) fi = 0.0f;
                    tmp[i] = e * fi;
                } else {
                    tmp[i] = e;
                }
            }
            qt[s][k] = M::pack(tmp);
        }
        qinv[s] = (GATE ? 1.0f : x.alpha) * fast_rcp(group4_sum(sum));
    }
    // the raw query fragments are dead: load the next block's into them
    if (nx.any)
        load_q_block<T, D>(qin, x.q, nx.row0, x.H_q, nx.hq, nx.pair == 0 ? 0 : 1, nx.pair == 0 ? 3 : 2, nx.nvalid, lane);

    // ---- intra-chunk scores on key tiles J = 0 .. I (query tile I), added into the same
    // per-key-tile operand. Tiles below the diagonal are whole; the diagonal
    // tile keeps j <= i. Scalar gate: the decay 2^(b_i - b_j) is split into
    // 2^(b_i - m) (here) and 2^(m - b_j) (in the key operand), or applied per
    // pair when the chunk's decay range is too wide to split.
    // The two waves sharing a SIMD run blocks (0, 3) and (1, 2); the younger
    // one, on (1, 2), loses issue arbitration and would finish alone, so it
    // takes a higher issue priority from here to the end of the block.
    if (QA == 1) __builtin_amdgcn_s_setprio(1);
    float bq[2] = {0.f, 0.f};
    float qsc[2];
    float4 bk[KTMAX + 1];
#pragma unroll
    for (int s = 0; s < 2; ++s) {
        if (GATE == 0) bq[s] = sm.b2s[i_loc[s]];
        qsc[s] = qinv[s] * ((GATE == 0 && !exact) ? fast_exp2(bq[s] - sm.mref[0]) : 1.0f);
    }
    if (GATE == 0 && exact) {
#pragma unroll
        for (int J = 0; J <= KTMAX; ++J) bk[J] = *reinterpret_cast<const float4*>(sm.b2s + 16 * J + 4 * g);
    }
    // the next key tile's operand fragments are requested before this tile's MFMAs
    Frag ibuf[2][KS];
    auto load_itile = [&](int J, Frag* dst) {
#pragma unroll
        for (int k = 0; k < KS; ++k) dst[k] = M::load(sm.Kb + (16 * J + col) * L::DP + M::KSTEP * k + KPL * g);
    };
    load_itile(0, ibuf[0]);
#pragma unroll
    for (int J = 0; J <= KTMAX; ++J) {
        if (J + 1 <= KTMAX) load_itile(J + 1, ibuf[(J + 1) & 1]);
        f32x4_t d4[2] = {zero4(), zero4()};
#pragma unroll
        for (int k = 0; k < KS; ++k) {
            const Frag a = ibuf[J & 1][k];
#pragma unroll
            for (int s = 0; s < 2; ++s)
                if (J <= QTS[s]) d4[s] = M::mma(a, qt[s][k], d4[s]);
        }
#pragma unroll
        for (int s = 0; s < 2; ++s) {
            if (J > QTS[s]) continue;
#pragma unroll
            for (int r = 0; r < 4; ++r) d4[s][r] *= qsc[s];
            if (nbad) {
                const RareLane rl = rare_lane(s);
                for (int nb = 0; nb < nbad; ++nb) {
                    const int c = sm.badlist[nb];
                    const float qc = rl.ok ? to_f32(rl.qr[c]) : 0.0f;
                    const float coef = x.alpha * fast_exp2((qc - qmax[s]) * kLog2e) * qinv[s];
                    const float b2i = sm.F[rl.il * L::FP + c];
#pragma unroll
                    for (int r = 0; r < 4; ++r) {
                        const int j = 16 * J + 4 * rl.g + r;
                        const float phik = sm.kinv[j] * fast_exp2((to_f32(Kcur[j * L::DP + c]) - sm.kmax[j]) * kLog2e);
                        const float term = coef * phik * fast_exp2(fminf(b2i - sm.F[j * L::FP + c], 0.0f));
                        d4[s][r] += j <= rl.il ? term : 0.0f;
                    }
                }
            }
            if (GATE == 0 && exact) {
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const float bj = r == 0 ? bk[J].x : r == 1 ? bk[J].y : r == 2 ? bk[J].z : bk[J].w;
                    d4[s][r] *= fast_exp2(fminf(bq[s] - bj, 0.0f));
                }
            }
            const int u = J - KTMIN;
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                float val = d4[s][r];
                if (J == QTS[s]) val = dl >= r ? val : 0.0f;  // diagonal tile: j <= i
                sc[s][u][r] += val;
            }
        }
        __builtin_amdgcn_sched_barrier(0);
    }

    // ---- bf16: pack the combined scores of the aligned key-tile pairs
    // (kt = 2G, 2G + 1); tiles outside query tile s's range are 0.
    auto scv = [&](int s, int kt, int r) -> float {
        const int u = kt - KTMIN;
        return inr(s, kt) ? sc[s][u < 0 ? 0 : u][r] : 0.0f;
    };
    Frag pf[2][NG];
    if constexpr (BF) {
#pragma unroll
        for (int s = 0; s < 2; ++s)
#pragma unroll
            for (int G = 0; G < NG; ++G) {
                const int kt0 = 2 * (GMIN + G);
                if (!inr(s, kt0) && !inr(s, kt0 + 1)) continue;
                float v8[8];
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    v8[r] = scv(s, kt0, r);
                    v8[4 + r] = scv(s, kt0 + 1, r);
                }
                pf[s][G] = M::pack(v8);
            }
    }
    // sink probabilities as the operand of a 32-key group whose upper 16 keys are zero
    Frag pfs[2];
    if constexpr (SINK && BF) {
#pragma unroll
        for (int s = 0; s < 2; ++s) {
            const float v8[8] = {ss[s][0], ss[s][1], ss[s][2], ss[s][3], 0.f, 0.f, 0.f, 0.f};
            pfs[s] = M::pack(v8);
        }
    }
    float inter_scale[2];
#pragma unroll
    for (int s = 0; s < 2; ++s) inter_scale[s] = GATE == 0 ? qinv[s] * fast_exp2(bq[s]) : qinv[s];

    // ---- one 16-wide slice of d_v at a time: inter + (intra + window), store
    T* orow[2];
#pragma unroll
    for (int s = 0; s < 2; ++s) orow[s] = x.o + ((x.row0 + i_loc[s]) * x.H_q + x.hq) * D + 4 * g;
#pragma unroll 1
    for (int t = 0; t < NT; ++t) {
        f32x4_t acc[2] = {zero4(), zero4()};
        // Resident state, bf16, scalar gate: every LDS operand of this slice
        // (the state pieces and the value fragments) is requested before the
        // first MFMA, so the slice waits for LDS once instead of twice.
        constexpr bool PRE = L::SLDS && BF && GATE == 0;
        float4 sraw[PRE ? 2 * KS : 1];
        Frag vfr[NG];
        if constexpr (PRE) {
#pragma unroll
            for (int k = 0; k < KS; ++k) {
                const float* src = sm.S32 + (16 * t + col) * L::SP + M::KSTEP * k + KPL * g;
                sraw[2 * k] = *reinterpret_cast<const float4*>(src);
                sraw[2 * k + 1] = *reinterpret_cast<const float4*>(src + 4);
            }
#pragma unroll
            for (int G = 0; G < NG; ++G) {
                const int kt = 2 * (GMIN + G);
                if (!(inr(0, kt) || inr(0, kt + 1) || inr(1, kt) || inr(1, kt + 1))) continue;
                vfr[G] = kt >= 0 ? load_key_frag(Vcur, L::VP, 16 * kt, 16 * t, lane)
                                 : load_key_frag(Vprv, L::VP, 16 * (kt + 4), 16 * t, lane);
            }
            __builtin_amdgcn_sched_barrier(0);
        }
#pragma unroll
        for (int k = 0; k < KS; ++k) {
            Frag a;
            if constexpr (PRE) {
                const float x[8] = {sraw[2 * k].x, sraw[2 * k].y, sraw[2 * k].z, sraw[2 * k].w,
                                    sraw[2 * k + 1].x, sraw[2 * k + 1].y, sraw[2 * k + 1].z, sraw[2 * k + 1].w};
                a = M::pack(x);
            } else if constexpr (L::SLDS) {
                a = resident_frag(sm, 16 * t + col, M::KSTEP * k + KPL * g);
            } else if constexpr (L::HG) {
                a = M::load(reinterpret_cast<const T*>(x.opg) + (16 * t + col) * D + M::KSTEP * k + KPL * g);
            } else {
                a = M::load(sm.St + (16 * t + col) * L::DP + M::KSTEP * k + KPL * g);
            }
            acc[0] = M::mma(a, qt[0][k], acc[0]);
            acc[1] = M::mma(a, qt[1][k], acc[1]);
        }
#pragma unroll
        for (int s = 0; s < 2; ++s) {
            acc[s] *= inter_scale[s];
            if (nbad) {
                const RareLane rl = rare_lane(s);
                for (int nb = 0; nb < nbad; ++nb) {
                    const int c = sm.badlist[nb];
                    const float qc = rl.ok ? to_f32(rl.qr[c]) : 0.0f;
                    const float bad_q =
                        x.alpha * fast_exp2((qc - qmax[s]) * kLog2e) * qinv[s] * fast_exp2(sm.F[rl.il * L::FP + c]);
#pragma unroll
                    for (int r = 0; r < 4; ++r)
                        acc[s][r] += bad_q * (L::SLDS ? sm.S32[(16 * t + 4 * rl.g + r) * L::SP + c]
                                              : L::HG ? x.opg[(16 * t + 4 * rl.g + r) * D + c]
                                                      : to_f32(sm.St[(16 * t + 4 * rl.g + r) * L::DP + c]));
                }
            }
        }
        if constexpr (BF) {
            // key tiles (2G, 2G + 1) form one aligned 32-key group
#pragma unroll
            for (int G = 0; G < NG; ++G) {
                const int kt = 2 * (GMIN + G);
                bool gl[2];
#pragma unroll
                for (int s = 0; s < 2; ++s) gl[s] = inr(s, kt) || inr(s, kt + 1);
                if (!gl[0] && !gl[1]) continue;
                Frag a;
                if constexpr (L::SLDS && GATE == 0) a = vfr[G];
                else a = kt >= 0 ? load_key_frag(Vcur, L::VP, 16 * kt, 16 * t, lane)
                                 : load_key_frag(Vprv, L::VP, 16 * (kt + 4), 16 * t, lane);
#pragma unroll
                for (int s = 0; s < 2; ++s)
                    if (gl[s]) acc[s] = M::mma(a, pf[s][G], acc[s]);
            }
        } else {
            const T* vrow_c = Vcur + (16 * t + col) * L::JP;
            const T* vrow_p = Vprv + (16 * t + col) * L::JP;
#pragma unroll
            for (int u = 0; u < NKT; ++u) {
                const int kt = KTMIN + u;
                const int kk = kt >= 0 ? kt : kt + 4;
                float pr[4];
                if (L::HG && kt < 0) {
                    // keys 16 kk + 4 g + r of the previous chunk, channel 16 t + col
                    const T* vg = x.vprv + (16 * kk + 4 * g) * x.prv_stride + 16 * t + col;
#pragma unroll
                    for (int r = 0; r < 4; ++r)
                        pr[r] = (x.npv > 0 && (inr(0, kt) || inr(1, kt))) ? to_f32(vg[r * x.prv_stride]) : 0.0f;
                } else {
                    const T* base = kt >= 0 ? vrow_c : vrow_p;
                    const float4 pv = *reinterpret_cast<const float4*>(base + 32 * (kk >> 1) + 8 * g + 4 * (kk & 1));
                    pr[0] = pv.x;
                    pr[1] = pv.y;
                    pr[2] = pv.z;
                    pr[3] = pv.w;
                }
#pragma unroll
                for (int s = 0; s < 2; ++s)
                    if (inr(s, kt)) {
#pragma unroll
                        for (int r = 0; r < 4; ++r)
                            acc[s] = M::mma(__builtin_bit_cast(Frag, pr[r]), __builtin_bit_cast(Frag, sc[s][u][r]), acc[s]);
                    }
            }
        }
        if constexpr (SINK) {
            // sink values: lane (col, g) takes channel 16 t + col of sinks 4 g + r
            const T* sv = x.sink_v + 16 * t + col;
            float vs[4];
#pragma unroll
            for (int r = 0; r < 4; ++r) vs[r] = to_f32(sv[(4 * g + r < x.n_sink ? 4 * g + r : x.n_sink - 1) * D]);
            if constexpr (BF) {
                const Frag a = __builtin_bit_cast(Frag, make_uint4(pack_bf16x2(vs[0], vs[1]), pack_bf16x2(vs[2], vs[3]), 0u, 0u));
                acc[0] = M::mma(a, pfs[0], acc[0]);
                acc[1] = M::mma(a, pfs[1], acc[1]);
            } else {
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    acc[0] = M::mma(__builtin_bit_cast(Frag, vs[r]), __builtin_bit_cast(Frag, ss[0][r]), acc[0]);
                    acc[1] = M::mma(__builtin_bit_cast(Frag, vs[r]), __builtin_bit_cast(Frag, ss[1][r]), acc[1]);
                }
            }
        }
#pragma unroll
        for (int s = 0; s < 2; ++s)
            if (row_ok[s]) {
                T* dst = orow[s] + 16 * t;
                if constexpr (BF) {
                    *reinterpret_cast<uint2*>(dst) =
                        make_uint2(pack_bf16x2(acc[s][0], acc[s][1]), pack_bf16x2(acc[s][2], acc[s][3]));
                } else {
                    *reinterpret_cast<float4*>(dst) = make_float4(acc[s][0], acc[s][1], acc[s][2], acc[s][3]);
                }
            }
    }
}

template <typename T, int D, int GATE, bool SINK>
__global__ __launch_bounds__(kPThreads) void prefill_output_kernel(PrefillParams p) {
    typedef Layout<T, D, GATE, true> L;
    __shared__ __align__(16) char smem[L::TOTAL];
    const Smem<T, D, GATE, true> sm(smem);
    constexpr int TPT = 64 / (kPThreads / D);

    const int s = blockIdx.x;
    const int h = blockIdx.y;
    const int64_t b = blockIdx.z;
    const int wave = threadIdx.x >> 6;
    const int64_t row_stride = int64_t(p.H_kv) * D;
    const T* kbase = static_cast<const T*>(p.k) + (b * p.T * p.H_kv + h) * D;
    const T* vbase = static_cast<const T*>(p.v) + (b * p.T * p.H_kv + h) * D;
    const int H_q = p.H_kv * p.n_rep;
    const size_t rec = size_t(D) * D + D;

    if constexpr (L::HG) {
        if (p.rec_mode) {
            // Segment-state record of segment s (every segment but the last):
            // the state reached from zero over its chunks and the log2 decay
            // of the whole segment per d_k row, as the segment-state kernels
            // write them for the other configurations.
            const int64_t cb = int64_t(s) * p.cps;
            const int64_t ce = cb + p.cps < p.n_chunks ? cb + p.cps : p.n_chunks;
            ChunkRegs<T, D> cr;
            load_chunk_issue<T, D>(cr, kbase, vbase, row_stride, cb * kChunk,
                                   p.T - cb * kChunk < kChunk ? int(p.T - cb * kChunk) : kChunk);
            f32x4_t acc[StateTiles<D>::TPW];
#pragma unroll
            for (int u = 0; u < StateTiles<D>::TPW; ++u) acc[u] = zero4();
            float lg = 0.f;
            load_chunk_commit(sm, 0, cr);
            for (int64_t c = cb; c < ce; ++c) {
                const int64_t t0 = c * kChunk;
                const int nvalid = p.T - t0 < kChunk ? int(p.T - t0) : kChunk;
                if (c + 1 < ce) {
                    const int64_t t1 = t0 + kChunk;
                    load_chunk_issue<T, D>(cr, kbase, vbase, row_stride, t1, p.T - t1 < kChunk ? int(p.T - t1) : kChunk);
                }
                if (threadIdx.x == 0) *sm.nbad = 0;
                if (threadIdx.x < D / 32) sm.badmask[threadIdx.x] = 0u;
                __syncthreads();
                float b2[TPT];
                gate_prep<T, D, GATE, true, TPT>(sm, 0, nvalid, p.alpha, b2);
                __syncthreads();
                state_advance(sm, 0, acc);
                if (threadIdx.x < D) lg += sm.blast[threadIdx.x];
                __syncthreads();
                if (c + 1 < ce) load_chunk_commit(sm, 0, cr);
            }
            float* dst = p.carry + ((size_t(b) * p.H_kv + h) * size_t(p.n_seg - 1) + s) * rec;
            store_state<D>(dst, acc);
            if (threadIdx.x < D) dst[size_t(D) * D + threadIdx.x] = lg;
            return;
        }
    }
    float* slot = p.state_slots + ((size_t(b) * p.H_kv + h) * size_t(p.n_seg) + s) * size_t(D) * D;
    float* opg = L::HG ? p.op_slots + ((size_t(b) * p.H_kv + h) * size_t(p.n_seg) + s) * size_t(D) * D : nullptr;
    const float* carry_in = s > 0 ? p.carry + ((size_t(b) * p.H_kv + h) * size_t(p.n_seg - 1) + (s - 1)) * rec
                            : p.S0 ? p.S0 + (size_t(b) * p.H_kv + h) * D * D : nullptr;
    // continuation: tokens already consumed, and how many of the 64 before the
    // first chunk exist (the ring holds the last min(pos, window))
    const int64_t pos_b = p.pos ? p.pos[b] : 0;
    const int npv0 = int(pos_b < p.window ? pos_b : p.window);
    const bool last_seg = s == p.n_seg - 1;

    const int64_t c_begin = int64_t(s) * p.cps;
    const int64_t c_end = c_begin + p.cps < p.n_chunks ? c_begin + p.cps : p.n_chunks;
    // K/V of the chunk about to be processed: the first one is loaded here,
    // together with the previous chunk (sliding window) and, with a resident
    // state, the state entering the segment; each following chunk is issued
    // before the previous chunk's output phase and stored to LDS after it.
    ChunkRegs<T, D> cr, cp;
    load_chunk_issue<T, D>(cr, kbase, vbase, row_stride, c_begin * kChunk,
                           p.T - c_begin * kChunk < kChunk ? int(p.T - c_begin * kChunk) : kChunk);
    if (L::HG) {
        // the previous chunk stays in global memory
    } else if (c_begin > 0) load_chunk_issue<T, D>(cp, kbase, vbase, row_stride, (c_begin - 1) * kChunk, kChunk);
    else if (npv0 > 0)
        load_ring_issue<T, D>(cp, static_cast<const T*>(p.ring_k) + (size_t(b) * p.H_kv + h) * p.window * D,
                              static_cast<const T*>(p.ring_v) + (size_t(b) * p.H_kv + h) * p.window * D, pos_b,
                              p.window, npv0);
    const int n_items = p.n_rep * 2;
    // query fragments of this wave's first output block (resident state:
    // each output block loads the next one's)
    QFrags<T, D> qpre;
    if (L::SLDS && wave < n_items) {
        const int pair = wave / p.n_rep;
        const int64_t t0 = c_begin * kChunk;
        load_q_block<T, D>(qpre, static_cast<const T*>(p.q), b * p.T + t0, H_q, h * p.n_rep + (wave % p.n_rep),
                           pair == 0 ? 0 : 1, pair == 0 ? 3 : 2, p.T - t0 < kChunk ? int(p.T - t0) : kChunk,
                           threadIdx.x & 63);
    }
    f32x4_t acc[StateTiles<D>::TPW];
    if constexpr (L::SLDS) load_state<D>(carry_in, acc);
    // global halo, continuation: the ring's tokens before the first chunk as
    // contiguous rows (zero before the sequence start), read after the
    // barrier below like the previous chunk of a later chunk
    T* halo_k = nullptr;
    T* halo_v = nullptr;
    if constexpr (L::HG) {
        if (c_begin == 0 && npv0 > 0) {
            halo_k = reinterpret_cast<T*>(p.halo) + (size_t(b) * p.H_kv + h) * 2 * 64 * D;
            halo_v = halo_k + 64 * D;
            const T* rk = static_cast<const T*>(p.ring_k) + (size_t(b) * p.H_kv + h) * p.window * D;
            const T* rv = static_cast<const T*>(p.ring_v) + (size_t(b) * p.H_kv + h) * p.window * D;
            for (int idx = threadIdx.x; idx < 64 * D; idx += kPThreads) {
                const int j = idx / D;
                const int64_t rr = j < 64 - npv0 ? -1 : (pos_b - 64 + j) % p.window;
                halo_k[idx] = rr >= 0 ? rk[rr * D + idx % D] : T(0);
                halo_v[idx] = rr >= 0 ? rv[rr * D + idx % D] : T(0);
            }
        }
    }
    if (L::HG) {
        load_chunk_commit(sm, 0, cr);
    } else {
        if (c_begin > 0 || npv0 > 0) load_chunk_commit(sm, int((c_begin + 1) & 1), cp);
        else zero_slot(sm, int((c_begin + 1) & 1));
        load_chunk_commit(sm, int(c_begin & 1), cr);
    }
    if constexpr (L::SLDS) {
        // Resident state: per chunk, gate statistics and the intra operand,
        // then the outputs (inter term from S entering the chunk), then the
        // state operand and the in-place state update.
        put_resident(sm, acc);
        __syncthreads();
        for (int64_t c = c_begin; c < c_end; ++c) {
            const int cur = int(c & 1);
            const int64_t t0 = c * kChunk;
            const int nvalid = p.T - t0 < kChunk ? int(p.T - t0) : kChunk;
            // Scalar gate: no barrier is needed here. scalar_gate_intra first
            // writes the key statistics, which the previous chunk no longer
            // reads after its last barrier, and writes dec, exact and the
            // intra operand only after a barrier of its own, which every wave
            // reaches after finishing the previous state update.
            if (GATE) {
                if (threadIdx.x == 0) *sm.nbad = 0;
                if (threadIdx.x < D / 32) sm.badmask[threadIdx.x] = 0u;
                __syncthreads();
            }
            float b2[TPT];
            if constexpr (GATE == 0) {
                scalar_gate_intra<T, D>(sm, cur, nvalid);
            } else {
                gate_stats<T, D, GATE, true, TPT>(sm, cur, nvalid, p.alpha, b2);
                __syncthreads();
                intra_key_operand<T, D, GATE, true, TPT>(sm, cur, b2);
            }
            __syncthreads();
            ItemCtx<T, D, GATE> x;
            x.q = static_cast<const T*>(p.q);
            x.o = static_cast<T*>(p.o);
            x.row0 = b * p.T + t0;
            x.H_q = H_q;
            x.nvalid = nvalid;
            x.window = p.window;
            x.npv = c > 0 ? 64 : npv0;
            x.alpha = p.alpha;
            x.sink_k = SINK ? static_cast<const T*>(p.sink_k) + size_t(h) * p.n_sink * D : nullptr;
            x.sink_v = SINK ? static_cast<const T*>(p.sink_v) + size_t(h) * p.n_sink * D : nullptr;
            x.n_sink = SINK ? p.n_sink : 0;
            x.cur = cur;
            // next chunk's K/V: in flight during the output phase
            if (c + 1 < c_end) {
                const int64_t t1 = t0 + kChunk;
                load_chunk_issue<T, D>(cr, kbase, vbase, row_stride, t1, p.T - t1 < kChunk ? int(p.T - t1) : kChunk);
            }
            for (int it = wave; it < n_items; it += kPWaves) {
                x.hq = h * p.n_rep + (it % p.n_rep);
                int lane = threadIdx.x & 63;
                asm volatile("" : "+v"(lane));  // keep lane-derived addresses inside the loop
                const int pair = it / p.n_rep;
                const QNext nx = next_block(it, wave, n_items, p.n_rep, h, b, p.T, c, c_end);
                if (pair == 0) output_block<T, D, GATE, 0, 3, SINK>(sm, x, lane, qpre, nx);
                else output_block<T, D, GATE, 1, 2, SINK>(sm, x, lane, qpre, nx);
                __builtin_amdgcn_s_setprio(0);
            }
            __syncthreads();
            if (c + 1 < c_end) load_chunk_commit(sm, cur ^ 1, cr);  // the previous chunk's slot is free now
            // Scalar gate (bf16): the state key operand phik_j 2^(b_last - b_j)
            // is the intra operand phik_j 2^(m - b_j) times the chunk constant
            // 2^(b_last - m), so the intra operand (token-major, read with
            // transposing loads in the same key order as V) is reused unless
            // this chunk takes the exact per-pair path.
            constexpr bool CAN_REUSE = GATE == 0 && L::VNAT;
            const bool reuse = CAN_REUSE && *sm.exact == 0;
            if (!reuse) state_key_operand<T, D, GATE, true, TPT>(sm, cur, nvalid, sm.blast, b2);
            __syncthreads();
            if constexpr (CAN_REUSE) {
                if (reuse) state_advance<T, D, GATE, true, true, true>(sm, cur, acc, fast_exp2(sm.blast[0] - sm.mref[0]));
                else state_advance<T, D, GATE, true, true>(sm, cur, acc);
            } else {
                state_advance<T, D, GATE, true, true>(sm, cur, acc);
            }
            if (c + 1 == c_end && last_seg) store_state<D>(p.S_T + (size_t(b) * p.H_kv + h) * D * D, acc);
            // the next chunk's first barrier orders these LDS reads before its gate scan
        }
        return;
    }
    // the state entering the segment goes to this workgroup's slot, which
    // every chunk then reloads (each lane reads back its own stores)
    load_state<D>(carry_in, acc);
    store_slot<D>(slot, acc);
    __syncthreads();
    for (int64_t c = c_begin; c < c_end; ++c) {
        const int cur = L::NSLOT == 2 ? int(c & 1) : 0;
        const int64_t t0 = c * kChunk;
        const int nvalid = p.T - t0 < kChunk ? int(p.T - t0) : kChunk;
        // Running state (entering this chunk), loaded now so its latency
        // overlaps the gate phase: nothing waits on it before the state phase
        // (the barriers up to there order LDS only, and vector memory
        // counters drain in order, so any earlier wait would include it).
        __builtin_amdgcn_sched_barrier(0);
        load_slot<D>(slot, acc);
        __builtin_amdgcn_sched_barrier(0);
        // Query fragments of this wave's first output block, in flight during
        // the state phases. bf16 issues them after the gate phase: their
        // address code waits on the vector memory counter (register reuse, a
        // spill reload), which at the chunk top would wait for the state.
        // fp32 issues them here (its fragment registers would otherwise be
        // live through the gate phase).
        constexpr bool LATE_Q = sizeof(T) == 2;
        auto issue_q = [&]() {
            int lane = threadIdx.x & 63;
            asm volatile("" : "+v"(lane));
            if constexpr (LATE_Q) {
                // every wave loads (a wave without an item loads item 0's
                // rows and never uses them), so no branch joins here
                const int it0 = wave < n_items ? wave : 0;
                const int pair = it0 / p.n_rep;
                load_q_block<T, D, true>(qpre, static_cast<const T*>(p.q), b * p.T + t0, H_q,
                                         h * p.n_rep + (it0 % p.n_rep), pair == 0 ? 0 : 1, pair == 0 ? 3 : 2, nvalid,
                                         lane);
            } else if (wave < n_items) {
                const int pair = wave / p.n_rep;
                load_q_block<T, D>(qpre, static_cast<const T*>(p.q), b * p.T + t0, H_q,
                                   h * p.n_rep + (wave % p.n_rep), pair == 0 ? 0 : 1, pair == 0 ? 3 : 2, nvalid, lane);
            }
        };
        if (!LATE_Q) issue_q();
        if (threadIdx.x == 0) *sm.nbad = 0;
        if (threadIdx.x < D / 32) sm.badmask[threadIdx.x] = 0u;
        lds_barrier();
        float b2[TPT];
        gate_prep<T, D, GATE, true, TPT>(sm, cur, nvalid, p.alpha, b2);
        if (LATE_Q) issue_q();
        lds_barrier();
        // state operand for this chunk (S entering it), then advance the state
        if constexpr (L::HG) publish_state_global(sm, opg, acc);
        else publish_state(sm, acc);
        state_advance(sm, cur, acc);
        if (c + 1 < c_end) store_slot<D>(slot, acc);
        else if (last_seg) store_state<D>(p.S_T + (size_t(b) * p.H_kv + h) * D * D, acc);
        __syncthreads();
        intra_key_operand<T, D, GATE, true, TPT>(sm, cur, b2);
        __syncthreads();
        ItemCtx<T, D, GATE> x;
        x.q = static_cast<const T*>(p.q);
        x.o = static_cast<T*>(p.o);
        x.row0 = b * p.T + t0;
        x.H_q = H_q;
        x.nvalid = nvalid;
        x.window = p.window;
        x.npv = c > 0 ? 64 : npv0;
        x.alpha = p.alpha;
        x.sink_k = SINK ? static_cast<const T*>(p.sink_k) + size_t(h) * p.n_sink * D : nullptr;
        x.sink_v = SINK ? static_cast<const T*>(p.sink_v) + size_t(h) * p.n_sink * D : nullptr;
        x.n_sink = SINK ? p.n_sink : 0;
        x.cur = cur;
        if constexpr (L::HG) {
            // previous chunk in global memory (read when x.npv > 0): the
            // sequence, or the continuation's halo rows
            const bool from_ring = c == 0 && npv0 > 0;
            x.kprv = from_ring ? halo_k : c > 0 ? kbase + (t0 - kChunk) * row_stride : kbase;
            x.vprv = from_ring ? halo_v : c > 0 ? vbase + (t0 - kChunk) * row_stride : vbase;
            x.prv_stride = from_ring ? D : row_stride;
            x.opg = opg;
        }
        // next chunk's K/V: in flight during the output phase, stored after it
        if (c + 1 < c_end) {
            const int64_t t1 = t0 + kChunk;
            load_chunk_issue<T, D>(cr, kbase, vbase, row_stride, t1, p.T - t1 < kChunk ? int(p.T - t1) : kChunk);
        }
        for (int it = wave; it < n_items; it += kPWaves) {
            x.hq = h * p.n_rep + (it % p.n_rep);
            int lane = threadIdx.x & 63;
            asm volatile("" : "+v"(lane));  // keep lane-derived addresses inside the loop
            const int pair = it / p.n_rep;
            if (it != wave)
                load_q_block<T, D, LATE_Q>(qpre, x.q, x.row0, H_q, x.hq, pair == 0 ? 0 : 1, pair == 0 ? 3 : 2, nvalid,
                                           lane);
            QNext nx;
            nx.any = false;  // without a resident state the registers are too few to load ahead
            if (pair == 0) output_block<T, D, GATE, 0, 3, SINK>(sm, x, lane, qpre, nx);
            else output_block<T, D, GATE, 1, 2, SINK>(sm, x, lane, qpre, nx);
            __builtin_amdgcn_s_setprio(0);
        }
        __syncthreads();
        if (c + 1 < c_end) {
            // the previous chunk's slot is free now (global halo: this chunk's)
            load_chunk_commit(sm, L::NSLOT == 2 ? cur ^ 1 : 0, cr);
            __syncthreads();
        }
    }
}

// ------------------------------------------------------------------ host side
template <typename T, int D, int GATE>
static hipError_t launch_prefill_t(const PrefillArgs& a) {
    PrefillParams p;
    p.q = a.q;
    p.k = a.k;
    p.v = a.v;
    p.o = a.o;
    p.S_T = a.S_T;
    p.carry = a.workspace;
    p.state_slots = a.workspace + a.plan.state_offset;
    p.op_slots = a.workspace + a.plan.op_offset;
    p.halo = a.workspace + a.plan.halo_offset;
    p.T = a.T;
    p.n_chunks = a.plan.n_chunks;
    p.cps = a.plan.cps;
    p.n_seg = a.plan.n_seg;
    p.H_kv = a.H_kv;
    p.n_rep = a.n_rep;
    p.window = a.window;
    p.alpha = a.alpha;
    p.S0 = a.S0;
    p.ring_k = a.ring_k;
    p.ring_v = a.ring_v;
    p.pos = a.pos;
    p.sink_k = a.sink_k;
    p.sink_v = a.sink_v;
    p.n_sink = a.n_sink;
    p.rec_mode = 0;
    hipStream_t st = static_cast<hipStream_t>(a.stream);
    // fp32 at d = 128: the output kernel in record mode writes the segment
    // records (the segment-state kernels are built for the other tile shapes)
    constexpr bool HG = Layout<T, D, GATE, true>::HG;
    if (HG && p.n_seg > 1 && (a.stage_mask & 1)) {
        PrefillParams pr = p;
        pr.rec_mode = 1;
        hipLaunchKernelGGL((prefill_output_kernel<T, D, GATE, false>), dim3(unsigned(p.n_seg - 1), a.H_kv, unsigned(a.B)),
                           dim3(kPThreads), 0, st, pr);
        const hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    if constexpr (!HG) if (p.n_seg > 1 && (a.stage_mask & 1)) {
        if constexpr (GATE == 0)
            hipLaunchKernelGGL((segment_state_scalar_kernel<T, D>), dim3(unsigned(p.n_seg - 1), a.H_kv, unsigned(a.B)),
                               dim3(kPThreads), 0, st, p);
        else
            hipLaunchKernelGGL((segment_state_vector_kernel<T, D>), dim3(unsigned(p.n_seg - 1), a.H_kv, unsigned(a.B)),
                               dim3(kPThreads), 0, st, p);
        const hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    if (p.n_seg > 1 && (a.stage_mask & 2)) {
        hipLaunchKernelGGL((carry_scan_kernel<D>), dim3(D * D / 256, a.H_kv, unsigned(a.B)), dim3(256), 0, st,
                           p.carry, p.S0, p.n_seg, p.H_kv);
        const hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    if (a.stage_mask & 4) {
        if (a.n_sink > 0)
            hipLaunchKernelGGL((prefill_output_kernel<T, D, GATE, true>), dim3(unsigned(p.n_seg), a.H_kv, unsigned(a.B)),
                               dim3(kPThreads), 0, st, p);
        else
            hipLaunchKernelGGL((prefill_output_kernel<T, D, GATE, false>), dim3(unsigned(p.n_seg), a.H_kv, unsigned(a.B)),
                               dim3(kPThreads), 0, st, p);
        return hipGetLastError();
    }
    return hipSuccess;
}

hipError_t launch_carry_scan(float* carry, int64_t n_seg, int H_kv, int64_t B, int d, void* stream) {
    if (n_seg <= 1) return hipSuccess;
    hipStream_t st = static_cast<hipStream_t>(stream);
    if (d == 64)
        hipLaunchKernelGGL((carry_scan_kernel<64>), dim3(64 * 64 / 256, H_kv, unsigned(B)), dim3(256), 0, st, carry,
                           nullptr, n_seg, H_kv);
    else
        hipLaunchKernelGGL((carry_scan_kernel<128>), dim3(128 * 128 / 256, H_kv, unsigned(B)), dim3(256), 0, st,
                           carry, nullptr, n_seg, H_kv);
    return hipGetLastError();
}

hipError_t launch_prefill(const PrefillArgs& a) {
    if (a.bf16) {
        if (a.d == 64) return a.gate ? launch_prefill_t<bf16_t, 64, 1>(a) : launch_prefill_t<bf16_t, 64, 0>(a);
        return a.gate ? launch_prefill_t<bf16_t, 128, 1>(a) : launch_prefill_t<bf16_t, 128, 0>(a);
    }
    if (a.d == 64) return a.gate ? launch_prefill_t<float, 64, 1>(a) : launch_prefill_t<float, 64, 0>(a);
    return a.gate ? launch_prefill_t<float, 128, 1>(a) : launch_prefill_t<float, 128, 0>(a);
}

}  // namespace liger
