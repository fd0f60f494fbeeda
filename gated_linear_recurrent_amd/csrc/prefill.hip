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
//   P1 segment_state_kernel : local end state L_s (from zero) and total log2
//                             decay of every segment but the last
//   P2 carry_scan_kernel    : S_in[s+1] = 2^(lg_s) (.) S_in[s] + L_s, in place
//   P3 prefill_output_kernel: per segment, walks its chunks from S_in[s],
//                             computes o, and (last segment) writes S_T
#include "device_common.h"
#include "kernels.h"

namespace liger {

constexpr int kPThreads = 512;
constexpr int kPWaves = kPThreads / 64;
constexpr float kEmax2 = 96.0f;  // largest log2 factor admitted to the MFMA path

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
    static constexpr int NSLOT = FULL ? 2 : 1;
    static constexpr int KB_ELEMS = (64 * DP > D * JP) ? 64 * DP : D * JP;

    static constexpr size_t K_OFF = 0;                                        // raw K [slot][64][DP]
    static constexpr size_t VT_OFF = K_OFF + size_t(NSLOT) * 64 * DP * E;     // V^T [slot][D][JP]
    static constexpr size_t KB_OFF = VT_OFF + size_t(NSLOT) * D * JP * E;     // K~ (state^T or intra)
    static constexpr size_t ST_OFF = KB_OFF + size_t(KB_ELEMS) * E;           // S'^T [D][DP]
    static constexpr size_t ST_BYTES = FULL ? size_t(D) * DP * E : 0;
    static constexpr size_t F_OFF = ST_OFF + ST_BYTES;                        // fp32 [64][FP]
    static constexpr size_t F_BYTES = (FULL && GATE) ? size_t(64) * FP * 4 : 0;
    static constexpr size_t TMP_OFF = F_OFF + F_BYTES;                        // gate-scan scratch
    // The scan scratch (part sums, raw references) lives inside the S'^T
    // region when there is one: that region is free until the state phase.
    static constexpr size_t TMP_FLOATS = size_t(kPThreads) + 3 * D;
    static constexpr bool TMP_ALIASED = FULL && (ST_BYTES >= TMP_FLOATS * 4);
    static constexpr size_t SMALL_OFF = TMP_ALIASED ? TMP_OFF : TMP_OFF + TMP_FLOATS * 4;
    // small persistent arrays: kmax[64] kinv[64] b2s[64] dec[D] mref[D] badlist[D] badmask[D/32] nbad
    static constexpr size_t SMALL_WORDS = 64 * 3 + D * 3 + D / 32 + 4;
    static constexpr size_t TOTAL = SMALL_OFF + SMALL_WORDS * 4;
    static_assert(TOTAL <= 160 * 1024, "LDS budget of a gfx950 workgroup exceeded");
};

template <typename T, int D, int GATE, bool FULL>
struct Smem {
    typedef Layout<T, D, GATE, FULL> L;
    T* K;      // [NSLOT][64][DP]
    T* Vt;     // [NSLOT][D][JP]
    T* Kb;     // [D][JP] (K~ state, transposed) then [64][DP] (K~ intra)
    T* St;     // [D][DP]
    float* F;  // [64][FP]
    float* part;  // [kPThreads]
    float* m2raw; // [D]
    float* bl2;   // [D]
    float* b0;    // [D]
    float* kmax;  // [64]
    float* kinv;  // [64]
    float* b2s;   // [64] scalar-gate cumulative log2 gate / scalar ell2 before the scan
    float* dec;   // [D] 2^(b_last) per d_k row
    float* mref;  // [D] log2 reference per channel (0 for bad channels)
    int* badlist; // [D]
    uint32_t* badmask;  // [D/32]
    int* nbad;

    __device__ explicit Smem(char* base) {
        K = reinterpret_cast<T*>(base + L::K_OFF);
        Vt = reinterpret_cast<T*>(base + L::VT_OFF);
        Kb = reinterpret_cast<T*>(base + L::KB_OFF);
        St = reinterpret_cast<T*>(base + L::ST_OFF);
        F = reinterpret_cast<float*>(base + L::F_OFF);
        float* tmp = reinterpret_cast<float*>(base + (L::TMP_ALIASED ? L::ST_OFF : L::TMP_OFF));
        part = tmp;
        m2raw = tmp + kPThreads;
        bl2 = m2raw + D;
        b0 = bl2 + D;
        float* sm = reinterpret_cast<float*>(base + L::SMALL_OFF);
        kmax = sm;
        kinv = sm + 64;
        b2s = sm + 128;
        dec = sm + 192;
        mref = dec + D;
        badlist = reinterpret_cast<int*>(mref + D);
        badmask = reinterpret_cast<uint32_t*>(badlist + D);
        nbad = reinterpret_cast<int*>(badmask + D / 32);
    }
};

struct PrefillParams {
    const void* q;
    const void* k;
    const void* v;
    void* o;
    float* S_T;
    float* carry;
    int64_t T;
    int64_t n_chunks;
    int64_t cps;
    int64_t n_seg;
    int H_kv;
    int n_rep;
    int window;
    float alpha;
};

// ------------------------------------------------------------ chunk loading
// K rows go to LDS as they are; V rows are written transposed (V^T[c][j]).
// Rows past the end of the sequence are zero.
template <typename T, int D, int GATE, bool FULL>
__device__ __forceinline__ void load_chunk(const Smem<T, D, GATE, FULL>& sm, int slot,
                                           const T* kbase, const T* vbase, int64_t row_stride,
                                           int64_t t0, int nvalid) {
    typedef Layout<T, D, GATE, FULL> L;
    constexpr int VPL = 16 / sizeof(T);
    constexpr int PPR = D / VPL;
    T* Ks = sm.K + slot * 64 * L::DP;
    T* Vts = sm.Vt + slot * D * L::JP;
    for (int idx = ltid(); idx < 64 * PPR; idx += kPThreads) {
        const int j = idx / PPR;
        const int c0 = (idx % PPR) * VPL;
        uint4 kk = make_uint4(0, 0, 0, 0), vv = make_uint4(0, 0, 0, 0);
        if (j < nvalid) {
            const int64_t off = (t0 + j) * row_stride + c0;
            kk = *reinterpret_cast<const uint4*>(kbase + off);
            vv = *reinterpret_cast<const uint4*>(vbase + off);
        }
        *reinterpret_cast<uint4*>(Ks + j * L::DP + c0) = kk;
        const T* ve = reinterpret_cast<const T*>(&vv);
#pragma unroll
        for (int e = 0; e < VPL; ++e) Vts[(c0 + e) * L::JP + j] = ve[e];
    }
}

template <typename T, int D, int GATE, bool FULL>
__device__ __forceinline__ void zero_slot(const Smem<T, D, GATE, FULL>& sm, int slot) {
    typedef Layout<T, D, GATE, FULL> L;
    uint32_t* kz = reinterpret_cast<uint32_t*>(sm.K + slot * 64 * L::DP);
    for (int i = ltid(); i < 64 * L::DP * int(sizeof(T)) / 4; i += kPThreads) kz[i] = 0u;
    uint32_t* vz = reinterpret_cast<uint32_t*>(sm.Vt + slot * D * L::JP);
    for (int i = ltid(); i < D * L::JP * int(sizeof(T)) / 4; i += kPThreads) vz[i] = 0u;
}

// ------------------------------------------------------- per-chunk gate work
// B1: softmax statistics of every key row (max, 1/sum) and, for the scalar
// gate, ell2_j = log2 sigmoid(mean_c k_j[c]). Rows past the end get 1/sum = 0
// so phi(k) vanishes there, and ell2 = 0.
template <typename T, int D, int GATE, bool FULL>
__device__ __forceinline__ void key_row_stats(const Smem<T, D, GATE, FULL>& sm, int slot, int nvalid) {
    typedef Layout<T, D, GATE, FULL> L;
    constexpr int EPL = D / 64;
    const int lane = ltid() & 63, wave = ltid() >> 6;
    const T* Ks = sm.K + slot * 64 * L::DP;
    for (int j = wave; j < 64; j += kPWaves) {
        float x[EPL];
        float mx = -INFINITY, s = 0.f;
#pragma unroll
        for (int e = 0; e < EPL; ++e) {
            x[e] = to_f32(Ks[j * L::DP + lane + 64 * e]);
            mx = fmaxf(mx, x[e]);
            s += x[e];
        }
        mx = wave_max(mx);
        float se = 0.f;
#pragma unroll
        for (int e = 0; e < EPL; ++e) se += fast_exp2((x[e] - mx) * kLog2e);
        se = wave_sum(se);
        if (GATE == 0) s = wave_sum(s);
        if (lane == 0) {
            const bool ok = j < nvalid;
            sm.kmax[j] = mx;
            sm.kinv[j] = ok ? 1.0f / se : 0.0f;
            if (GATE == 0) sm.b2s[j] = ok ? log2_sigmoid(s * (1.0f / D)) : 0.0f;
        }
    }
}

// Scalar gate: inclusive prefix sum of ell2 over the chunk (one wave).
template <typename T, int D, int GATE, bool FULL>
__device__ __forceinline__ void scalar_gate_scan(const Smem<T, D, GATE, FULL>& sm) {
    if (ltid() < 64) {
        const int lane = ltid();
        float x = sm.b2s[lane];
#pragma unroll
        for (int o = 1; o < 64; o <<= 1) {
            const float y = __shfl_up(x, o, 64);
            if (lane >= o) x += y;
        }
        sm.b2s[lane] = x;
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
    const int c = ltid() % D;
    const int part = ltid() / D;
    const T* Ks = sm.K + slot * 64 * L::DP;
    const int lo = c > 0 ? c - 1 : 0;
    const int hi = c + 3 < D ? c + 3 : D;
    const float inv_cnt = 1.0f / static_cast<float>(hi - lo);
    float run = 0.f;
#pragma unroll
    for (int jj = 0; jj < TPT; ++jj) {
        const int j = part * TPT + jj;
        float x = 0.f;
        for (int m = lo; m < hi; ++m) x += to_f32(Ks[j * L::DP + m]);
        run += j < nvalid ? log2_sigmoid(x * inv_cnt) : 0.0f;
        b2[jj] = run;
    }
    sm.part[part * D + c] = run;
    __syncthreads();
    float off = 0.f;
    for (int p = 0; p < part; ++p) off += sm.part[p * D + c];
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
// Wave w owns TPW 16x16 tiles (rt, t) of the d x d state, held in fp32
// accumulators: acc[u][r] = S[16 rt + 4 (L>>4) + r][16 t + (L&15)].
template <int D>
struct StateTiles {
    static constexpr int NTT = D / 16;
    static constexpr int TPW = NTT * NTT / kPWaves;
    static_assert(TPW >= 1, "state tiles per wave");
    __device__ static __forceinline__ int rt(int wave, int u) { return (wave * TPW + u) / NTT; }
    __device__ static __forceinline__ int ct(int wave, int u) { return (wave * TPW + u) % NTT; }
};

// S <- diag(dec) S + Kst^T V over the current chunk (Kst^T = Kb as [D][JP]).
template <typename T, int D, int GATE, bool FULL>
__device__ __forceinline__ void state_advance(const Smem<T, D, GATE, FULL>& sm, int slot,
                                              f32x4_t (&acc)[StateTiles<D>::TPW]) {
    typedef Layout<T, D, GATE, FULL> L;
    typedef Mfma<T> M;
    typedef StateTiles<D> ST;
    const int lane = ltid() & 63, wave = ltid() >> 6;
    const int col = lane & 15, g = lane >> 4;
    const T* Vts = sm.Vt + slot * D * L::JP;
#pragma unroll
    for (int u = 0; u < ST::TPW; ++u) {
        const int rt = ST::rt(wave, u), t = ST::ct(wave, u);
        f32x4_t d = zero4();
#pragma unroll
        for (int ks = 0; ks < 64 / M::KSTEP; ++ks) {
            const typename M::frag a = M::load(sm.Kb + (16 * rt + col) * L::JP + M::KSTEP * ks + M::KPL * g);
            const typename M::frag b = M::load(Vts + (16 * t + col) * L::JP + M::KSTEP * ks + M::KPL * g);
            d = M::mma(a, b, d);
        }
        const int r0 = 16 * rt + 4 * g;
#pragma unroll
        for (int r = 0; r < 4; ++r) acc[u][r] = sm.dec[r0 + r] * acc[u][r] + d[r];
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

// -------------------------------------------- gate prep shared by P1 and P3
// After this: dec, mref, badlist/badmask/nbad, F (P3, vector) and the
// transposed state key operand Kb[c][j] = phik_j[c] 2^(b_last[c] - b_j[c]).
// Returns (through b2) the per-thread cumulative gates for the intra operand.
template <typename T, int D, int GATE, bool FULL, int TPT>
__device__ __forceinline__ void gate_prep(const Smem<T, D, GATE, FULL>& sm, int slot, int nvalid,
                                          float alpha, float (&b2)[TPT]) {
    typedef Layout<T, D, GATE, FULL> L;
    const T* Ks = sm.K + slot * 64 * L::DP;
    key_row_stats(sm, slot, nvalid);
    __syncthreads();
    if (GATE == 0) {
        scalar_gate_scan(sm);
        __syncthreads();
        const float bl = sm.b2s[nvalid - 1];
        for (int idx = ltid(); idx < 64 * D; idx += kPThreads) {
            const int j = idx & 63, c = idx >> 6;
            const float kv = to_f32(Ks[j * L::DP + c]);
            sm.Kb[c * L::JP + j] =
                from_f32<T>(sm.kinv[j] * fast_exp2((kv - sm.kmax[j]) * kLog2e + bl - sm.b2s[j]));
        }
        if (ltid() < D) {
            sm.dec[ltid()] = fast_exp2(bl);
            sm.mref[ltid()] = 0.0f;
        }
    } else {
        vector_gate_scan<T, D, GATE, FULL, TPT>(sm, slot, nvalid, b2);
        __syncthreads();
        const int c = ltid() % D;
        const int part = ltid() / D;
        const float m2 = sm.m2raw[c];
        const float bl = sm.bl2[c];
        const bool bad = fmaxf(sm.b0[c] - m2, m2 - bl) > kEmax2;
        const float mref = bad ? 0.0f : m2;
        if (part == 0) {
            sm.mref[c] = mref;
            sm.dec[c] = fast_exp2(bl);
            if (FULL && bad) {
                const int idx = atomicAdd(sm.nbad, 1);
                sm.badlist[idx] = c;
                atomicOr(&sm.badmask[c >> 5], 1u << (c & 31));
            }
        }
#pragma unroll
        for (int jj = 0; jj < TPT; ++jj) {
            const int j = part * TPT + jj;
            const float kv = to_f32(Ks[j * L::DP + c]);
            sm.Kb[c * L::JP + j] =
                from_f32<T>(sm.kinv[j] * fast_exp2((kv - sm.kmax[j]) * kLog2e + bl - b2[jj]));
            if (FULL) sm.F[j * L::FP + c] = bad ? b2[jj] : alpha * fast_exp2(b2[jj] - mref);
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
        for (int idx = ltid(); idx < 64 * D; idx += kPThreads) {
            const int j = idx / D, c = idx % D;
            const float kv = to_f32(Ks[j * L::DP + c]);
            sm.Kb[j * L::DP + c] = from_f32<T>(sm.kinv[j] * fast_exp2((kv - sm.kmax[j]) * kLog2e));
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
template <typename T, int D, int GATE>
__global__ __launch_bounds__(kPThreads) void segment_state_kernel(PrefillParams p) {
    typedef Layout<T, D, GATE, false> L;
    __shared__ __align__(16) char smem[L::TOTAL];
    const Smem<T, D, GATE, false> sm(smem);
    constexpr int TPT = 64 / (kPThreads / D);

    const int s = blockIdx.x;
    const int h = blockIdx.y;
    const int64_t b = blockIdx.z;
    const int64_t row_stride = int64_t(p.H_kv) * D;
    const T* kbase = static_cast<const T*>(p.k) + (b * p.T * p.H_kv + h) * D;
    const T* vbase = static_cast<const T*>(p.v) + (b * p.T * p.H_kv + h) * D;

    f32x4_t acc[StateTiles<D>::TPW];
    load_state<D>(nullptr, acc);
    float lg = 0.f;  // total log2 decay of the segment for channel threadIdx.x (< D)
    const int64_t c_begin = int64_t(s) * p.cps;
    const int64_t c_end = c_begin + p.cps;  // never the last segment: always whole chunks
    for (int64_t c = c_begin; c < c_end; ++c) {
        const int64_t t0 = c * kChunk;
        load_chunk(sm, 0, kbase, vbase, row_stride, t0, kChunk);
        __syncthreads();
        float b2[TPT];
        gate_prep<T, D, GATE, false, TPT>(sm, 0, kChunk, p.alpha, b2);
        __syncthreads();
        if (threadIdx.x < D) lg += GATE ? sm.bl2[threadIdx.x] : sm.b2s[kChunk - 1];
        state_advance(sm, 0, acc);
        __syncthreads();
    }
    const size_t rec = size_t(D) * D + D;
    float* dst = p.carry + ((size_t(b) * p.H_kv + h) * size_t(p.n_seg - 1) + s) * rec;
    store_state<D>(dst, acc);
    if (threadIdx.x < D) dst[size_t(D) * D + threadIdx.x] = lg;
}

// ------------------------------------------------------------------ P2
template <int D>
__global__ __launch_bounds__(256) void carry_scan_kernel(float* __restrict__ carry, int64_t n_seg, int H_kv) {
    constexpr int NV4 = D * D / 4;
    const int e4 = blockIdx.x * 256 + threadIdx.x;
    if (e4 >= NV4) return;
    const int h = blockIdx.y;
    const int64_t b = blockIdx.z;
    const size_t rec = size_t(D) * D + D;
    float* base = carry + (size_t(b) * H_kv + h) * size_t(n_seg - 1) * rec;
    const int r = (e4 * 4) / D;
    float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
    constexpr int BATCH = 8;
    for (int64_t s0 = 0; s0 < n_seg - 1; s0 += BATCH) {
        float4 Ls[BATCH];
        float lg[BATCH];
#pragma unroll
        for (int u = 0; u < BATCH; ++u) {
            if (s0 + u < n_seg - 1) {
                const float* recp = base + (s0 + u) * rec;
                Ls[u] = *reinterpret_cast<const float4*>(recp + e4 * 4);
                lg[u] = recp[size_t(D) * D + r];
            }
        }
#pragma unroll
        for (int u = 0; u < BATCH; ++u) {
            if (s0 + u < n_seg - 1) {
                const float f = fast_exp2(lg[u]);
                acc.x = f * acc.x + Ls[u].x;
                acc.y = f * acc.y + Ls[u].y;
                acc.z = f * acc.z + Ls[u].z;
                acc.w = f * acc.w + Ls[u].w;
                *reinterpret_cast<float4*>(base + (s0 + u) * rec + e4 * 4) = acc;
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
    int I;             // 16-row query tile inside the chunk
    int nvalid;
    int window;
    bool have_prev;    // a previous chunk exists (chunk index > 0)
    float alpha;
    int cur;
};

template <typename T, int D, int GATE, int I>
__device__ __forceinline__ void output_item(const Smem<T, D, GATE, true>& sm, const ItemCtx<T, D, GATE>& x,
                                            int lane) {
    typedef Layout<T, D, GATE, true> L;
    typedef Mfma<T> M;
    typedef typename M::frag Frag;
    constexpr int KS = D / M::KSTEP;
    constexpr int KPL = M::KPL;
    constexpr int NT = D / 16;
    constexpr bool BF = sizeof(T) == 2;
    const int col = lane & 15, g = lane >> 4;
    const int i_loc = 16 * I + col;
    const bool row_ok = i_loc < x.nvalid;
    const T* qrow = x.q + ((x.row0 + (row_ok ? i_loc : 0)) * x.H_q + x.hq) * D;
    const T* Kcur = sm.K + x.cur * 64 * L::DP;
    const T* Kprv = sm.K + (x.cur ^ 1) * 64 * L::DP;
    const T* Vcur = sm.Vt + x.cur * D * L::JP;
    const T* Vprv = sm.Vt + (x.cur ^ 1) * D * L::JP;
    const int nbad = GATE ? *sm.nbad : 0;

    // ---- query row. qr: raw fragment (window operand). qt: unnormalised
    // e^(q - max) times the gate factor (recurrence operand); the softmax
    // normaliser qinv is applied to the products, which are linear in phi(q).
    Frag qr[KS];
#pragma unroll
    for (int s = 0; s < KS; ++s) {
        if constexpr (BF) {
            const uint4 u = row_ok ? *reinterpret_cast<const uint4*>(qrow + M::KSTEP * s + KPL * g)
                                   : make_uint4(0, 0, 0, 0);
            qr[s] = __builtin_bit_cast(Frag, u);
        } else {
            qr[s] = row_ok ? reinterpret_cast<const float*>(qrow)[M::KSTEP * s + g] : 0.0f;
        }
    }
    auto qval = [&](int s, int i) -> float {
        if constexpr (BF) {
            const uint4 u = __builtin_bit_cast(uint4, qr[s]);
            const uint32_t w = (i >> 1) == 0 ? u.x : (i >> 1) == 1 ? u.y : (i >> 1) == 2 ? u.z : u.w;
            return __uint_as_float((i & 1) ? (w & 0xffff0000u) : (w << 16));
        } else {
            return __builtin_bit_cast(float, qr[s]);
        }
    };
    float qmax = -INFINITY;
#pragma unroll
    for (int s = 0; s < KS; ++s)
#pragma unroll
        for (int i = 0; i < KPL; ++i) qmax = fmaxf(qmax, qval(s, i));
    qmax = group4_max(qmax);
    Frag qt[KS];
    float qsum = 0.f;
#pragma unroll
    for (int s = 0; s < KS; ++s) {
        float tmp[KPL];
#pragma unroll
        for (int i = 0; i < KPL; ++i) {
            const float e = fast_exp2((qval(s, i) - qmax) * kLog2e);
            qsum += e;
            if (GATE) {
                const int ch = M::KSTEP * s + KPL * g + i;
                float f = sm.F[i_loc * L::FP + ch];
                if (nbad && ((sm.badmask[ch >> 5] >> (ch & 31)) & 1u)) f = 0.0f;
                tmp[i] = e * f;
            } else {
                tmp[i] = e;
            }
        }
        qt[s] = M::pack(tmp);
    }
    // alpha folded here; for the vector gate F already carries alpha
    const float qinv = (GATE ? 1.0f : x.alpha) / group4_sum(qsum);

    // ---- sliding-window scores over key tiles kt = I-4 .. I (relative to
    // the chunk start; negative tiles live in the previous chunk's slot)
    constexpr int U0 = I - 4;
    bool live[5];
    float pw[5][4];
    {
        const float lscale = kLog2e * rsqrtf(static_cast<float>(D));
        float lmax = -INFINITY;
#pragma unroll
        for (int u = 0; u < 5; ++u) {
            const int kt = U0 + u;
            live[u] = (kt >= 0 || x.have_prev) && (16 * kt + 15 > 16 * I - x.window);
#pragma unroll
            for (int r = 0; r < 4; ++r) pw[u][r] = -INFINITY;
            if (live[u]) {
                const T* krow = kt >= 0 ? Kcur + (16 * kt + col) * L::DP : Kprv + (16 * kt + 64 + col) * L::DP;
                f32x4_t d4 = zero4();
#pragma unroll
                for (int s = 0; s < KS; ++s) d4 = M::mma(M::load(krow + M::KSTEP * s + KPL * g), qr[s], d4);
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int j = 16 * kt + 4 * g + r;
                    const bool ok = (j <= i_loc) && (j > i_loc - x.window);
                    pw[u][r] = ok ? d4[r] * lscale : -INFINITY;
                    lmax = fmaxf(lmax, pw[u][r]);
                }
            }
        }
        lmax = group4_max(lmax);
        float lsum = 0.f;
#pragma unroll
        for (int u = 0; u < 5; ++u)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const float e = live[u] ? fast_exp2(pw[u][r] - lmax) : 0.0f;
                pw[u][r] = e;
                lsum += e;
            }
        const float pscale = (1.0f - x.alpha) / group4_sum(lsum);
#pragma unroll
        for (int u = 0; u < 5; ++u)
#pragma unroll
            for (int r = 0; r < 4; ++r) pw[u][r] *= pscale;
    }

    // ---- intra-chunk scores A[i][j] = Q~_i . K~_j, causal; lane holds
    // j = 16J + 4g + r for query i = i_loc
    float aw[I + 1][4];
#pragma unroll
    for (int J = 0; J <= I; ++J) {
        f32x4_t a4 = zero4();
#pragma unroll
        for (int s = 0; s < KS; ++s)
            a4 = M::mma(M::load(sm.Kb + (16 * J + col) * L::DP + M::KSTEP * s + KPL * g), qt[s], a4);
#pragma unroll
        for (int r = 0; r < 4; ++r) a4[r] *= qinv;
        for (int nb = 0; nb < nbad; ++nb) {
            const int c = sm.badlist[nb];
            const float qc = row_ok ? to_f32(qrow[c]) : 0.0f;
            const float coef = x.alpha * fast_exp2((qc - qmax) * kLog2e) * qinv;
            const float b2i = sm.F[i_loc * L::FP + c];
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int j = 16 * J + 4 * g + r;
                const float phik = sm.kinv[j] * fast_exp2((to_f32(Kcur[j * L::DP + c]) - sm.kmax[j]) * kLog2e);
                const float term = coef * phik * fast_exp2(fminf(b2i - sm.F[j * L::FP + c], 0.0f));
                a4[r] += j <= i_loc ? term : 0.0f;
            }
        }
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int j = 16 * J + 4 * g + r;
            float val = a4[r];
            if (GATE == 0) val *= fast_exp2(fminf(sm.b2s[i_loc] - sm.b2s[j], 0.0f));
            aw[J][r] = j <= i_loc ? val : 0.0f;
        }
    }

    // ---- operand fragments of the score matrices. bf16: a k-step of 32 keys
    // takes two 16-key tiles; the V^T operand below reads the same key order.
    constexpr int NA = (I + 2) / 2;
    Frag af[NA], pf[3];
    if constexpr (BF) {
#pragma unroll
        for (int pj = 0; pj < NA; ++pj) {
            float v8[8];
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                v8[r] = aw[2 * pj][r];
                v8[4 + r] = 2 * pj + 1 <= I ? aw[2 * pj + 1 <= I ? 2 * pj + 1 : 0][r] : 0.0f;
            }
            af[pj] = M::pack(v8);
        }
#pragma unroll
        for (int pu = 0; pu < 3; ++pu) {
            float v8[8];
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                v8[r] = pw[2 * pu][r];
                v8[4 + r] = 2 * pu + 1 < 5 ? pw[2 * pu + 1 < 5 ? 2 * pu + 1 : 0][r] : 0.0f;
            }
            pf[pu] = M::pack(v8);
        }
    }
    const float inter_scale = GATE == 0 ? qinv * fast_exp2(sm.b2s[i_loc]) : qinv;
    float bad_coef = 0.0f;

    // ---- one 16-wide slice of d_v at a time: inter + intra + window, store
    T* orow = x.o + ((x.row0 + i_loc) * x.H_q + x.hq) * D;
#pragma unroll 2
    for (int t = 0; t < NT; ++t) {
        f32x4_t acc = zero4();
#pragma unroll
        for (int s = 0; s < KS; ++s)
            acc = M::mma(M::load(sm.St + (16 * t + col) * L::DP + M::KSTEP * s + KPL * g), qt[s], acc);
        acc *= inter_scale;
        for (int nb = 0; nb < nbad; ++nb) {
            const int c = sm.badlist[nb];
            const float qc = row_ok ? to_f32(qrow[c]) : 0.0f;
            bad_coef = x.alpha * fast_exp2((qc - qmax) * kLog2e) * qinv * fast_exp2(sm.F[i_loc * L::FP + c]);
#pragma unroll
            for (int r = 0; r < 4; ++r) acc[r] += bad_coef * to_f32(sm.St[(16 * t + 4 * g + r) * L::DP + c]);
        }
        const T* vrow_c = Vcur + (16 * t + col) * L::JP;
        const T* vrow_p = Vprv + (16 * t + col) * L::JP + 64;
        if constexpr (BF) {
#pragma unroll
            for (int pj = 0; pj < NA; ++pj) {
                const uint2 lo = *reinterpret_cast<const uint2*>(vrow_c + 32 * pj + 4 * g);
                const uint2 hi = *reinterpret_cast<const uint2*>(vrow_c + 32 * pj + 16 + 4 * g);
                acc = M::mma(__builtin_bit_cast(Frag, make_uint4(lo.x, lo.y, hi.x, hi.y)), af[pj], acc);
            }
#pragma unroll
            for (int pu = 0; pu < 3; ++pu) {
                const int u0 = 2 * pu, u1 = 2 * pu + 1;
                const bool l1 = u1 < 5 && live[u1 < 5 ? u1 : 0];
                if (live[u0] || l1) {
                    const int kt0 = U0 + u0;
                    const int kt1 = u1 < 5 ? U0 + u1 : kt0;
                    const T* p0 = kt0 >= 0 ? vrow_c + 16 * kt0 : vrow_p + 16 * kt0;
                    const T* p1 = kt1 >= 0 ? vrow_c + 16 * kt1 : vrow_p + 16 * kt1;
                    const uint2 lo = *reinterpret_cast<const uint2*>(p0 + 4 * g);
                    const uint2 hi = *reinterpret_cast<const uint2*>(p1 + 4 * g);
                    acc = M::mma(__builtin_bit_cast(Frag, make_uint4(lo.x, lo.y, hi.x, hi.y)), pf[pu], acc);
                }
            }
        } else {
#pragma unroll
            for (int J = 0; J <= I; ++J)
#pragma unroll
                for (int r = 0; r < 4; ++r)
                    acc = M::mma(M::load(vrow_c + 16 * J + 4 * g + r), __builtin_bit_cast(Frag, aw[J][r]), acc);
#pragma unroll
            for (int u = 0; u < 5; ++u)
                if (live[u]) {
                    const int kt = U0 + u;
                    const T* pr = kt >= 0 ? vrow_c + 16 * kt : vrow_p + 16 * kt;
#pragma unroll
                    for (int r = 0; r < 4; ++r)
                        acc = M::mma(M::load(pr + 4 * g + r), __builtin_bit_cast(Frag, pw[u][r]), acc);
                }
        }
        if (row_ok) {
            T* dst = orow + 16 * t + 4 * g;
            if constexpr (BF) {
                *reinterpret_cast<uint2*>(dst) = make_uint2(pack_bf16x2(acc[0], acc[1]), pack_bf16x2(acc[2], acc[3]));
            } else {
                *reinterpret_cast<float4*>(dst) = make_float4(acc[0], acc[1], acc[2], acc[3]);
            }
        }
    }
}

template <typename T, int D, int GATE>
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

    f32x4_t acc[StateTiles<D>::TPW];
    load_state<D>(s == 0 ? nullptr : p.carry + ((size_t(b) * p.H_kv + h) * size_t(p.n_seg - 1) + (s - 1)) * rec, acc);

    const int64_t c_begin = int64_t(s) * p.cps;
    const int64_t c_end = c_begin + p.cps < p.n_chunks ? c_begin + p.cps : p.n_chunks;
    if (c_begin > 0) {
        load_chunk(sm, int((c_begin - 1) & 1), kbase, vbase, row_stride, (c_begin - 1) * kChunk, kChunk);
    } else {
        zero_slot(sm, int((c_begin + 1) & 1));
    }
    for (int64_t c = c_begin; c < c_end; ++c) {
        const int cur = int(c & 1);
        const int64_t t0 = c * kChunk;
        const int nvalid = p.T - t0 < kChunk ? int(p.T - t0) : kChunk;
        if (threadIdx.x == 0) *sm.nbad = 0;
        if (threadIdx.x < D / 32) sm.badmask[threadIdx.x] = 0u;
        load_chunk(sm, cur, kbase, vbase, row_stride, t0, nvalid);
        __syncthreads();
        float b2[TPT];
        gate_prep<T, D, GATE, true, TPT>(sm, cur, nvalid, p.alpha, b2);
        __syncthreads();
        // state operand for this chunk (S entering it), then advance the state
        publish_state(sm, acc);
        state_advance(sm, cur, acc);
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
        x.have_prev = c > 0;
        x.alpha = p.alpha;
        x.cur = cur;
        const int n_items = p.n_rep * 4;
        for (int it = wave; it < n_items; it += kPWaves) {
            const int ti = it / p.n_rep;
            x.hq = h * p.n_rep + (it % p.n_rep);
            int lane = threadIdx.x & 63;
            asm volatile("" : "+v"(lane));  // keep lane-derived addresses inside the loop
            // pairs query tiles {0,3} and {1,2} on the waves of the two halves
            switch (ti) {
                case 0: output_item<T, D, GATE, 0>(sm, x, lane); break;
                case 1: output_item<T, D, GATE, 1>(sm, x, lane); break;
                case 2: output_item<T, D, GATE, 3>(sm, x, lane); break;
                default: output_item<T, D, GATE, 2>(sm, x, lane); break;
            }
        }
        __syncthreads();
    }
    if (s == p.n_seg - 1) store_state<D>(p.S_T + (size_t(b) * p.H_kv + h) * D * D, acc);
}

// ------------------------------------------------------------------ host side
PrefillPlan make_prefill_plan(int64_t B, int64_t T, int H_kv, int d, bool bf16, int64_t chunks_per_segment) {
    PrefillPlan pl;
    pl.n_chunks = (T + kChunk - 1) / kChunk;
    int64_t cps = chunks_per_segment;
    if (cps <= 0) {
        // One output workgroup per compute unit (two when the LDS footprint allows).
        const int64_t per_cu = (bf16 && d == 64) ? 2 : 1;
        const int64_t target = 256 * per_cu;
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
    pl.workspace_bytes = size_t(B) * H_kv * size_t(pl.n_seg - 1) * pl.carry_floats * sizeof(float);
    return pl;
}

template <typename T, int D, int GATE>
static hipError_t launch_prefill_t(const PrefillArgs& a) {
    PrefillParams p;
    p.q = a.q;
    p.k = a.k;
    p.v = a.v;
    p.o = a.o;
    p.S_T = a.S_T;
    p.carry = a.workspace;
    p.T = a.T;
    p.n_chunks = a.plan.n_chunks;
    p.cps = a.plan.cps;
    p.n_seg = a.plan.n_seg;
    p.H_kv = a.H_kv;
    p.n_rep = a.n_rep;
    p.window = a.window;
    p.alpha = a.alpha;
    hipStream_t st = static_cast<hipStream_t>(a.stream);
    if (p.n_seg > 1 && (a.stage_mask & 1)) {
        hipLaunchKernelGGL((segment_state_kernel<T, D, GATE>), dim3(unsigned(p.n_seg - 1), a.H_kv, unsigned(a.B)),
                           dim3(kPThreads), 0, st, p);
        const hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    if (p.n_seg > 1 && (a.stage_mask & 2)) {
        hipLaunchKernelGGL((carry_scan_kernel<D>), dim3((D * D / 4 + 255) / 256, a.H_kv, unsigned(a.B)), dim3(256), 0, st,
                           p.carry, p.n_seg, p.H_kv);
        const hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    if (a.stage_mask & 4) {
        hipLaunchKernelGGL((prefill_output_kernel<T, D, GATE>), dim3(unsigned(p.n_seg), a.H_kv, unsigned(a.B)),
                           dim3(kPThreads), 0, st, p);
        return hipGetLastError();
    }
    return hipSuccess;
}

hipError_t launch_prefill(const PrefillArgs& a) {
    if (a.bf16) {
        if (a.d == 64) return a.gate ? launch_prefill_t<bf16_t, 64, 1>(a) : launch_prefill_t<bf16_t, 64, 0>(a);
        return a.gate ? launch_prefill_t<bf16_t, 128, 1>(a) : launch_prefill_t<bf16_t, 128, 0>(a);
    }
    if (a.d == 64) return a.gate ? launch_prefill_t<float, 64, 1>(a) : launch_prefill_t<float, 64, 0>(a);
    return hipErrorInvalidValue;  // fp32 with d = 128 exceeds the LDS budget of this kernel
}

}  // namespace liger
