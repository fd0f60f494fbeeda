// Backward of the Liger Attention prefill for gfx950: gradients dq, dk, dv
// (float32) of sum(o * dO) for o = alpha GRM + (1 - alpha) SWA over whole
// sequences from a zero state, bf16 inputs (paper-notes page "Liger:
// Linearizing Large Language Models to Gated Recurrent Structures": unified
// gated linear recurrence; Liger Attention; the gate built from the key
// projection, here pooled as in the forward).
//
// GRM part, in 64-token chunks. With b the inclusive cumulative log2 gate of
// a chunk (relative to its start, per d_k channel; b <= 0, non-increasing),
// Delta = b of the last row, S0 the state entering the chunk and U the
// adjoint flowing into the chunk's last state from later tokens:
//   dphi(q_s^h) = 2^(b_s) (.) (S0 alpha dO_s^h) + sum_{t<=s} 2^(b_s-b_t) (.) phik_t A^h[s][t]
//   dphi(k_t)   = 2^(Delta-b_t) (.) (U v_t)     + sum_{s>=t} 2^(b_s-b_t) (.) sum_h phiq_s^h A^h[s][t]
//   dv_t        = (phik_t (.) 2^(Delta-b_t)) U  + sum_{s>=t} sum_h B^h[t][s] alpha dO_s^h
// with A^h[s][t] = alpha dO_s^h . v_t and B^h[t][s] = sum_c phik_t[c] 2^(b_s-b_t)[c] phiq_s^h[c].
// States between chunks: S0 of chunk c+1 = 2^Delta_c (.) S0_c + sum_t (phik_t (.) 2^(Delta-b_t))^T v_t,
// and U_{c-1} = 2^Delta_c (.) U_c + sum_{s,h} (phiq_s^h (.) 2^(b_s))^T alpha dO_s^h (U_last = 0),
// both the same first-order scan, run on per-chunk records.
// Gate: treating the cumulative natural-log gate B_t = sum_{u<=t} ln g_u as
// free variables, dL/dB_t = sum_h phiq_t^h (.) dphi(q_t^h) - phik_t (.) dphi(k_t)
// (every pair term of o depends on B_s - B_t only), so
// d ln g_u = sum_{t>=u} dL/dB_t, d x_u = d ln g_u (1 - g_u) for g = sigmoid(x),
// and the pool's transpose carries dx to dk.
// Decays inside a chunk are split around a per-channel reference m (b of row
// 31): phik_t 2^(m-b_t) and phiq_s 2^(b_s-m) are MFMA operands. A channel
// whose factors could exceed 2^96 ("extreme") is left out of the products
// and evaluated pair by pair in fp32 instead.
//
// SWA part (window w <= 64, self included, scale 1/sqrt(d)): per query the
// softmax p over its window, dp = (1-alpha) dO . v, dz = p (dp - sum p dp),
// dq += dz k / sqrt(d), dk += dz q / sqrt(d), dv += p (1-alpha) dO.
//
// Kernels, in stream order:
//   bwd_records_kernel : per chunk, the forward and adjoint chunk records
//   carry scans        : chunk-start states S0 and adjoints U (prefill.hip)
//   bwd_chunk_kernel   : GRM gradients of one chunk: dq, dk (feature-map
//                        part), dv written; dL/dB rows and chunk sums stored
//   bwd_swa_q_kernel   : window softmax per query; dq += ..; row statistics
//   bwd_swa_k_kernel   : per key tile: dk += .., dv += ..; then the gate chain of
//                        the chunk (suffix sums of dL/dB, sigmoid and pool
//                        transpose) into the same dk update
// Computed operands enter the bf16 MFMA as hi + lo bf16 pairs (fp32-accurate
// products), raw bf16 inputs as they are. Barriers order LDS only: no kernel
// here reads back a global value it wrote.
#include "device_common.h"
#include "kernels.h"

namespace liger {
namespace {

constexpr int kBT = 512;  // threads of the chunk kernels (8 waves)
constexpr int kST = 256;  // threads of the window kernels (4 waves)
constexpr float kExtreme = 96.0f;

struct BwdParams {
    const bf16_t* q;
    const bf16_t* k;
    const bf16_t* v;
    const bf16_t* dO;
    float* dq;
    float* dk;
    float* dv;
    float* fwd;    // [B][H_kv][n-1][d*d + d] forward chunk records -> chunk-start states
    float* adj;    // [B][H_kv][n-1][d*d + d] adjoint chunk records (reversed) -> U
    float* db;     // [B][H_kv][T][d] dL/dB per row
    float* tot;    // [B][H_kv][n][d] chunk sums of db
    float* stats;  // [B][T][H_q][2] window softmax: log2-sum-exp, sum p dp
    int64_t T;
    int64_t n;
    int H_kv;
    int n_rep;
    int window;
    float alpha;
};

__device__ __forceinline__ void bf8_to_f32(uint4 u, float* f) {
    f[0] = __uint_as_float(u.x << 16);
    f[1] = __uint_as_float(u.x & 0xffff0000u);
    f[2] = __uint_as_float(u.y << 16);
    f[3] = __uint_as_float(u.y & 0xffff0000u);
    f[4] = __uint_as_float(u.z << 16);
    f[5] = __uint_as_float(u.z & 0xffff0000u);
    f[6] = __uint_as_float(u.w << 16);
    f[7] = __uint_as_float(u.w & 0xffff0000u);
}

// Maximum over the 16 lanes of a fragment row group, on DPP.
__device__ __forceinline__ float group16_max(float v) {
    v = fmaxf(v, dpp<kDppXor1>(v));
    v = fmaxf(v, dpp<kDppXor2>(v));
    v = fmaxf(v, dpp<kDppHalfMirror>(v));
    return fmaxf(v, dpp<kDppMirror>(v));
}
// Sum over the 16 lanes of a fragment row group (lanes with the same L >> 4), on DPP.
__device__ __forceinline__ float group16_sum(float v) {
    v += dpp<kDppXor1>(v);
    v += dpp<kDppXor2>(v);
    v += dpp<kDppHalfMirror>(v);
    return v + dpp<kDppMirror>(v);
}

// x = hi + lo + e with hi, lo bf16 (round to nearest even) and |e| <= 2^-17 |x|:
// two bf16 MFMAs against an exact bf16 operand give the fp32-accurate product.
__device__ __forceinline__ void split_bf16x8(const float* x, bf16x8_t& hi, bf16x8_t& lo) {
    uint32_t h[4], l[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        h[i] = pack_bf16x2(x[2 * i], x[2 * i + 1]);
        l[i] = pack_bf16x2(x[2 * i] - __uint_as_float(h[i] << 16), x[2 * i + 1] - __uint_as_float(h[i] & 0xffff0000u));
    }
    hi = __builtin_bit_cast(bf16x8_t, make_uint4(h[0], h[1], h[2], h[3]));
    lo = __builtin_bit_cast(bf16x8_t, make_uint4(l[0], l[1], l[2], l[3]));
}

// Rows 0..63 of a bf16 matrix (row stride `stride` elements) into LDS as
// float32 (pitch in floats); rows >= nv are zero.
// (Fixed trip counts, loads first: every global load of a thread is in
// flight before the first LDS store.)
template <int D, int NTH>
__device__ __forceinline__ void stage_f32(float* dst, int pitch, const bf16_t* src, int64_t stride, int nv) {
    constexpr int PPR = D / 8, PER = 64 * PPR / NTH;
    static_assert(PER * NTH == 64 * PPR, "pieces divide over the threads");
    uint4 u[PER];
#pragma unroll
    for (int e = 0; e < PER; ++e) {
        const int idx = threadIdx.x + e * NTH, r = idx / PPR, c = (idx % PPR) * 8;
        u[e] = r < nv ? *reinterpret_cast<const uint4*>(src + r * stride + c) : make_uint4(0, 0, 0, 0);
    }
#pragma unroll
    for (int e = 0; e < PER; ++e) {
        const int idx = threadIdx.x + e * NTH, r = idx / PPR, c = (idx % PPR) * 8;
        float f[8];
        bf8_to_f32(u[e], f);
        float4* d4 = reinterpret_cast<float4*>(dst + r * pitch + c);
        d4[0] = make_float4(f[0], f[1], f[2], f[3]);
        d4[1] = make_float4(f[4], f[5], f[6], f[7]);
    }
}

// Rows 0..ROWS-1 of a bf16 matrix into LDS as bf16 (pitch in elements);
// rows >= nv are zero.
template <int D, int ROWS, int NTH>
__device__ __forceinline__ void stage_bf16(bf16_t* dst, int pitch, const bf16_t* src, int64_t stride, int nv) {
    constexpr int PPR = D / 8, PER = ROWS * PPR / NTH;
    static_assert(PER * NTH == ROWS * PPR, "pieces divide over the threads");
    uint4 u[PER];
#pragma unroll
    for (int e = 0; e < PER; ++e) {
        const int idx = threadIdx.x + e * NTH, r = idx / PPR, c = (idx % PPR) * 8;
        u[e] = r < nv ? *reinterpret_cast<const uint4*>(src + r * stride + c) : make_uint4(0, 0, 0, 0);
    }
#pragma unroll
    for (int e = 0; e < PER; ++e) {
        const int idx = threadIdx.x + e * NTH, r = idx / PPR, c = (idx % PPR) * 8;
        *reinterpret_cast<uint4*>(dst + r * pitch + c) = u[e];
    }
}

// Softmax over the d channels of each of the 64 rows of x (fp32, in place),
// eight lanes per row; rows >= nv become zero.
template <int D>
__device__ __forceinline__ void row_softmax(float* x, int pitch, int nv) {
    const int row = threadIdx.x >> 3, part = threadIdx.x & 7;
    float* xr = x + row * pitch;
    float v[D / 8];
    float mx = -INFINITY;
#pragma unroll
    for (int i = 0; i < D / 8; ++i) {
        v[i] = xr[part + 8 * i];
        mx = fmaxf(mx, v[i]);
    }
    mx = group8_max(mx);
    float s = 0.f;
#pragma unroll
    for (int i = 0; i < D / 8; ++i) {
        v[i] = fast_exp2((v[i] - mx) * kLog2e);
        s += v[i];
    }
    s = group8_sum(s);
    const float inv = row < nv ? 1.0f / s : 0.0f;
#pragma unroll
    for (int i = 0; i < D / 8; ++i) xr[part + 8 * i] = v[i] * inv;
}

// Chunk set-up shared by the records and gradient kernels: raw k staged in
// sK (fp32) becomes phi(k); sBeta gets the inclusive cumulative log2 gate;
// scratch needs kBT floats. Ends synchronised.
template <int D, int GATE, int BP = D>
__device__ __forceinline__ void chunk_gate(float* sK, int FP, float* sBeta, float* scratch, int nv) {
    const int row = threadIdx.x >> 3, part = threadIdx.x & 7;
    const float* kr = sK + row * FP;
    // log2 sigmoid of the pooled raw key
    if (GATE == 0) {
        float s = 0.f;
#pragma unroll
        for (int i = 0; i < D / 8; ++i) s += kr[part + 8 * i];
        s = group8_sum(s);
        const float l2 = row < nv ? log2_sigmoid(s * (1.0f / D)) : 0.f;
#pragma unroll
        for (int i = 0; i < D / 8; ++i) sBeta[row * BP + part + 8 * i] = l2;
    } else {
#pragma unroll
        for (int i = 0; i < D / 8; ++i) {
            const int c = part + 8 * i;
            int n;
            const float s = pool4_taps<D>(kr, c, n);
            sBeta[row * BP + c] = row < nv ? log2_sigmoid(s / static_cast<float>(n)) : 0.f;
        }
    }
    lds_barrier();
    row_softmax<D>(sK, FP, nv);
    // inclusive scan of the log2 gates over the 64 rows, per channel
    constexpr int P = kBT / D, TPP = 64 / P;
    const int c = threadIdx.x % D, pp = threadIdx.x / D;
    float run = 0.f;
#pragma unroll
    for (int u = 0; u < TPP; ++u) {
        float* e = &sBeta[(pp * TPP + u) * BP + c];
        run += *e;
        *e = run;
    }
    scratch[pp * D + c] = run;
    lds_barrier();
    float off = 0.f;
    for (int j = 0; j < pp; ++j) off += scratch[j * D + c];
#pragma unroll
    for (int u = 0; u < TPP; ++u) sBeta[(pp * TPP + u) * BP + c] += off;
    lds_barrier();
}

// Split values x = hi + lo kept in two bf16 tiles (|x - hi - lo| <= 2^-17 |x|).
// Two adjacent elements (idx even) as one 32-bit store per tile.
__device__ __forceinline__ void put_split2(bf16_t* hi, bf16_t* lo, int idx, float x0, float x1) {
    const uint32_t h = pack_bf16x2(x0, x1);
    *reinterpret_cast<uint32_t*>(hi + idx) = h;
    *reinterpret_cast<uint32_t*>(lo + idx) =
        pack_bf16x2(x0 - __uint_as_float(h << 16), x1 - __uint_as_float(h & 0xffff0000u));
}

// Scalar-gate form of chunk_gate: the gate is one value per token, so the
// cumulative log2 gate is kept per token (sB[64]) instead of broadcast over
// the channels. The prefix is summed in the same order as chunk_gate's (runs
// of 64 / (kBT / D) tokens, then the earlier runs' totals), so both give the
// same bits. scratch needs kBT / D floats. Ends synchronised.
template <int D>
__device__ __forceinline__ void chunk_gate_scalar(float* sK, int FP, float* sB, float* scratch, int nv) {
    const int row = threadIdx.x >> 3, part = threadIdx.x & 7;
    const float* kr = sK + row * FP;
    float s = 0.f;
#pragma unroll
    for (int i = 0; i < D / 8; ++i) s += kr[part + 8 * i];
    s = group8_sum(s);
    if (part == 0) sB[row] = row < nv ? log2_sigmoid(s * (1.0f / D)) : 0.f;
    lds_barrier();
    row_softmax<D>(sK, FP, nv);
    constexpr int P = kBT / D, TPP = 64 / P;
    if (threadIdx.x < P) {
        const int pp = threadIdx.x;
        float run = 0.f;
#pragma unroll
        for (int u = 0; u < TPP; ++u) {
            run += sB[pp * TPP + u];
            sB[pp * TPP + u] = run;
        }
        scratch[pp] = run;
    }
    lds_barrier();
    if (threadIdx.x < 64) {
        const int pp = threadIdx.x / TPP;
        float off = 0.f;
        for (int j = 0; j < pp; ++j) off += scratch[j];
        sB[threadIdx.x] += off;
    }
    lds_barrier();
}

// ---------------------------------------------------------------- records
// Forward record of chunk c (c < n-1): L = sum_t (phik_t (.) 2^(Delta-b_t))^T v_t, lg = Delta.
// Adjoint record of chunk c (c > 0), stored at index n-1-c:
// X = alpha sum_{s,h} (phiq_s^h (.) 2^(b_s))^T dO_s^h, lg = Delta.
// Both are contractions over the chunk's tokens: the scaled feature operand
// is split into bf16 hi + lo tiles, and both operands are read token-major
// with transposing loads (32 tokens per MFMA).
template <int D, int GATE>
__global__ __launch_bounds__(kBT) void bwd_records_kernel(BwdParams p) {
    typedef Mfma<bf16_t> M;
    constexpr int FPK = D + 16, HP = D + 16;
    constexpr int NCB = D / 16;
    constexpr int WPC = 8 / NCB;   // waves per channel block
    constexpr int NE = NCB / WPC;  // column tiles per wave
    // Scalar gate: the cumulative gate is per token, and the workgroup fits
    // twice in a compute unit's LDS.
    constexpr bool SCAL = GATE == 0;
    // raw k -> phi(k) (fp32, pitch FPK); later the hi and lo bf16 tiles [64][HP] in the same bytes
    __shared__ __align__(16) float sK[64 * FPK];
    __shared__ __align__(16) float sBeta[SCAL ? 64 : 64 * D];
    __shared__ __align__(16) bf16_t sV[64 * HP];
    __shared__ __align__(16) bf16_t sO[64 * HP];
    __shared__ float sScr[kBT];
    __shared__ float sDelta[D];
    static_assert(64 * FPK * 4 == 2 * 64 * HP * 2, "hi and lo tiles fill the phi(k) tile");
    bf16_t* sXh = reinterpret_cast<bf16_t*>(sK);
    bf16_t* sXl = sXh + 64 * HP;

    const int c = blockIdx.x, hk = blockIdx.y;
    const int64_t b = blockIdx.z, n = p.n, T = p.T, t0 = 64 * static_cast<int64_t>(c);
    const bool need_fwd = c < n - 1, need_adj = c > 0;
    if (!need_fwd && !need_adj) return;
    const int nv = static_cast<int>(T - t0 < 64 ? T - t0 : 64);
    const int H_q = p.H_kv * p.n_rep;
    const int64_t kvs = static_cast<int64_t>(p.H_kv) * D, qs = static_cast<int64_t>(H_q) * D;
    const int tid = threadIdx.x, lane = tid & 63, col = lane & 15, g = lane >> 4;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave index, uniform
    const int cb = w % NCB, eb0 = (w / NCB) * NE;

    stage_f32<D, kBT>(sK, FPK, p.k + ((b * T + t0) * p.H_kv + hk) * D, kvs, nv);
    stage_bf16<D, 64, kBT>(sV, HP, p.v + ((b * T + t0) * p.H_kv + hk) * D, kvs, nv);
    lds_barrier();
    if constexpr (SCAL) chunk_gate_scalar<D>(sK, FPK, sBeta, sScr, nv);
    else chunk_gate<D, GATE>(sK, FPK, sBeta, sScr, nv);
    // cumulative log2 gate of token t on channel ch
    auto beta = [&](int t, int ch) -> float { return SCAL ? sBeta[t] : sBeta[t * D + ch]; };
    if (tid < D) sDelta[tid] = beta(63, tid);
    lds_barrier();
    const size_t rec = size_t(D) * D + D;

    // acc[u] += (X^T Y)^T over the 64 tokens, X = hi + lo tiles (channel-indexed
    // record rows), Y token-major bf16. The tile is held transposed: lane
    // (col, g) holds record row 16 cb + col, columns 16 (eb0 + u) + 4 g + r,
    // so a row's four values leave with one 16-byte store.
    auto contract = [&](const bf16_t* Y, f32x4_t* acc) {
#pragma unroll
        for (int G = 0; G < 2; ++G) {
            const M::frag xh = load_key_frag(sXh, HP, 32 * G, 16 * cb, lane);
            const M::frag xl = load_key_frag(sXl, HP, 32 * G, 16 * cb, lane);
#pragma unroll
            for (int u = 0; u < NE; ++u) {
                const M::frag y = load_key_frag(Y, HP, 32 * G, 16 * (eb0 + u), lane);
                acc[u] = M::mma(y, xh, acc[u]);
                acc[u] = M::mma(y, xl, acc[u]);
            }
        }
    };
    auto store_record = [&](float* dst, const f32x4_t* acc, float scale) {
#pragma unroll
        for (int u = 0; u < NE; ++u)
            *reinterpret_cast<float4*>(dst + (16 * cb + col) * D + 16 * (eb0 + u) + 4 * g) =
                make_float4(scale * acc[u][0], scale * acc[u][1], scale * acc[u][2], scale * acc[u][3]);
    };
    // element (t, ch) of the split operand lives at [t][ch] of the hi and lo tiles
    auto put_split = [&](int t, int ch, float x) {
        const uint32_t h = pack_bf16x2(x, 0.f) & 0xffffu;
        sXh[t * HP + ch] = static_cast<bf16_t>(h);
        sXl[t * HP + ch] = f32_to_bf16(x - __uint_as_float(h << 16));
    };

    f32x4_t acc[NE];
    if (need_fwd) {
        // K~ = phi(k) (.) 2^(Delta - b), read out before its bytes are reused
        constexpr int PER = 64 * D / kBT;
        float kt[PER];
#pragma unroll
        for (int e = 0; e < PER; ++e) {
            const int idx = tid + e * kBT, t = idx / D, ch = idx % D;
            kt[e] = sK[t * FPK + ch] * fast_exp2(sDelta[ch] - beta(t, ch));
        }
        lds_barrier();
#pragma unroll
        for (int e = 0; e < PER; ++e) {
            const int idx = tid + e * kBT;
            put_split(idx / D, idx % D, kt[e]);
        }
        lds_barrier();
#pragma unroll
        for (int u = 0; u < NE; ++u) acc[u] = zero4();
        contract(sV, acc);
        float* dst = p.fwd + ((b * p.H_kv + hk) * (n - 1) + c) * rec;
        store_record(dst, acc, 1.0f);
        if (tid < D) dst[size_t(D) * D + tid] = sDelta[tid];
    }
    if (need_adj) {
#pragma unroll
        for (int u = 0; u < NE; ++u) acc[u] = zero4();
        // raw q and dO pieces (8 bf16) of a head; the next head's are loaded
        // while the current one is contracted. PPR consecutive lanes hold
        // one token row, so the row softmax of q reduces over those lanes
        // and Q~ = phi(q) (.) 2^(b) goes from registers to the split tiles.
        constexpr int PPR = D / 8, PER = 64 * PPR / kBT;
        static_assert(PPR == 8 || PPR == 16, "a token row spans 8 or 16 lanes");
        uint4 qraw[PER], oraw[PER];
        auto issue_head = [&](int hq) {
            const bf16_t* qg = p.q + ((b * T + t0) * H_q + hq) * D;
            const bf16_t* og = p.dO + ((b * T + t0) * H_q + hq) * D;
#pragma unroll
            for (int e = 0; e < PER; ++e) {
                const int idx = tid + e * kBT, r = idx / PPR, c8 = (idx % PPR) * 8;
                qraw[e] = r < nv ? *reinterpret_cast<const uint4*>(qg + r * qs + c8) : make_uint4(0, 0, 0, 0);
                oraw[e] = r < nv ? *reinterpret_cast<const uint4*>(og + r * qs + c8) : make_uint4(0, 0, 0, 0);
            }
        };
        issue_head(hk * p.n_rep);
        for (int h = 0; h < p.n_rep; ++h) {
            const int hq = hk * p.n_rep + h;
            lds_barrier();  // the previous head's contraction has read the tiles
#pragma unroll
            for (int e = 0; e < PER; ++e) {
                const int idx = tid + e * kBT, r = idx / PPR, c8 = (idx % PPR) * 8;
                float f[8];
                bf8_to_f32(qraw[e], f);
                float mx = f[0];
#pragma unroll
                for (int i = 1; i < 8; ++i) mx = fmaxf(mx, f[i]);
                mx = PPR == 16 ? group16_max(mx) : group8_max(mx);
                float sum = 0.f;
#pragma unroll
                for (int i = 0; i < 8; ++i) {
                    f[i] = fast_exp2((f[i] - mx) * kLog2e);
                    sum += f[i];
                }
                sum = PPR == 16 ? group16_sum(sum) : group8_sum(sum);
                const float inv = r < nv ? 1.0f / sum : 0.0f;
#pragma unroll
                for (int i = 0; i < 8; i += 2)
                    put_split2(sXh, sXl, r * HP + c8 + i, f[i] * inv * fast_exp2(beta(r, c8 + i)),
                               f[i + 1] * inv * fast_exp2(beta(r, c8 + i + 1)));
                *reinterpret_cast<uint4*>(sO + r * HP + c8) = oraw[e];
            }
            if (h + 1 < p.n_rep) issue_head(hq + 1);
            lds_barrier();
            contract(sO, acc);
        }
        float* dst = p.adj + ((b * p.H_kv + hk) * (n - 1) + (n - 1 - c)) * rec;
        store_record(dst, acc, p.alpha);
        if (tid < D) dst[size_t(D) * D + tid] = sDelta[tid];
    }
}

// ---------------------------------------------------------------- GRM gradients
// Sum of N (4 or 8) partials stored contiguously (16-byte aligned).
template <int N>
__device__ __forceinline__ float row_total(const float* p) {
    const float4 a = *reinterpret_cast<const float4*>(p);
    float s = (a.x + a.y) + (a.z + a.w);
    if constexpr (N == 8) {
        const float4 b = *reinterpret_cast<const float4*>(p + 4);
        s += (b.x + b.y) + (b.z + b.w);
    }
    return s;
}
// The lane index as a value the compiler cannot move: code derived from it
// stays where it is written (a rare path inside a loop is not hoisted).
__device__ __forceinline__ int opaque_lane(int lane) {
    asm volatile("" : "+v"(lane));
    return lane;
}
// A split value read back: hi + lo.
__device__ __forceinline__ float get_split(const bf16_t* hi, const bf16_t* lo, int idx) {
    return bf16_to_f32(hi[idx]) + bf16_to_f32(lo[idx]);
}
// Eight elements of a row in the key_pos order of load_key_frag: [kb + 4g, +4) then [kb + 16 + 4g, +4).
__device__ __forceinline__ bf16x8_t row_keypos(const bf16_t* row, int kb, int g) {
    const uint2 a = *reinterpret_cast<const uint2*>(row + kb + 4 * g);
    const uint2 b = *reinterpret_cast<const uint2*>(row + kb + 16 + 4 * g);
    return __builtin_bit_cast(bf16x8_t, make_uint4(a.x, a.y, b.x, b.y));
}
// Element j of a fragment cleared where bit j of `bits` is set.
__device__ __forceinline__ bf16x8_t clear_elems(bf16x8_t f, uint32_t bits) {
    uint4 u = __builtin_bit_cast(uint4, f);
    uint32_t* w = reinterpret_cast<uint32_t*>(&u);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const uint32_t m = (((bits >> (2 * i)) & 1u) ? 0xffffu : 0u) | (((bits >> (2 * i + 1)) & 1u) ? 0xffff0000u : 0u);
        w[i] &= ~m;
    }
    return __builtin_bit_cast(bf16x8_t, u);
}
// acc += X Y for X = xh + xl, Y = yh + yl (the xl yl term is below 2^-16 relative)
__device__ __forceinline__ f32x4_t mma3(bf16x8_t xh, bf16x8_t xl, bf16x8_t yh, bf16x8_t yl, f32x4_t acc) {
    acc = Mfma<bf16_t>::mma(xh, yh, acc);
    acc = Mfma<bf16_t>::mma(xh, yl, acc);
    return Mfma<bf16_t>::mma(xl, yh, acc);
}

// One workgroup per (chunk, key/value head, sequence); the query heads of the
// group are taken one after another. Every [64 x d] result (dphi(q^h),
// dphi(k), dv, dL/dB) is computed transposed, as [d x 64] tiles: wave w owns
// channel block jb = w mod (d/16) and NTI consecutive 16-row tiles, and lane
// (col, g) holds channels 16 jb + 4 g + r of row 16 i + col, so results leave
// as float4 per lane. Computed operands (K^, Q^, A^h, alpha B^h, K~ and the
// states) enter the bf16 MFMA as hi + lo pairs, raw bf16 inputs as they are;
// products whose contraction index is the token run on transposing loads.
template <int D, int GATE>
__global__ __launch_bounds__(kBT) void bwd_chunk_kernel(BwdParams p) {
    typedef Mfma<bf16_t> M;
    typedef M::frag Frag;
    constexpr int FP = D + 4;   // raw k staging pitch (fp32)
    constexpr int XP = D + 8;   // split operand tiles [64][XP]
    constexpr int BP = D + 4;   // cumulative gate pitch
    constexpr int VP = D + 8;   // raw v and dO tiles
    constexpr int AP = 64 + 8;  // A / B tiles [64][AP]
    constexpr int NCB = D / 16;
    constexpr int WPC = 8 / NCB;
    constexpr int NTI = 4 / WPC;
    constexpr int KS = D / M::KSTEP;
    __shared__ __align__(16) bf16_t sQx[2 * 64 * XP];  // Q^ hi, lo; raw k (fp32) during set-up; K~ hi, lo at the end
    __shared__ __align__(16) bf16_t sKx[2 * 64 * XP];  // K^ hi, lo: phik 2^(m-b) (extreme channels: phik)
    __shared__ __align__(16) float sBeta[64 * BP];
    __shared__ __align__(16) bf16_t sV[64 * VP];
    __shared__ __align__(16) bf16_t sO[64 * VP];
    __shared__ __align__(16) bf16_t sAx[2 * 64 * AP];  // A^h[s][t] hi, lo; then alpha B^h[t][s] stored at [s][t]
    __shared__ __align__(16) float sRow[64 * NCB];
    __shared__ __align__(16) float sM[D];
    __shared__ __align__(16) float sDelta[D];
    __shared__ uint32_t sExt[D / 32];
    static_assert(64 * FP * 4 <= 2 * 64 * XP * 2, "raw k staging fits the Q^ tiles");
    static_assert(2 * 64 * AP * 2 >= kBT * 4, "scan scratch fits the A tiles");
    static_assert(2 * 64 * AP * 2 >= WPC * D * 4, "column sums fit the A tiles");
    float* sCol = reinterpret_cast<float*>(sAx);  // [WPC][D], used after the last A / B tile
    float* sKraw = reinterpret_cast<float*>(sQx);
    bf16_t* sQh = sQx;
    bf16_t* sQl = sQx + 64 * XP;
    bf16_t* sKh = sKx;
    bf16_t* sKl = sKx + 64 * XP;
    bf16_t* sAh = sAx;
    bf16_t* sAl = sAx + 64 * AP;

    const int c = blockIdx.x, hk = blockIdx.y;
    const int64_t b = blockIdx.z, n = p.n, T = p.T, t0 = 64 * static_cast<int64_t>(c);
    const int nv = static_cast<int>(T - t0 < 64 ? T - t0 : 64);
    const int H_q = p.H_kv * p.n_rep;
    const int64_t kvs = static_cast<int64_t>(p.H_kv) * D, qs = static_cast<int64_t>(H_q) * D;
    const int tid = threadIdx.x, lane = tid & 63, col = lane & 15, g = lane >> 4;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave index, uniform
    // with one wave per channel block every wave starts at row tile 0 (known at compile time)
    const int jb = w % NCB, i0 = WPC == 1 ? 0 : (w / NCB) * NTI;
    const int cf = 16 * jb + col;     // the channel of this lane's operand fragments
    const int ch0 = 16 * jb + 4 * g;  // the channels ch0 .. ch0 + 3 of this lane's results
    const float alpha = p.alpha;
    const size_t rec = size_t(D) * D + D;

    stage_f32<D, kBT>(sKraw, FP, p.k + ((b * T + t0) * p.H_kv + hk) * D, kvs, nv);
    stage_bf16<D, 64, kBT>(sV, VP, p.v + ((b * T + t0) * p.H_kv + hk) * D, kvs, nv);
    lds_barrier();
    chunk_gate<D, GATE, BP>(sKraw, FP, sBeta, reinterpret_cast<float*>(sAx), nv);
    if (tid < D) {
        const float m = sBeta[31 * BP + tid], dl = sBeta[63 * BP + tid];
        sM[tid] = m;
        sDelta[tid] = dl;
        const bool ext = fmaxf(sBeta[tid] - m, m - dl) > kExtreme;
        const uint64_t bal = __ballot(ext);
        if (lane == 0) {  // wave w covers channels 64 w .. 64 w + 63
            sExt[2 * w] = static_cast<uint32_t>(bal);
            sExt[2 * w + 1] = static_cast<uint32_t>(bal >> 32);
        }
    }
    lds_barrier();
    uint32_t any_ext = 0;
#pragma unroll
    for (int j = 0; j < D / 32; ++j) any_ext |= sExt[j];
    auto is_ext = [&](int ch) -> bool { return (sExt[ch >> 5] >> (ch & 31)) & 1u; };
    for (int idx = tid; idx < 32 * D; idx += kBT) {  // two adjacent channels per item
        const int t = idx / (D / 2), ch = 2 * (idx % (D / 2));
        float x0 = sKraw[t * FP + ch], x1 = sKraw[t * FP + ch + 1];
        if (!is_ext(ch)) x0 *= fast_exp2(sM[ch] - sBeta[t * BP + ch]);
        if (!is_ext(ch + 1)) x1 *= fast_exp2(sM[ch + 1] - sBeta[t * BP + ch + 1]);
        put_split2(sKh, sKl, t * XP + ch, x0, x1);
    }
    const bool colx = is_ext(cf);                             // this lane's fragment channel
    const uint32_t extr = (sExt[ch0 >> 5] >> (ch0 & 31)) & 0xfu;  // result channels ch0 + r
    const Frag fzero = M::zero();
    const float4 m4 = *reinterpret_cast<const float4*>(sM + ch0);
    const float mr[4] = {m4.x, m4.y, m4.z, m4.w};
    // state entering the chunk (fragments S0[cf][e]; none for the first chunk)
    const float* S0row = c > 0 ? p.fwd + ((b * p.H_kv + hk) * (n - 1) + (c - 1)) * rec + size_t(cf) * D : nullptr;
    lds_barrier();

    f32x4_t accK[NTI], accV[NTI], accDB[NTI];
#pragma unroll
    for (int u = 0; u < NTI; ++u) {
        accK[u] = zero4();
        accV[u] = zero4();
        accDB[u] = zero4();
    }
    // four cumulative gates b[row][ch0 .. ch0 + 3]
    auto beta4 = [&](int row) -> float4 { return *reinterpret_cast<const float4*>(sBeta + row * BP + ch0); };
    // four split values [row][ch0 .. ch0 + 3] of a pair of tiles
    auto split4 = [&](const bf16_t* hi, const bf16_t* lo, int idx, float* out) {
        const uint2 h = *reinterpret_cast<const uint2*>(hi + idx), l = *reinterpret_cast<const uint2*>(lo + idx);
        out[0] = __uint_as_float(h.x << 16) + __uint_as_float(l.x << 16);
        out[1] = __uint_as_float(h.x & 0xffff0000u) + __uint_as_float(l.x & 0xffff0000u);
        out[2] = __uint_as_float(h.y << 16) + __uint_as_float(l.y << 16);
        out[3] = __uint_as_float(h.y & 0xffff0000u) + __uint_as_float(l.y & 0xffff0000u);
    };

    // Raw q rows (Q^ layout: 16 lanes per row, channel pairs 2 l + 32 i; a
    // wave's four rows per instruction are 4 apart, so their LDS rows fall on
    // disjoint banks) and raw dO pieces of the next head are loaded while the
    // current head computes.
    const int l16 = lane & 15, sub = lane >> 4;
    auto q_row = [&](int pass) { return (w & 3) + 16 * ((w >> 2) + 2 * pass) + 4 * sub; };
    constexpr int OPT = 64 * D / 8 / kBT;  // dO pieces (8 bf16) per thread
    uint32_t qraw[2][D / 32];
    uint4 oraw[OPT];
    auto issue_head = [&](int hq) {
#pragma unroll
        for (int pass = 0; pass < 2; ++pass) {
            const int row = q_row(pass);
            const bf16_t* qr = p.q + ((b * T + t0 + (row < nv ? row : 0)) * H_q + hq) * D + 2 * l16;
#pragma unroll
            for (int i = 0; i < D / 32; ++i) qraw[pass][i] = row < nv ? *reinterpret_cast<const uint32_t*>(qr + 32 * i) : 0u;
        }
        const bf16_t* og = p.dO + ((b * T + t0) * H_q + hq) * D;
#pragma unroll
        for (int e = 0; e < OPT; ++e) {
            const int idx = tid + e * kBT, r = idx / (D / 8), c8 = (idx % (D / 8)) * 8;
            oraw[e] = r < nv ? *reinterpret_cast<const uint4*>(og + r * qs + c8) : make_uint4(0, 0, 0, 0);
        }
    };
    issue_head(hk * p.n_rep);

    for (int h = 0; h < p.n_rep; ++h) {
        const int hq = hk * p.n_rep + h;
        // Q^ = phi(q) 2^(b-m) (extreme channels: phi(q))
        {
#pragma unroll
            for (int pass = 0; pass < 2; ++pass) {
                const int row = q_row(pass);
                float v[D / 16];
#pragma unroll
                for (int i = 0; i < D / 32; ++i) {
                    v[2 * i] = __uint_as_float(qraw[pass][i] << 16);
                    v[2 * i + 1] = __uint_as_float(qraw[pass][i] & 0xffff0000u);
                }
                float mx = v[0];
#pragma unroll
                for (int i = 1; i < D / 16; ++i) mx = fmaxf(mx, v[i]);
                mx = group16_max(mx);
                float sum = 0.f;
#pragma unroll
                for (int i = 0; i < D / 16; ++i) {
                    v[i] = fast_exp2((v[i] - mx) * kLog2e);
                    sum += v[i];
                }
                sum = group16_sum(sum);
                const float inv = row < nv ? 1.0f / sum : 0.0f;
#pragma unroll
                for (int i = 0; i < D / 32; ++i) {
                    const int ch = 2 * l16 + 32 * i;
                    float y0 = v[2 * i] * inv, y1 = v[2 * i + 1] * inv;
                    const float2 bb = *reinterpret_cast<const float2*>(sBeta + row * BP + ch);
                    if (!is_ext(ch)) y0 *= fast_exp2(bb.x - sM[ch]);
                    if (!is_ext(ch + 1)) y1 *= fast_exp2(bb.y - sM[ch + 1]);
                    put_split2(sQh, sQl, row * XP + ch, y0, y1);
                }
            }
        }
#pragma unroll
        for (int e = 0; e < OPT; ++e) {
            const int idx = tid + e * kBT;
            *reinterpret_cast<uint4*>(sO + (idx / (D / 8)) * VP + (idx % (D / 8)) * 8) = oraw[e];
        }
        if (h + 1 < p.n_rep) issue_head(hq + 1);
        lds_barrier();
        // A^h = alpha dO V^T, zero above the diagonal, as A^T tiles (rows t, columns s):
        // tiles w and w + 8 of the 4 x 4 grid; lane (s col, g) holds t = 16 it + 4 g + r
        {
            const int is0 = w >> 2, it0 = w & 3, is1 = is0 + 2;
            f32x4_t a0 = zero4(), a1 = zero4();
            const bool live0 = it0 <= is0, live1 = it0 <= is1;
#pragma unroll
            for (int k = 0; k < KS; ++k) {
                const Frag x = M::load(sV + (16 * it0 + col) * VP + 8 * g + M::KSTEP * k);
                if (live0) a0 = M::mma(x, M::load(sO + (16 * is0 + col) * VP + 8 * g + M::KSTEP * k), a0);
                if (live1) a1 = M::mma(x, M::load(sO + (16 * is1 + col) * VP + 8 * g + M::KSTEP * k), a1);
            }
            const int s0 = 16 * is0 + col, s1 = 16 * is1 + col, tb = 16 * it0 + 4 * g;
            float y0[4], y1[4];
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                y0[r] = tb + r <= s0 ? alpha * a0[r] : 0.f;
                y1[r] = tb + r <= s1 ? alpha * a1[r] : 0.f;
            }
            put_split2(sAh, sAl, s0 * AP + tb, y0[0], y0[1]);
            put_split2(sAh, sAl, s0 * AP + tb + 2, y0[2], y0[3]);
            put_split2(sAh, sAl, s1 * AP + tb, y1[0], y1[1]);
            put_split2(sAh, sAl, s1 * AP + tb + 2, y1[2], y1[3]);
        }
        lds_barrier();

        // dphi(q^h)^T: state term (accS) and intra-chunk term (accI)
        f32x4_t accS[NTI], accI[NTI];
#pragma unroll
        for (int u = 0; u < NTI; ++u) {
            accS[u] = zero4();
            accI[u] = zero4();
        }
        if (S0row) {
#pragma unroll
            for (int k = 0; k < KS; ++k) {
                const float4 y0 = *reinterpret_cast<const float4*>(S0row + M::KSTEP * k + 8 * g);
                const float4 y1 = *reinterpret_cast<const float4*>(S0row + M::KSTEP * k + 8 * g + 4);
                const float xs[8] = {y0.x, y0.y, y0.z, y0.w, y1.x, y1.y, y1.z, y1.w};
                Frag xh, xl;
                split_bf16x8(xs, xh, xl);
#pragma unroll
                for (int u = 0; u < NTI; ++u) {
                    const Frag y = M::load(sO + (16 * (i0 + u) + col) * VP + 8 * g + M::KSTEP * k);
                    accS[u] = M::mma(xh, y, accS[u]);
                    accS[u] = M::mma(xl, y, accS[u]);
                }
            }
        }
#pragma unroll
        for (int G = 0; G < 2; ++G) {
            Frag xh = load_key_frag(sKh, XP, 32 * G, 16 * jb, lane);
            Frag xl = load_key_frag(sKl, XP, 32 * G, 16 * jb, lane);
            if (colx) {
                xh = fzero;
                xl = fzero;
            }
#pragma unroll
            for (int u = 0; u < NTI; ++u) {
                const int i = i0 + u;
                if (32 * G > 16 * i + 15) continue;  // keys after every query of the tile
                const bf16_t* ar = sAh + (16 * i + col) * AP;
                const bf16_t* al = sAl + (16 * i + col) * AP;
                accI[u] = mma3(xh, xl, row_keypos(ar, 32 * G, g), row_keypos(al, 32 * G, g), accI[u]);
            }
        }
        if (any_ext && extr) {
            // lane indices re-derived here, so that the addresses of this rare
            // path are not hoisted out of the head loop (and spilled) with it
            const int lo = opaque_lane(lane), col_o = lo & 15, ch0_o = 16 * jb + 4 * (lo >> 4);
#pragma unroll
            for (int u = 0; u < NTI; ++u)
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    if (!((extr >> r) & 1u)) continue;
                    const int s = 16 * (i0 + u) + col_o, ch = ch0_o + r;
                    const float bs = sBeta[s * BP + ch];
                    float sum = 0.f;
                    for (int t = 0; t <= s; ++t)
                        sum += get_split(sAh, sAl, s * AP + t) * get_split(sKh, sKl, t * XP + ch) *
                               fast_exp2(bs - sBeta[t * BP + ch]);
                    accI[u][r] = sum;
                }
        }
        float dpq[NTI][4], pq[NTI][4];
#pragma unroll
        for (int u = 0; u < NTI; ++u) {
            const int s = 16 * (i0 + u) + col;
            const float4 b4 = beta4(s);
            const float bs[4] = {b4.x, b4.y, b4.z, b4.w};
            float qh[4];
            split4(sQh, sQl, s * XP + ch0, qh);
            float rsum = 0.f;
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const bool ex = (extr >> r) & 1u;
                const float intra = ex ? accI[u][r] : accI[u][r] * fast_exp2(bs[r] - mr[r]);
                dpq[u][r] = intra + alpha * accS[u][r] * fast_exp2(bs[r]);
                pq[u][r] = ex ? qh[r] : qh[r] * fast_exp2(mr[r] - bs[r]);
                const float pd = pq[u][r] * dpq[u][r];
                accDB[u][r] += pd;
                rsum += pd;
            }
            rsum = group4_sum(rsum);
            if (g == 0) sRow[s * NCB + jb] = rsum;
        }
        lds_barrier();
        // dq^h = phi(q) (.) (dphi(q) - <dphi(q), phi(q)>)
        {
            float* dq = p.dq + ((b * T + t0) * H_q + hq) * D + ch0;
#pragma unroll
            for (int u = 0; u < NTI; ++u) {
                const int s = 16 * (i0 + u) + col;
                const float rs = row_total<NCB>(sRow + s * NCB);
                if (s < nv)
                    *reinterpret_cast<float4*>(dq + s * qs) =
                        make_float4(pq[u][0] * (dpq[u][0] - rs), pq[u][1] * (dpq[u][1] - rs),
                                    pq[u][2] * (dpq[u][2] - rs), pq[u][3] * (dpq[u][3] - rs));
            }
        }
        // dphi(k)^T intra-chunk term, summed over the heads
#pragma unroll
        for (int G = 0; G < 2; ++G) {
            Frag xh = load_key_frag(sQh, XP, 32 * G, 16 * jb, lane);
            Frag xl = load_key_frag(sQl, XP, 32 * G, 16 * jb, lane);
            if (colx) {
                xh = fzero;
                xl = fzero;
            }
#pragma unroll
            for (int u = 0; u < NTI; ++u) {
                const int i = i0 + u;
                if (32 * G + 31 < 16 * i) continue;  // queries before every key of the tile
                accK[u] = mma3(xh, xl, load_key_frag(sAh, AP, 32 * G, 16 * i, lane),
                               load_key_frag(sAl, AP, 32 * G, 16 * i, lane), accK[u]);
            }
        }
        if (any_ext && extr) {
            const int lo = opaque_lane(lane), col_o = lo & 15, ch0_o = 16 * jb + 4 * (lo >> 4);
#pragma unroll
            for (int u = 0; u < NTI; ++u)
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    if (!((extr >> r) & 1u)) continue;
                    const int t = 16 * (i0 + u) + col_o, ch = ch0_o + r;
                    const float bt = sBeta[t * BP + ch];
                    float sum = 0.f;
                    for (int s = t; s < 64; ++s)
                        sum += get_split(sAh, sAl, s * AP + t) * get_split(sQh, sQl, s * XP + ch) *
                               fast_exp2(sBeta[s * BP + ch] - bt);
                    accK[u][r] += sum;
                }
        }
        lds_barrier();

        // alpha B^h[t][s] (s >= t), stored at [s][t] over A^h; tiles w and w + 8 of
        // the 4 x 4 grid (row tile t-block, column tile s-block), computed together
        {
            const int it0 = w >> 2, is0 = w & 3, it1 = it0 + 2;
            const bool live0 = is0 >= it0, live1 = is0 >= it1;
            f32x4_t a0 = zero4(), a1 = zero4();
#pragma unroll
            for (int k = 0; k < KS; ++k) {
                const int cb = M::KSTEP * k + 8 * g;  // this lane group's 8 channels
                const Frag yh = M::load(sQh + (16 * is0 + col) * XP + cb);
                const Frag yl = M::load(sQl + (16 * is0 + col) * XP + cb);
                Frag xh0 = M::load(sKh + (16 * it0 + col) * XP + cb), xl0 = M::load(sKl + (16 * it0 + col) * XP + cb);
                Frag xh1 = M::load(sKh + (16 * it1 + col) * XP + cb), xl1 = M::load(sKl + (16 * it1 + col) * XP + cb);
                if (any_ext) {
                    const uint32_t bits = (sExt[cb >> 5] >> (cb & 31)) & 0xffu;
                    xh0 = clear_elems(xh0, bits);
                    xl0 = clear_elems(xl0, bits);
                    xh1 = clear_elems(xh1, bits);
                    xl1 = clear_elems(xl1, bits);
                }
                if (live0) a0 = mma3(xh0, xl0, yh, yl, a0);
                if (live1) a1 = mma3(xh1, xl1, yh, yl, a1);
            }
            const int s = 16 * is0 + col, tb0 = 16 * it0 + 4 * g, tb1 = 16 * it1 + 4 * g;
            if (any_ext) {
                const int lo = opaque_lane(lane);
                const int s_o = 16 * is0 + (lo & 15), tb0_o = 16 * it0 + 4 * (lo >> 4), tb1_o = 16 * it1 + 4 * (lo >> 4);
#pragma unroll
                for (int r = 0; r < 4; ++r) {
#pragma unroll
                    for (int tl = 0; tl < 2; ++tl) {
                        const int t = (tl ? tb1_o : tb0_o) + r;
                        if (s_o < t) continue;
                        float sum = 0.f;
                        for (int wd = 0; wd < D / 32; ++wd) {
                            uint32_t bits = sExt[wd];
                            while (bits) {
                                const int ch = 32 * wd + __builtin_ctz(bits);
                                bits &= bits - 1;
                                sum += get_split(sKh, sKl, t * XP + ch) * get_split(sQh, sQl, s_o * XP + ch) *
                                       fast_exp2(sBeta[s_o * BP + ch] - sBeta[t * BP + ch]);
                            }
                        }
                        if (tl) a1[r] += sum;
                        else a0[r] += sum;
                    }
                }
            }
            float y0[4], y1[4];
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                y0[r] = s >= tb0 + r ? alpha * a0[r] : 0.f;
                y1[r] = s >= tb1 + r ? alpha * a1[r] : 0.f;
            }
            put_split2(sAh, sAl, s * AP + tb0, y0[0], y0[1]);
            put_split2(sAh, sAl, s * AP + tb0 + 2, y0[2], y0[3]);
            put_split2(sAh, sAl, s * AP + tb1, y1[0], y1[1]);
            put_split2(sAh, sAl, s * AP + tb1 + 2, y1[2], y1[3]);
        }
        lds_barrier();
        // dv^T intra-chunk term: sum_s dO_s[e] alpha B^h[t][s]
#pragma unroll
        for (int G = 0; G < 2; ++G) {
            const Frag x = load_key_frag(sO, VP, 32 * G, 16 * jb, lane);
#pragma unroll
            for (int u = 0; u < NTI; ++u) {
                const int i = i0 + u;
                if (32 * G + 31 < 16 * i) continue;
                accV[u] = M::mma(x, load_key_frag(sAh, AP, 32 * G, 16 * i, lane), accV[u]);
                accV[u] = M::mma(x, load_key_frag(sAl, AP, 32 * G, 16 * i, lane), accV[u]);
            }
        }
        lds_barrier();
    }

    // adjoint entering the chunk's last state (none for the last chunk)
    const float* Ubase = c < n - 1 ? p.adj + ((b * p.H_kv + hk) * (n - 1) + (n - 2 - c)) * rec : nullptr;
    // dphi(k)^T = intra + 2^(Delta-b) (.) (U v), U v from fragments U[cf][e]
    f32x4_t us[NTI];
#pragma unroll
    for (int u = 0; u < NTI; ++u) us[u] = zero4();
    if (Ubase) {
        const float* Urow = Ubase + size_t(cf) * D;
#pragma unroll
        for (int k = 0; k < KS; ++k) {
            const float4 y0 = *reinterpret_cast<const float4*>(Urow + M::KSTEP * k + 8 * g);
            const float4 y1 = *reinterpret_cast<const float4*>(Urow + M::KSTEP * k + 8 * g + 4);
            const float xs[8] = {y0.x, y0.y, y0.z, y0.w, y1.x, y1.y, y1.z, y1.w};
            Frag xh, xl;
            split_bf16x8(xs, xh, xl);
#pragma unroll
            for (int u = 0; u < NTI; ++u) {
                const Frag y = M::load(sV + (16 * (i0 + u) + col) * VP + 8 * g + M::KSTEP * k);
                us[u] = M::mma(xh, y, us[u]);
                us[u] = M::mma(xl, y, us[u]);
            }
        }
    }
    const float4 d4 = *reinterpret_cast<const float4*>(sDelta + ch0);
    const float dlr[4] = {d4.x, d4.y, d4.z, d4.w};
    float dpk[NTI][4], pk[NTI][4];
#pragma unroll
    for (int u = 0; u < NTI; ++u) {
        const int t = 16 * (i0 + u) + col;
        const float4 b4 = beta4(t);
        const float bt[4] = {b4.x, b4.y, b4.z, b4.w};
        float kh[4], kt[4];
        split4(sKh, sKl, t * XP + ch0, kh);
        float rsum = 0.f;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const bool ex = (extr >> r) & 1u;
            const float intra = ex ? accK[u][r] : accK[u][r] * fast_exp2(mr[r] - bt[r]);
            dpk[u][r] = intra + us[u][r] * fast_exp2(dlr[r] - bt[r]);
            pk[u][r] = ex ? kh[r] : kh[r] * fast_exp2(bt[r] - mr[r]);
            kt[r] = pk[u][r] * fast_exp2(dlr[r] - bt[r]);  // K~
            const float pd = pk[u][r] * dpk[u][r];
            accDB[u][r] -= pd;
            rsum += pd;
        }
        put_split2(sQh, sQl, t * XP + ch0, kt[0], kt[1]);
        put_split2(sQh, sQl, t * XP + ch0 + 2, kt[2], kt[3]);
        rsum = group4_sum(rsum);
        if (g == 0) sRow[t * NCB + jb] = rsum;
    }
    lds_barrier();
    // dv^T += U^T K~^T: X = U[32 k + 8 g ..][cf], Y = K~ rows
    if (Ubase) {
        const float* Ucol = Ubase + cf;
#pragma unroll
        for (int k = 0; k < KS; ++k) {
            float xs[8];
#pragma unroll
            for (int j = 0; j < 8; ++j) xs[j] = Ucol[size_t(M::KSTEP * k + 8 * g + j) * D];
            Frag xh, xl;
            split_bf16x8(xs, xh, xl);
#pragma unroll
            for (int u = 0; u < NTI; ++u) {
                const int row = 16 * (i0 + u) + col;
                accV[u] = mma3(xh, xl, M::load(sQh + row * XP + M::KSTEP * k + 8 * g),
                               M::load(sQl + row * XP + M::KSTEP * k + 8 * g), accV[u]);
            }
        }
    }
    // outputs (float4 per lane: channels ch0 .. ch0 + 3 of row t)
    float* dk = p.dk + ((b * T + t0) * p.H_kv + hk) * D + ch0;
    float* dv = p.dv + ((b * T + t0) * p.H_kv + hk) * D + ch0;
    float* db = p.db + ((b * p.H_kv + hk) * T + t0) * D + ch0;
    float csum[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int u = 0; u < NTI; ++u) {
        const int t = 16 * (i0 + u) + col;
        const float rs = row_total<NCB>(sRow + t * NCB);
        if (t < nv) {
            *reinterpret_cast<float4*>(dk + t * kvs) =
                make_float4(pk[u][0] * (dpk[u][0] - rs), pk[u][1] * (dpk[u][1] - rs), pk[u][2] * (dpk[u][2] - rs),
                            pk[u][3] * (dpk[u][3] - rs));
            *reinterpret_cast<float4*>(dv + t * kvs) = make_float4(accV[u][0], accV[u][1], accV[u][2], accV[u][3]);
            *reinterpret_cast<float4*>(db + t * D) = make_float4(accDB[u][0], accDB[u][1], accDB[u][2], accDB[u][3]);
#pragma unroll
            for (int r = 0; r < 4; ++r) csum[r] += accDB[u][r];
        }
    }
    // chunk sums of dL/dB per channel: over this lane's rows, then the 16 row lanes
#pragma unroll
    for (int r = 0; r < 4; ++r) csum[r] = group16_sum(csum[r]);
    if (col == 0) *reinterpret_cast<float4*>(sCol + (w / NCB) * D + ch0) = make_float4(csum[0], csum[1], csum[2], csum[3]);
    lds_barrier();
    if (tid < D) {
        float s = 0.f;
#pragma unroll
        for (int j = 0; j < WPC; ++j) s += sCol[j * D + tid];
        p.tot[((b * p.H_kv + hk) * n + c) * D + tid] = s;
    }
}

// ---------------------------------------------------------------- gate chain
// d ln g_u = sum_{t >= u} dL/dB_t (later chunks through their sums), then
// dx = d ln g (1 - g) and the pool's transpose. Leaves the dk contribution of
// the chunk's row t, channel c at add[t * FP + c] (either sK or sS) and ends
// synchronised. sK, sS: fp32 [64][FP] scratch, sSuf: kST floats.
template <int D, int GATE, int FP>
__device__ __forceinline__ const float* gate_chain(const BwdParams& p, int c, int hk, int64_t b, float* sK, float* sS,
                                                   float* sSuf) {
    const int64_t n = p.n, T = p.T, t0 = 64 * static_cast<int64_t>(c);
    const int nv = static_cast<int>(T - t0 < 64 ? T - t0 : 64);
    const int64_t kvs = static_cast<int64_t>(p.H_kv) * D;
    const int tid = threadIdx.x;
    stage_f32<D, kST>(sK, FP, p.k + ((b * T + t0) * p.H_kv + hk) * D, kvs, nv);
    {
        const float* src = p.db + ((b * p.H_kv + hk) * T + t0) * D;
        constexpr int PPR = D / 4, PER = 64 * PPR / kST;
        float4 u[PER];
#pragma unroll
        for (int e = 0; e < PER; ++e) {
            const int idx = tid + e * kST, t = idx / PPR, c4 = (idx % PPR) * 4;
            u[e] = t < nv ? *reinterpret_cast<const float4*>(src + t * D + c4) : make_float4(0.f, 0.f, 0.f, 0.f);
        }
#pragma unroll
        for (int e = 0; e < PER; ++e) {
            const int idx = tid + e * kST, t = idx / PPR, c4 = (idx % PPR) * 4;
            *reinterpret_cast<float4*>(sS + t * FP + c4) = u[e];
        }
    }
    {
        // sum of the chunk sums after this chunk: thread (channel, part) takes
        // every P-th later chunk, 16 loads in flight at a time
        constexpr int P = kST / D, U = 16;
        const int ch = tid % D, part = tid / D;
        const float* tot = p.tot + (b * p.H_kv + hk) * n * D + ch;
        float a[U];
#pragma unroll
        for (int u = 0; u < U; ++u) a[u] = 0.f;
        for (int64_t j0 = c + 1 + part; j0 < n; j0 += U * P) {
#pragma unroll
            for (int u = 0; u < U; ++u) {
                const int64_t j = j0 + u * P;
                if (j < n) a[u] += tot[j * D];
            }
        }
#pragma unroll
        for (int u = 1; u < U; ++u) a[0] += a[u];
        sSuf[part * D + ch] = a[0];
    }
    lds_barrier();
    if (tid < D) {
        // reverse inclusive scan down the chunk's rows, in registers
        float run = 0.f;
#pragma unroll
        for (int j = 0; j < kST / D; ++j) run += sSuf[j * D + tid];
        float r[64];
#pragma unroll
        for (int t = 0; t < 64; ++t) r[t] = sS[t * FP + tid];  // rows >= nv hold 0
#pragma unroll
        for (int t = 63; t >= 0; --t) {
            run += r[t];
            sS[t * FP + tid] = run;
        }
    }
    lds_barrier();
    if (GATE == 0) {
        // four lanes per row: ds_t = (sum_c d ln g_t[c]) (1 - g_t) / d on every channel
        const int row = tid >> 2, part = tid & 3;
        float sk = 0.f, ss = 0.f;
        for (int i = part; i < D; i += 4) {
            sk += sK[row * FP + i];
            ss += sS[row * FP + i];
        }
        sk += dpp<kDppXor1>(sk);
        sk += dpp<kDppXor2>(sk);
        ss += dpp<kDppXor1>(ss);
        ss += dpp<kDppXor2>(ss);
        const float ds = ss * sigmoidf_stable(-sk * (1.0f / D)) * (1.0f / D);
        lds_barrier();
        for (int i = part; i < D; i += 4) sS[row * FP + i] = ds;
        lds_barrier();
        return sS;
    }
    for (int idx = tid; idx < 64 * D; idx += kST) {
        const int t = idx / D, ch = idx % D;
        int n;
        const float sum = pool4_taps<D>(sK + t * FP, ch, n);
        const float x = sum / static_cast<float>(n);
        sS[t * FP + ch] *= sigmoidf_stable(-x) / static_cast<float>(n);
    }
    lds_barrier();
    // pool transpose: channel c'' collects channels c'' - 2 .. c'' + 1
    for (int idx = tid; idx < 64 * D; idx += kST) {
        const int t = idx / D, ch = idx % D;
        float add = 0.f;
#pragma unroll
        for (int j = ch - 2; j <= ch + 1; ++j)
            if (j >= 0 && j < D) add += sS[t * FP + j];
        sK[t * FP + ch] = add;  // raw k no longer needed
    }
    lds_barrier();
    return sK;
}

// ---------------------------------------------------------------- window: queries
// One workgroup per (chunk, key/value head, sequence); wave i holds query
// tile i of the chunk, all query heads of the group in turn. Keys of the
// previous and the current chunk are staged once (token-major, rows 8 banks
// apart for the transposing reads). Key tiles are taken in aligned pairs
// (2G, 2G + 1), the 32-key groups of the dq product.
template <int D>
__global__ __launch_bounds__(kST) void bwd_swa_q_kernel(BwdParams p) {
    typedef Mfma<bf16_t> M;
    constexpr int HP = D + 16, KS = D / M::KSTEP, NCB = D / 16;
    __shared__ __align__(16) bf16_t sK[128 * HP];
    __shared__ __align__(16) bf16_t sV[128 * HP];

    const int c = blockIdx.x, hk = blockIdx.y;
    const int64_t b = blockIdx.z, T = p.T, t0 = 64 * static_cast<int64_t>(c);
    const int H_q = p.H_kv * p.n_rep;
    const int64_t qs = static_cast<int64_t>(H_q) * D;
    const int tid = threadIdx.x, lane = tid & 63, col = lane & 15, g = lane >> 4;
    const int wi = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave index, uniform
    // key row kk of the tiles is token t0 - 64 + kk
    {
        const int64_t first = t0 - 64;
        const int lo = first < 0 ? 64 : 0;
        const int hi = static_cast<int>(T - first < 128 ? T - first : 128);
        constexpr int PPR = D / 8, PER = 128 * PPR / kST;
        uint4 ku[PER], vu[PER];
#pragma unroll
        for (int e = 0; e < PER; ++e) {
            const int idx = tid + e * kST, r = idx / PPR, cpos = (idx % PPR) * 8;
            const bool ok = r >= lo && r < hi;
            const int64_t off = ((b * T + first + (ok ? r : lo)) * p.H_kv + hk) * D + cpos;
            ku[e] = ok ? *reinterpret_cast<const uint4*>(p.k + off) : make_uint4(0, 0, 0, 0);
            vu[e] = ok ? *reinterpret_cast<const uint4*>(p.v + off) : make_uint4(0, 0, 0, 0);
        }
#pragma unroll
        for (int e = 0; e < PER; ++e) {
            const int idx = tid + e * kST, r = idx / PPR, cpos = (idx % PPR) * 8;
            *reinterpret_cast<uint4*>(sK + r * HP + cpos) = ku[e];
            *reinterpret_cast<uint4*>(sV + r * HP + cpos) = vu[e];
        }
    }
    lds_barrier();
    const int w = p.window;
    const float sc = kLog2e * rsqrtf(static_cast<float>(D));
    const float beta = 1.0f - p.alpha;
    const int qq = 64 + 16 * wi + col;  // this lane's query in key-row coordinates
    const int64_t qtok = t0 + 16 * wi + col;
    const int kt0 = 2 * (wi >> 1);                   // first key tile of the aligned pairs
    const int ktlo = max(wi, (64 + 16 * wi - w + 1) >> 4);  // live key tiles: ktlo .. wi + 4
    const int64_t qrow = qtok < T ? qtok : T - 1;

    // this lane's query row of head hq: q and dO fragments; the next head's are
    // loaded while the current one computes
    M::frag qf[KS], of[KS];
    auto load_frags = [&](int hq, M::frag* qd, M::frag* od) {
        const bf16_t* qr = p.q + (b * T + qrow) * qs + hq * D + 8 * g;
        const bf16_t* orow = p.dO + (b * T + qrow) * qs + hq * D + 8 * g;
#pragma unroll
        for (int k = 0; k < KS; ++k) {
            qd[k] = M::load(qr + M::KSTEP * k);
            od[k] = M::load(orow + M::KSTEP * k);
        }
    };
    load_frags(hk * p.n_rep, qf, of);
    for (int h = 0; h < p.n_rep; ++h) {
        const int hq = hk * p.n_rep + h;
        // this head's dq rows (added to below), in flight during the scores
        float* dqrow = p.dq + (b * T + qrow) * qs + hq * D + 4 * g;
        float4 dqv[NCB];
#pragma unroll
        for (int cb = 0; cb < NCB; ++cb) dqv[cb] = *reinterpret_cast<const float4*>(dqrow + 16 * cb);
        // scores and value products on key tiles kt0 .. kt0 + 5: lane (query col, g) holds keys 16 kt + 4 g + r
        f32x4_t z[6], dp[6];
        float mx = -INFINITY;
#pragma unroll
        for (int j = 0; j < 6; ++j) {
            const int kt = kt0 + j;
            z[j] = f32x4_t{-INFINITY, -INFINITY, -INFINITY, -INFINITY};  // p = 0 outside every window
            dp[j] = zero4();
            if (kt < ktlo || kt > wi + 4) continue;
            z[j] = zero4();
#pragma unroll
            for (int k = 0; k < KS; ++k) {
                z[j] = M::mma(M::load(sK + (16 * kt + col) * HP + 8 * g + M::KSTEP * k), qf[k], z[j]);
                dp[j] = M::mma(M::load(sV + (16 * kt + col) * HP + 8 * g + M::KSTEP * k), of[k], dp[j]);
            }
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int kk = 16 * kt + 4 * g + r;
                const bool live = kk <= qq && kk > qq - w && t0 - 64 + kk >= 0;
                z[j][r] = live ? z[j][r] * sc : -INFINITY;
                mx = fmaxf(mx, z[j][r]);
            }
        }
        if (h + 1 < p.n_rep) load_frags(hq + 1, qf, of);  // the fragments of this head are consumed
        mx = group4_max(mx);
        float l = 0.f;
#pragma unroll
        for (int j = 0; j < 6; ++j)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                z[j][r] = fast_exp2(z[j][r] - mx);
                l += z[j][r];
            }
        l = group4_sum(l);
        const float inv = 1.0f / l;
        float ds = 0.f;
#pragma unroll
        for (int j = 0; j < 6; ++j)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                z[j][r] *= inv;
                dp[j][r] *= beta;
                ds += z[j][r] * dp[j][r];
            }
        ds = group4_sum(ds);
        if (g == 0 && qtok < T) {
            float* st = p.stats + ((b * T + qtok) * H_q + hq) * 2;
            st[0] = mx + fast_log2(l);
            st[1] = ds;
        }
        // dz = p (dp - sum p dp), split into bf16 hi + lo per aligned key pair
        M::frag zh[3], zl[3];
#pragma unroll
        for (int G = 0; G < 3; ++G) {
            float v8[8];
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                v8[r] = z[2 * G][r] * (dp[2 * G][r] - ds);
                v8[4 + r] = z[2 * G + 1][r] * (dp[2 * G + 1][r] - ds);
            }
            split_bf16x8(v8, zh[G], zl[G]);
        }
        // dq^T[c][q] = sum_key k[key][c] dz[key][q] / sqrt(d)
        const float rs = rsqrtf(static_cast<float>(D));
#pragma unroll
        for (int cb = 0; cb < NCB; ++cb) {
            f32x4_t a = zero4();
#pragma unroll
            for (int G = 0; G < 3; ++G) {
                const int kt = kt0 + 2 * G;
                if (kt + 1 < ktlo || kt > wi + 4) continue;
                const M::frag kx = load_key_frag(sK, HP, 16 * kt, 16 * cb, lane);
                a = M::mma(kx, zh[G], a);
                a = M::mma(kx, zl[G], a);
            }
            if (qtok < T) {
                float4 o = dqv[cb];
                o.x += a[0] * rs;
                o.y += a[1] * rs;
                o.z += a[2] * rs;
                o.w += a[3] * rs;
                *reinterpret_cast<float4*>(dqrow + 16 * cb) = o;
            }
        }
    }
}

// ---------------------------------------------------------------- window: keys
// One workgroup per (chunk, key/value head, sequence); wave i holds key tile
// i of the chunk. The queries that can see those keys are in this chunk and
// the next, taken in aligned query-tile pairs (2G, 2G + 1); dk and dv are
// summed over the query heads of the group.
template <int D, int GATE, bool WIN>
__global__ __launch_bounds__(kST) __attribute__((amdgpu_waves_per_eu(2))) void bwd_swa_k_kernel(BwdParams p) {
    typedef Mfma<bf16_t> M;
    constexpr int HP = D + 16, KS = D / M::KSTEP, NCB = D / 16;
    __shared__ __align__(16) bf16_t sQ[128 * HP];
    __shared__ __align__(16) bf16_t sO[128 * HP];
    __shared__ float sL[kST];  // window statistics: log2-sum-exp in [0, 128), sum p dp in [128, 256); gate scratch later
    float* sDs = sL + 128;

    const int c = blockIdx.x, hk = blockIdx.y;
    const int64_t b = blockIdx.z, T = p.T, t0 = 64 * static_cast<int64_t>(c);
    const int H_q = p.H_kv * p.n_rep;
    const int64_t kvs = static_cast<int64_t>(p.H_kv) * D, qs = static_cast<int64_t>(H_q) * D;
    const int tid = threadIdx.x, lane = tid & 63, col = lane & 15, g = lane >> 4;
    const int wi = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave index, uniform
    const int w = p.window;
    const float sc = kLog2e * rsqrtf(static_cast<float>(D));
    const float beta = 1.0f - p.alpha;
    const int nq = static_cast<int>(T - t0 < 128 ? T - t0 : 128);  // query rows present
    const int kj = 16 * wi + col;                                   // this lane's key (chunk-local)
    const int64_t ktok = t0 + kj;
    const int64_t krow = ktok < T ? ktok : T - 1;
    const int qt0 = 2 * (wi >> 1);                     // first query tile of the aligned pairs
    const int qthi = min(7, (16 * wi + 15 + w - 1) >> 4);  // live query tiles: wi .. qthi

    M::frag kf[KS], vf[KS];
    {
        const bf16_t* kr = p.k + (b * T + krow) * kvs + hk * D + 8 * g;
        const bf16_t* vr = p.v + (b * T + krow) * kvs + hk * D + 8 * g;
#pragma unroll
        for (int k = 0; k < KS; ++k) {
            kf[k] = M::load(kr + M::KSTEP * k);
            vf[k] = M::load(vr + M::KSTEP * k);
        }
    }
    f32x4_t adk[NCB], adv[NCB];
#pragma unroll
    for (int j = 0; j < NCB; ++j) {
        adk[j] = zero4();
        adv[j] = zero4();
    }
    for (int h = 0; h < (WIN ? p.n_rep : 0); ++h) {
        const int hq = hk * p.n_rep + h;
        lds_barrier();
        stage_bf16<D, 128, kST>(sQ, HP, p.q + ((b * T + t0) * H_q + hq) * D, qs, nq);
        stage_bf16<D, 128, kST>(sO, HP, p.dO + ((b * T + t0) * H_q + hq) * D, qs, nq);
        if (tid < 128) {
            const bool ok = tid < nq;
            const float* st = p.stats + ((b * T + t0 + (ok ? tid : 0)) * H_q + hq) * 2;
            sL[tid] = ok ? st[0] : 0.f;
            sDs[tid] = ok ? st[1] : 0.f;
        }
        lds_barrier();
        // S[q][key] on query tiles qt0 .. qt0 + 5: lane (key col, g) holds queries 16 qt + 4 g + r
        M::frag ph[3], pl[3], dh[3], dl[3];
#pragma unroll
        for (int G = 0; G < 3; ++G) {
            float pv[8], dv8[8];
#pragma unroll
            for (int half = 0; half < 2; ++half) {
                const int qt = qt0 + 2 * G + half;
                f32x4_t z = zero4(), dp = zero4();
                const bool live_tile = qt >= wi && qt <= qthi;
                if (live_tile) {
#pragma unroll
                    for (int k = 0; k < KS; ++k) {
                        z = M::mma(M::load(sQ + (16 * qt + col) * HP + 8 * g + M::KSTEP * k), kf[k], z);
                        dp = M::mma(M::load(sO + (16 * qt + col) * HP + 8 * g + M::KSTEP * k), vf[k], dp);
                    }
                }
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int qi = 16 * qt + 4 * g + r;
                    const bool live = live_tile && qi >= kj && qi < kj + w && qi < nq;
                    const float pr = live ? fast_exp2(z[r] * sc - sL[qi]) : 0.f;
                    pv[4 * half + r] = beta * pr;
                    dv8[4 * half + r] = live ? pr * (beta * dp[r] - sDs[qi]) : 0.f;
                }
            }
            split_bf16x8(dv8, dh[G], dl[G]);
            split_bf16x8(pv, ph[G], pl[G]);
        }
        // dk^T[c][key] += sum_q q[q][c] dz[q][key]; dv^T[e][key] += sum_q dO[q][e] beta p[q][key]
#pragma unroll
        for (int cb = 0; cb < NCB; ++cb) {
#pragma unroll
            for (int G = 0; G < 3; ++G) {
                const int qt = qt0 + 2 * G;
                if (qt + 1 < wi || qt > qthi) continue;
                const M::frag qx = load_key_frag(sQ, HP, 16 * qt, 16 * cb, lane);
                const M::frag ox = load_key_frag(sO, HP, 16 * qt, 16 * cb, lane);
                adk[cb] = M::mma(qx, dh[G], adk[cb]);
                adk[cb] = M::mma(qx, dl[G], adk[cb]);
                adv[cb] = M::mma(ox, ph[G], adv[cb]);
                adv[cb] = M::mma(ox, pl[G], adv[cb]);
            }
        }
    }
    // the gate's share of dk for this chunk's keys, in the bytes of the q and dO tiles
    constexpr int GFP = D + 4;
    static_assert(64 * GFP * 4 <= 128 * HP * 2, "gate scratch fits a query tile");
    lds_barrier();
    const float* gadd = gate_chain<D, GATE, GFP>(p, c, hk, b, reinterpret_cast<float*>(sQ), reinterpret_cast<float*>(sO),
                                                 sL);
    if (ktok < T) {
        const float rs = rsqrtf(static_cast<float>(D));
#pragma unroll
        for (int cb = 0; cb < NCB; ++cb) {
            const float4 ga = *reinterpret_cast<const float4*>(gadd + kj * GFP + 16 * cb + 4 * g);
            float4* pk = reinterpret_cast<float4*>(p.dk + (b * T + ktok) * kvs + hk * D + 16 * cb + 4 * g);
            float4 x = *pk;
            x.x += adk[cb][0] * rs + ga.x;
            x.y += adk[cb][1] * rs + ga.y;
            x.z += adk[cb][2] * rs + ga.z;
            x.w += adk[cb][3] * rs + ga.w;
            *pk = x;
            if (WIN) {
                float4* pv = reinterpret_cast<float4*>(p.dv + (b * T + ktok) * kvs + hk * D + 16 * cb + 4 * g);
                float4 y = *pv;
                y.x += adv[cb][0];
                y.y += adv[cb][1];
                y.z += adv[cb][2];
                y.w += adv[cb][3];
                *pv = y;
            }
        }
    }
}

template <int D, int GATE>
hipError_t launch_bwd_t(const BackwardArgs& a) {
    BwdParams p;
    p.q = static_cast<const bf16_t*>(a.q);
    p.k = static_cast<const bf16_t*>(a.k);
    p.v = static_cast<const bf16_t*>(a.v);
    p.dO = static_cast<const bf16_t*>(a.dO);
    p.dq = a.dq;
    p.dk = a.dk;
    p.dv = a.dv;
    p.T = a.T;
    p.n = (a.T + 63) / 64;
    p.H_kv = a.H_kv;
    p.n_rep = a.n_rep;
    p.window = a.window;
    p.alpha = a.alpha;
    const size_t rec = size_t(D) * D + D;
    const size_t nrec = size_t(a.B) * a.H_kv * size_t(p.n - 1) * rec;
    p.fwd = a.workspace;
    p.adj = p.fwd + nrec;
    p.db = p.adj + nrec;
    p.tot = p.db + size_t(a.B) * a.H_kv * a.T * D;
    p.stats = p.tot + size_t(a.B) * a.H_kv * p.n * D;
    hipStream_t st = static_cast<hipStream_t>(a.stream);
    const dim3 grid(static_cast<unsigned>(p.n), a.H_kv, static_cast<unsigned>(a.B));
    if (p.n > 1) {
        hipLaunchKernelGGL((bwd_records_kernel<D, GATE>), grid, dim3(kBT), 0, st, p);
        hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
        e = launch_carry_scan(p.fwd, p.n, a.H_kv, a.B, D, a.stream);
        if (e != hipSuccess) return e;
        e = launch_carry_scan(p.adj, p.n, a.H_kv, a.B, D, a.stream);
        if (e != hipSuccess) return e;
    }
    hipLaunchKernelGGL((bwd_chunk_kernel<D, GATE>), grid, dim3(kBT), 0, st, p);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    if (p.alpha != 1.0f) {
        hipLaunchKernelGGL((bwd_swa_q_kernel<D>), grid, dim3(kST), 0, st, p);
        e = hipGetLastError();
        if (e != hipSuccess) return e;
        hipLaunchKernelGGL((bwd_swa_k_kernel<D, GATE, true>), grid, dim3(kST), 0, st, p);
    } else {
        // no window part: only the gate's share of dk
        hipLaunchKernelGGL((bwd_swa_k_kernel<D, GATE, false>), grid, dim3(kST), 0, st, p);
    }
    return hipGetLastError();
}

}  // namespace

hipError_t launch_backward(const BackwardArgs& a) {
    if (a.T == 0 || a.B == 0) return hipSuccess;
    if (a.d == 64) return a.gate ? launch_bwd_t<64, 1>(a) : launch_bwd_t<64, 0>(a);
    return a.gate ? launch_bwd_t<128, 1>(a) : launch_bwd_t<128, 0>(a);
}

}  // namespace liger
