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
//   bwd_swa_k_kernel   : per key tile: dk += .., dv += ..
//   bwd_gate_kernel    : suffix sums of dL/dB, sigmoid and pool transpose: dk += ..
// Contractions with raw bf16 operands use the bf16 MFMA (products exact in
// fp32); those with computed operands use the fp32 MFMA.
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

__device__ __forceinline__ f32x4_t mma4(float x, float y, f32x4_t acc) {
    return __builtin_amdgcn_mfma_f32_16x16x4f32(x, y, acc, 0, 0, 0);
}

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

// Sum over the 16 lanes of a fragment row group (lanes with the same L >> 4).
__device__ __forceinline__ float group16_sum(float v) {
#pragma unroll
    for (int o = 1; o < 16; o <<= 1) v += __shfl_xor(v, o, 64);
    return v;
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
template <int D, int NTH>
__device__ __forceinline__ void stage_f32(float* dst, int pitch, const bf16_t* src, int64_t stride, int nv) {
    constexpr int PPR = D / 8;
    for (int idx = threadIdx.x; idx < 64 * PPR; idx += NTH) {
        const int r = idx / PPR, c = (idx % PPR) * 8;
        uint4 u = make_uint4(0, 0, 0, 0);
        if (r < nv) u = *reinterpret_cast<const uint4*>(src + r * stride + c);
        float f[8];
        bf8_to_f32(u, f);
        float4* d4 = reinterpret_cast<float4*>(dst + r * pitch + c);
        d4[0] = make_float4(f[0], f[1], f[2], f[3]);
        d4[1] = make_float4(f[4], f[5], f[6], f[7]);
    }
}

// Rows 0..ROWS-1 of a bf16 matrix into LDS as bf16 (pitch in elements);
// rows >= nv are zero.
template <int D, int ROWS, int NTH>
__device__ __forceinline__ void stage_bf16(bf16_t* dst, int pitch, const bf16_t* src, int64_t stride, int nv) {
    constexpr int PPR = D / 8;
    for (int idx = threadIdx.x; idx < ROWS * PPR; idx += NTH) {
        const int r = idx / PPR, c = (idx % PPR) * 8;
        uint4 u = make_uint4(0, 0, 0, 0);
        if (r < nv) u = *reinterpret_cast<const uint4*>(src + r * stride + c);
        *reinterpret_cast<uint4*>(dst + r * pitch + c) = u;
    }
}

// Softmax over the d channels of each of the 64 rows of x (fp32, in place),
// eight lanes per row; rows >= nv become zero. With SCALE, element (t, c) is
// then multiplied by 2^(e[t][c]) unless channel c is flagged in `keep`.
template <int D, bool SCALE>
__device__ __forceinline__ void row_softmax(float* x, int pitch, int nv, const float* e, const float* mref,
                                            const uint32_t* keep) {
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
    for (int i = 0; i < D / 8; ++i) {
        const int c = part + 8 * i;
        float y = v[i] * inv;
        if (SCALE) {
            const bool ext = (keep[c >> 5] >> (c & 31)) & 1u;
            if (!ext) y *= fast_exp2(e[row * D + c] - mref[c]);
        }
        xr[c] = y;
    }
}

// Chunk set-up shared by the records and gradient kernels: raw k staged in
// sK (fp32) becomes phi(k); sBeta gets the inclusive cumulative log2 gate;
// scratch needs kBT floats. Ends synchronised.
template <int D, int GATE>
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
        for (int i = 0; i < D / 8; ++i) sBeta[row * D + part + 8 * i] = l2;
    } else {
#pragma unroll
        for (int i = 0; i < D / 8; ++i) {
            const int c = part + 8 * i;
            const int lo = c > 0 ? c - 1 : 0, hi = c + 3 < D ? c + 3 : D;
            float s = 0.f;
            for (int j = lo; j < hi; ++j) s += kr[j];
            sBeta[row * D + c] = row < nv ? log2_sigmoid(s / static_cast<float>(hi - lo)) : 0.f;
        }
    }
    __syncthreads();
    row_softmax<D, false>(sK, FP, nv, nullptr, nullptr, nullptr);
    // inclusive scan of the log2 gates over the 64 rows, per channel
    constexpr int P = kBT / D, TPP = 64 / P;
    const int c = threadIdx.x % D, pp = threadIdx.x / D;
    float run = 0.f;
#pragma unroll
    for (int u = 0; u < TPP; ++u) {
        float* e = &sBeta[(pp * TPP + u) * D + c];
        run += *e;
        *e = run;
    }
    scratch[pp * D + c] = run;
    __syncthreads();
    float off = 0.f;
    for (int j = 0; j < pp; ++j) off += scratch[j * D + c];
#pragma unroll
    for (int u = 0; u < TPP; ++u) sBeta[(pp * TPP + u) * D + c] += off;
    __syncthreads();
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
    constexpr int FPK = D + 16, FP = D + 4, HP = D + 16;
    constexpr int NCB = D / 16;
    constexpr int WPC = 8 / NCB;   // waves per channel block
    constexpr int NE = NCB / WPC;  // column tiles per wave
    // raw k -> phi(k) (fp32, pitch FPK); later the hi and lo bf16 tiles [64][HP] in the same bytes
    __shared__ __align__(16) float sK[64 * FPK];
    __shared__ __align__(16) float sQ[64 * FP];
    __shared__ __align__(16) float sBeta[64 * D];
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
    __syncthreads();
    chunk_gate<D, GATE>(sK, FPK, sBeta, sScr, nv);
    if (tid < D) sDelta[tid] = sBeta[63 * D + tid];
    __syncthreads();
    const size_t rec = size_t(D) * D + D;

    // acc[u] += X Y over the 64 tokens, X = hi + lo tiles (channel-indexed rows), Y token-major bf16
    auto contract = [&](const bf16_t* Y, f32x4_t* acc) {
#pragma unroll
        for (int G = 0; G < 2; ++G) {
            const M::frag xh = load_key_frag(sXh, HP, 32 * G, 16 * cb, lane);
            const M::frag xl = load_key_frag(sXl, HP, 32 * G, 16 * cb, lane);
#pragma unroll
            for (int u = 0; u < NE; ++u) {
                const M::frag y = load_key_frag(Y, HP, 32 * G, 16 * (eb0 + u), lane);
                acc[u] = M::mma(xh, y, acc[u]);
                acc[u] = M::mma(xl, y, acc[u]);
            }
        }
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
            kt[e] = sK[t * FPK + ch] * fast_exp2(sDelta[ch] - sBeta[t * D + ch]);
        }
        __syncthreads();
#pragma unroll
        for (int e = 0; e < PER; ++e) {
            const int idx = tid + e * kBT;
            put_split(idx / D, idx % D, kt[e]);
        }
        __syncthreads();
#pragma unroll
        for (int u = 0; u < NE; ++u) acc[u] = zero4();
        contract(sV, acc);
        float* dst = p.fwd + ((b * p.H_kv + hk) * (n - 1) + c) * rec;
#pragma unroll
        for (int u = 0; u < NE; ++u)
#pragma unroll
            for (int r = 0; r < 4; ++r) dst[(16 * cb + 4 * g + r) * D + 16 * (eb0 + u) + col] = acc[u][r];
        if (tid < D) dst[size_t(D) * D + tid] = sDelta[tid];
    }
    if (need_adj) {
#pragma unroll
        for (int u = 0; u < NE; ++u) acc[u] = zero4();
        for (int h = 0; h < p.n_rep; ++h) {
            const int hq = hk * p.n_rep + h;
            __syncthreads();
            stage_f32<D, kBT>(sQ, FP, p.q + ((b * T + t0) * H_q + hq) * D, qs, nv);
            stage_bf16<D, 64, kBT>(sO, HP, p.dO + ((b * T + t0) * H_q + hq) * D, qs, nv);
            __syncthreads();
            // Q~ = phi(q) (.) 2^(b), written as the split operand
            {
                const int row = tid >> 3, part = tid & 7;
                const float* xr = sQ + row * FP;
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
                for (int i = 0; i < D / 8; ++i) {
                    const int cc = part + 8 * i;
                    put_split(row, cc, v[i] * inv * fast_exp2(sBeta[row * D + cc]));
                }
            }
            __syncthreads();
            contract(sO, acc);
        }
        float* dst = p.adj + ((b * p.H_kv + hk) * (n - 1) + (n - 1 - c)) * rec;
#pragma unroll
        for (int u = 0; u < NE; ++u)
#pragma unroll
            for (int r = 0; r < 4; ++r)
                dst[(16 * cb + 4 * g + r) * D + 16 * (eb0 + u) + col] = p.alpha * acc[u][r];
        if (tid < D) dst[size_t(D) * D + tid] = sDelta[tid];
    }
}

// ---------------------------------------------------------------- GRM gradients
// One workgroup per (chunk, key/value head, sequence); the query heads of the
// group are taken one after another. Every [64 x d] result (dphi(q^h),
// dphi(k), dv, dL/dB) uses the same tiles: wave w owns column block
// w mod (d/16) and NTI consecutive 16-row tiles.
template <int D, int GATE>
__global__ __launch_bounds__(kBT) void bwd_chunk_kernel(BwdParams p) {
    typedef Mfma<bf16_t> M;
    constexpr int FP = D + 4, HP = D + 8, AP = 68;
    constexpr int NCB = D / 16;
    constexpr int WPC = 8 / NCB;
    constexpr int NTI = 4 / WPC;
    constexpr int KQ = D / 4;  // contraction elements per lane group in the permuted products
    constexpr int KS = D / M::KSTEP;
    __shared__ __align__(16) float sKh[64 * FP];  // K^: phik 2^(m-b) (extreme channels: phik)
    __shared__ __align__(16) float sQ[64 * FP];   // Q^ of the current head; afterwards K~
    __shared__ __align__(16) float sBeta[64 * D];
    __shared__ __align__(16) bf16_t sV[64 * HP];
    __shared__ __align__(16) bf16_t sO[64 * HP];
    __shared__ __align__(16) float sA[64 * AP];   // A^h[s][t]; then alpha B^h stored as [s][t]
    __shared__ float sRow[64 * NCB];
    __shared__ float sCol[WPC * D];
    __shared__ float sM[D], sDelta[D];
    __shared__ uint32_t sExt[D / 32];

    const int c = blockIdx.x, hk = blockIdx.y;
    const int64_t b = blockIdx.z, n = p.n, T = p.T, t0 = 64 * static_cast<int64_t>(c);
    const int nv = static_cast<int>(T - t0 < 64 ? T - t0 : 64);
    const int H_q = p.H_kv * p.n_rep;
    const int64_t kvs = static_cast<int64_t>(p.H_kv) * D, qs = static_cast<int64_t>(H_q) * D;
    const int tid = threadIdx.x, lane = tid & 63, col = lane & 15, g = lane >> 4;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave index, uniform
    // with one wave per column block every wave starts at row tile 0 (known at compile time)
    const int jb = w % NCB, i0 = WPC == 1 ? 0 : (w / NCB) * NTI;
    const int cc = 16 * jb + col;  // this lane's output column
    const float alpha = p.alpha;
    const size_t rec = size_t(D) * D + D;

    stage_f32<D, kBT>(sKh, FP, p.k + ((b * T + t0) * p.H_kv + hk) * D, kvs, nv);
    stage_bf16<D, 64, kBT>(sV, HP, p.v + ((b * T + t0) * p.H_kv + hk) * D, kvs, nv);
    __syncthreads();
    chunk_gate<D, GATE>(sKh, FP, sBeta, sA, nv);
    if (tid < D) {
        const float m = sBeta[31 * D + tid], dl = sBeta[63 * D + tid];
        sM[tid] = m;
        sDelta[tid] = dl;
        const bool ext = fmaxf(sBeta[tid] - m, m - dl) > kExtreme;
        const uint64_t bal = __ballot(ext);
        if (lane == 0) {  // wave w covers channels 64 w .. 64 w + 63
            sExt[2 * w] = static_cast<uint32_t>(bal);
            sExt[2 * w + 1] = static_cast<uint32_t>(bal >> 32);
        }
    }
    __syncthreads();
    uint32_t any_ext = 0;
#pragma unroll
    for (int j = 0; j < D / 32; ++j) any_ext |= sExt[j];
    for (int idx = tid; idx < 64 * D; idx += kBT) {
        const int t = idx / D, ch = idx % D;
        if (!((sExt[ch >> 5] >> (ch & 31)) & 1u)) sKh[t * FP + ch] *= fast_exp2(sM[ch] - sBeta[t * D + ch]);
    }
    const bool colx = (sExt[cc >> 5] >> (cc & 31)) & 1u;
    // extreme flags of the contraction channels g*KQ + ks of this lane group
    const uint32_t kbits = KQ == 32 ? sExt[g] : ((sExt[g >> 1] >> (16 * (g & 1))) & 0xffffu);

    // state entering the chunk (Y operands S0[cc][g*KQ + ks]; none for the first chunk)
    const float* S0row = c > 0 ? p.fwd + ((b * p.H_kv + hk) * (n - 1) + (c - 1)) * rec + size_t(cc) * D + g * KQ
                               : nullptr;
    __syncthreads();

    f32x4_t accK[NTI], accV[NTI], accDB[NTI];
#pragma unroll
    for (int u = 0; u < NTI; ++u) {
        accK[u] = zero4();
        accV[u] = zero4();
        accDB[u] = zero4();
    }

    for (int h = 0; h < p.n_rep; ++h) {
        const int hq = hk * p.n_rep + h;
        stage_f32<D, kBT>(sQ, FP, p.q + ((b * T + t0) * H_q + hq) * D, qs, nv);
        stage_bf16<D, 64, kBT>(sO, HP, p.dO + ((b * T + t0) * H_q + hq) * D, qs, nv);
        __syncthreads();
        // Q^ = phi(q) 2^(b-m) (extreme channels: phi(q))
        row_softmax<D, true>(sQ, FP, nv, sBeta, sM, sExt);
        // A^h = alpha dO V^T, zero above the diagonal
        {
            // tiles w and w + 8 of the 4 x 4 grid (row tile s-block, column tile t-block)
            const int is0 = w >> 2, it0 = w & 3, is1 = (w + 8) >> 2, it1 = w & 3;
            f32x4_t a0 = zero4(), a1 = zero4();
            const bool live0 = it0 <= is0, live1 = it1 <= is1;
#pragma unroll
            for (int k = 0; k < KS; ++k) {
                if (live0)
                    a0 = M::mma(M::load(sO + (16 * is0 + col) * HP + 8 * g + M::KSTEP * k),
                                M::load(sV + (16 * it0 + col) * HP + 8 * g + M::KSTEP * k), a0);
                if (live1)
                    a1 = M::mma(M::load(sO + (16 * is1 + col) * HP + 8 * g + M::KSTEP * k),
                                M::load(sV + (16 * it1 + col) * HP + 8 * g + M::KSTEP * k), a1);
            }
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int s0 = 16 * is0 + 4 * g + r, t0c = 16 * it0 + col;
                const int s1 = 16 * is1 + 4 * g + r, t1c = 16 * it1 + col;
                sA[s0 * AP + t0c] = t0c <= s0 ? alpha * a0[r] : 0.f;
                sA[s1 * AP + t1c] = t1c <= s1 ? alpha * a1[r] : 0.f;
            }
        }
        __syncthreads();

        // dphi(q^h): state term and intra-chunk term
        f32x4_t accS[NTI], accI[NTI];
#pragma unroll
        for (int u = 0; u < NTI; ++u) {
            accS[u] = zero4();
            accI[u] = zero4();
        }
        if (S0row) {
#pragma unroll 2
            for (int k8 = 0; k8 < KQ / 8; ++k8) {
                const float4 y0 = reinterpret_cast<const float4*>(S0row)[2 * k8];
                const float4 y1 = reinterpret_cast<const float4*>(S0row)[2 * k8 + 1];
                const float ys[8] = {y0.x, y0.y, y0.z, y0.w, y1.x, y1.y, y1.z, y1.w};
#pragma unroll
                for (int u = 0; u < NTI; ++u) {
                    float xf[8];
                    bf8_to_f32(*reinterpret_cast<const uint4*>(sO + (16 * (i0 + u) + col) * HP + g * KQ + 8 * k8), xf);
#pragma unroll
                    for (int j = 0; j < 8; ++j) accS[u] = mma4(xf[j], ys[j], accS[u]);
                }
            }
        }
#pragma unroll
        for (int tb = 0; tb < 4; ++tb)
#pragma unroll
            for (int kk = 0; kk < 4; ++kk) {
                const int tok = 16 * tb + 4 * g + kk;
                const float y = colx ? 0.f : sKh[tok * FP + cc];
#pragma unroll
                for (int u = 0; u < NTI; ++u)
                    if (tb <= i0 + u) accI[u] = mma4(sA[(16 * (i0 + u) + col) * AP + tok], y, accI[u]);
            }
        if (any_ext && colx) {
#pragma unroll
            for (int u = 0; u < NTI; ++u)
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int s = 16 * (i0 + u) + 4 * g + r;
                    const float bs = sBeta[s * D + cc];
                    float sum = 0.f;
                    for (int t = 0; t <= s; ++t)
                        sum += sA[s * AP + t] * sKh[t * FP + cc] * fast_exp2(bs - sBeta[t * D + cc]);
                    accI[u][r] = sum;
                }
        }
        float dpq[NTI][4], pq[NTI][4];
#pragma unroll
        for (int u = 0; u < NTI; ++u)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int s = 16 * (i0 + u) + 4 * g + r;
                const float bs = sBeta[s * D + cc], m = sM[cc];
                const float intra = colx ? accI[u][r] : accI[u][r] * fast_exp2(bs - m);
                dpq[u][r] = intra + alpha * accS[u][r] * fast_exp2(bs);
                const float qh = sQ[s * FP + cc];
                pq[u][r] = colx ? qh : qh * fast_exp2(m - bs);
                const float pd = pq[u][r] * dpq[u][r];
                accDB[u][r] += pd;
                const float rs = group16_sum(pd);
                if (col == 0) sRow[s * NCB + jb] = rs;
            }
        // dphi(k) intra-chunk term, summed over the heads
#pragma unroll
        for (int sb = 0; sb < 4; ++sb)
#pragma unroll
            for (int kk = 0; kk < 4; ++kk) {
                const int s = 16 * sb + 4 * g + kk;
                const float y = colx ? 0.f : sQ[s * FP + cc];
#pragma unroll
                for (int u = 0; u < NTI; ++u)
                    if (sb >= i0 + u) accK[u] = mma4(sA[s * AP + 16 * (i0 + u) + col], y, accK[u]);
            }
        if (any_ext && colx) {
#pragma unroll
            for (int u = 0; u < NTI; ++u)
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int t = 16 * (i0 + u) + 4 * g + r;
                    const float bt = sBeta[t * D + cc];
                    float sum = 0.f;
                    for (int s = t; s < 64; ++s)
                        sum += sA[s * AP + t] * sQ[s * FP + cc] * fast_exp2(sBeta[s * D + cc] - bt);
                    accK[u][r] += sum;
                }
        }
        __syncthreads();

        // alpha B^h[t][s] (s >= t), stored transposed over A^h; tiles w and w + 8 of
        // the 4 x 4 grid (row tile t-block, column tile s-block), computed together
        {
            const int it0 = w >> 2, is0 = w & 3, it1 = (w + 8) >> 2, is1 = w & 3;
            const bool live0 = is0 >= it0, live1 = is1 >= it1;
            f32x4_t a0 = zero4(), a1 = zero4();
#pragma unroll
            for (int k4 = 0; k4 < KQ / 4; ++k4) {
                const float4 y4 = *reinterpret_cast<const float4*>(sQ + (16 * is0 + col) * FP + g * KQ + 4 * k4);
                const float4 x40 = *reinterpret_cast<const float4*>(sKh + (16 * it0 + col) * FP + g * KQ + 4 * k4);
                const float4 x41 = *reinterpret_cast<const float4*>(sKh + (16 * it1 + col) * FP + g * KQ + 4 * k4);
                const float ys[4] = {y4.x, y4.y, y4.z, y4.w};
                const float xs0[4] = {x40.x, x40.y, x40.z, x40.w}, xs1[4] = {x41.x, x41.y, x41.z, x41.w};
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    const bool ext = (kbits >> (4 * k4 + j)) & 1u;
                    if (live0) a0 = mma4(ext ? 0.f : xs0[j], ys[j], a0);
                    if (live1) a1 = mma4(ext ? 0.f : xs1[j], ys[j], a1);
                }
            }
            if (any_ext) {
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int s = 16 * is0 + col;
#pragma unroll
                    for (int tl = 0; tl < 2; ++tl) {
                        const int t = 16 * (tl ? it1 : it0) + 4 * g + r;
                        if (s < t) continue;
                        float sum = 0.f;
                        for (int wd = 0; wd < D / 32; ++wd) {
                            uint32_t bits = sExt[wd];
                            while (bits) {
                                const int ch = 32 * wd + __builtin_ctz(bits);
                                bits &= bits - 1;
                                sum += sKh[t * FP + ch] * sQ[s * FP + ch] *
                                       fast_exp2(sBeta[s * D + ch] - sBeta[t * D + ch]);
                            }
                        }
                        if (tl) a1[r] += sum;
                        else a0[r] += sum;
                    }
                }
            }
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int s = 16 * is0 + col;
                const int t0r = 16 * it0 + 4 * g + r, t1r = 16 * it1 + 4 * g + r;
                sA[s * AP + t0r] = s >= t0r ? alpha * a0[r] : 0.f;
                sA[s * AP + t1r] = s >= t1r ? alpha * a1[r] : 0.f;
            }
        }
        // dq^h = phi(q) (.) (dphi(q) - <dphi(q), phi(q)>)
        {
            float* dq = p.dq + ((b * T + t0) * H_q + hq) * D + cc;
#pragma unroll
            for (int u = 0; u < NTI; ++u)
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int s = 16 * (i0 + u) + 4 * g + r;
                    float rs = 0.f;
#pragma unroll
                    for (int j = 0; j < NCB; ++j) rs += sRow[s * NCB + j];
                    if (s < nv) dq[s * qs] = pq[u][r] * (dpq[u][r] - rs);
                }
        }
        __syncthreads();
        // dv intra-chunk term: sum_s alpha B^h[t][s] dO_s
#pragma unroll
        for (int sb = 0; sb < 4; ++sb)
#pragma unroll
            for (int kk = 0; kk < 4; ++kk) {
                const int s = 16 * sb + 4 * g + kk;
                const float y = bf16_to_f32(sO[s * HP + cc]);
#pragma unroll
                for (int u = 0; u < NTI; ++u)
                    if (sb >= i0 + u) accV[u] = mma4(sA[s * AP + 16 * (i0 + u) + col], y, accV[u]);
            }
        __syncthreads();
    }

    // adjoint entering the chunk's last state (Y operands U[cc][g*KQ + ks]; none for the last chunk)
    const float* Urow = c < n - 1 ? p.adj + ((b * p.H_kv + hk) * (n - 1) + (n - 2 - c)) * rec + size_t(cc) * D + g * KQ
                                  : nullptr;
    // dphi(k) = intra + 2^(Delta-b) (.) (U v)
    float dpk[NTI][4], pk[NTI][4];
#pragma unroll
    for (int u = 0; u < NTI; ++u) {
        const int i = i0 + u;
        f32x4_t us = zero4();
        if (Urow) {
#pragma unroll 2
            for (int k8 = 0; k8 < KQ / 8; ++k8) {
                const float4 y0 = reinterpret_cast<const float4*>(Urow)[2 * k8];
                const float4 y1 = reinterpret_cast<const float4*>(Urow)[2 * k8 + 1];
                const float ys[8] = {y0.x, y0.y, y0.z, y0.w, y1.x, y1.y, y1.z, y1.w};
                float xf[8];
                bf8_to_f32(*reinterpret_cast<const uint4*>(sV + (16 * i + col) * HP + g * KQ + 8 * k8), xf);
#pragma unroll
                for (int j = 0; j < 8; ++j) us = mma4(xf[j], ys[j], us);
            }
        }
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int t = 16 * i + 4 * g + r;
            const float bt = sBeta[t * D + cc], m = sM[cc], dl = sDelta[cc];
            const float intra = colx ? accK[u][r] : accK[u][r] * fast_exp2(m - bt);
            dpk[u][r] = intra + us[r] * fast_exp2(dl - bt);
            const float kh = sKh[t * FP + cc];
            pk[u][r] = colx ? kh : kh * fast_exp2(bt - m);
            sQ[t * FP + cc] = pk[u][r] * fast_exp2(dl - bt);  // K~
            const float pd = pk[u][r] * dpk[u][r];
            accDB[u][r] -= pd;
            const float rs = group16_sum(pd);
            if (col == 0) sRow[t * NCB + jb] = rs;
        }
    }
    __syncthreads();
    // dv += K~ U: Y = U[g*KQ + ks][cc]
    {
        const bool has_u = c < n - 1;
        const float* Ub = p.adj + ((b * p.H_kv + hk) * (n - 1) + (has_u ? n - 2 - c : 0)) * rec + cc;
#pragma unroll
        for (int k4 = 0; k4 < KQ / 4; ++k4) {
            float ys[4];
#pragma unroll
            for (int j = 0; j < 4; ++j) ys[j] = has_u ? Ub[size_t(g * KQ + 4 * k4 + j) * D] : 0.f;
#pragma unroll
            for (int u = 0; u < NTI; ++u) {
                const float4 x4 = *reinterpret_cast<const float4*>(sQ + (16 * (i0 + u) + col) * FP + g * KQ + 4 * k4);
                accV[u] = mma4(x4.x, ys[0], accV[u]);
                accV[u] = mma4(x4.y, ys[1], accV[u]);
                accV[u] = mma4(x4.z, ys[2], accV[u]);
                accV[u] = mma4(x4.w, ys[3], accV[u]);
            }
        }
    }
    // outputs
    float* dk = p.dk + ((b * T + t0) * p.H_kv + hk) * D + cc;
    float* dv = p.dv + ((b * T + t0) * p.H_kv + hk) * D + cc;
    float* db = p.db + ((b * p.H_kv + hk) * T + t0) * D + cc;
    float csum = 0.f;
#pragma unroll
    for (int u = 0; u < NTI; ++u)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int t = 16 * (i0 + u) + 4 * g + r;
            float rs = 0.f;
#pragma unroll
            for (int j = 0; j < NCB; ++j) rs += sRow[t * NCB + j];
            if (t < nv) {
                dk[t * kvs] = pk[u][r] * (dpk[u][r] - rs);
                dv[t * kvs] = accV[u][r];
                db[t * D] = accDB[u][r];
                csum += accDB[u][r];
            }
        }
    csum = group4_sum(csum);
    if (g == 0) sCol[(w / NCB) * D + cc] = csum;
    __syncthreads();
    if (tid < D) {
        float s = 0.f;
#pragma unroll
        for (int j = 0; j < WPC; ++j) s += sCol[j * D + tid];
        p.tot[((b * p.H_kv + hk) * n + c) * D + tid] = s;
    }
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
        constexpr int PPR = D / 8;
        for (int idx = tid; idx < 128 * PPR; idx += kST) {
            const int r = idx / PPR, cpos = (idx % PPR) * 8;
            uint4 ku = make_uint4(0, 0, 0, 0), vu = make_uint4(0, 0, 0, 0);
            if (r >= lo && r < hi) {
                const int64_t off = ((b * T + first + r) * p.H_kv + hk) * D + cpos;
                ku = *reinterpret_cast<const uint4*>(p.k + off);
                vu = *reinterpret_cast<const uint4*>(p.v + off);
            }
            *reinterpret_cast<uint4*>(sK + r * HP + cpos) = ku;
            *reinterpret_cast<uint4*>(sV + r * HP + cpos) = vu;
        }
    }
    __syncthreads();
    const int w = p.window;
    const float sc = kLog2e * rsqrtf(static_cast<float>(D));
    const float beta = 1.0f - p.alpha;
    const int qq = 64 + 16 * wi + col;  // this lane's query in key-row coordinates
    const int64_t qtok = t0 + 16 * wi + col;
    const int kt0 = 2 * (wi >> 1);                   // first key tile of the aligned pairs
    const int ktlo = max(wi, (64 + 16 * wi - w + 1) >> 4);  // live key tiles: ktlo .. wi + 4
    const int64_t qrow = qtok < T ? qtok : T - 1;

    for (int h = 0; h < p.n_rep; ++h) {
        const int hq = hk * p.n_rep + h;
        const bf16_t* qr = p.q + (b * T + qrow) * qs + hq * D + 8 * g;
        const bf16_t* orow = p.dO + (b * T + qrow) * qs + hq * D + 8 * g;
        M::frag qf[KS], of[KS];
#pragma unroll
        for (int k = 0; k < KS; ++k) {
            qf[k] = M::load(qr + M::KSTEP * k);
            of[k] = M::load(orow + M::KSTEP * k);
        }
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
                float4* dst = reinterpret_cast<float4*>(p.dq + (b * T + qtok) * qs + hq * D + 16 * cb + 4 * g);
                float4 o = *dst;
                o.x += a[0] * rs;
                o.y += a[1] * rs;
                o.z += a[2] * rs;
                o.w += a[3] * rs;
                *dst = o;
            }
        }
    }
}

// ---------------------------------------------------------------- window: keys
// One workgroup per (chunk, key/value head, sequence); wave i holds key tile
// i of the chunk. The queries that can see those keys are in this chunk and
// the next, taken in aligned query-tile pairs (2G, 2G + 1); dk and dv are
// summed over the query heads of the group.
template <int D>
__global__ __launch_bounds__(kST) __attribute__((amdgpu_waves_per_eu(2))) void bwd_swa_k_kernel(BwdParams p) {
    typedef Mfma<bf16_t> M;
    constexpr int HP = D + 16, KS = D / M::KSTEP, NCB = D / 16;
    __shared__ __align__(16) bf16_t sQ[128 * HP];
    __shared__ __align__(16) bf16_t sO[128 * HP];
    __shared__ float sL[128], sDs[128];

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
    for (int h = 0; h < p.n_rep; ++h) {
        const int hq = hk * p.n_rep + h;
        __syncthreads();
        stage_bf16<D, 128, kST>(sQ, HP, p.q + ((b * T + t0) * H_q + hq) * D, qs, nq);
        stage_bf16<D, 128, kST>(sO, HP, p.dO + ((b * T + t0) * H_q + hq) * D, qs, nq);
        if (tid < 128) {
            const bool ok = tid < nq;
            const float* st = p.stats + ((b * T + t0 + (ok ? tid : 0)) * H_q + hq) * 2;
            sL[tid] = ok ? st[0] : 0.f;
            sDs[tid] = ok ? st[1] : 0.f;
        }
        __syncthreads();
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
    if (ktok < T) {
        const float rs = rsqrtf(static_cast<float>(D));
#pragma unroll
        for (int cb = 0; cb < NCB; ++cb) {
            float4* pk = reinterpret_cast<float4*>(p.dk + (b * T + ktok) * kvs + hk * D + 16 * cb + 4 * g);
            float4* pv = reinterpret_cast<float4*>(p.dv + (b * T + ktok) * kvs + hk * D + 16 * cb + 4 * g);
            float4 x = *pk, y = *pv;
            x.x += adk[cb][0] * rs;
            x.y += adk[cb][1] * rs;
            x.z += adk[cb][2] * rs;
            x.w += adk[cb][3] * rs;
            y.x += adv[cb][0];
            y.y += adv[cb][1];
            y.z += adv[cb][2];
            y.w += adv[cb][3];
            *pk = x;
            *pv = y;
        }
    }
}

// ---------------------------------------------------------------- gate chain
// d ln g_u = sum_{t >= u} dL/dB_t (later chunks through their sums), then
// dx = d ln g (1 - g) and the pool's transpose: dk += ..
template <int D, int GATE>
__global__ __launch_bounds__(kST) void bwd_gate_kernel(BwdParams p) {
    constexpr int FP = D + 4;
    __shared__ __align__(16) float sK[64 * FP];
    __shared__ __align__(16) float sS[64 * FP];
    __shared__ float sSuf[kST];

    const int c = blockIdx.x, hk = blockIdx.y;
    const int64_t b = blockIdx.z, n = p.n, T = p.T, t0 = 64 * static_cast<int64_t>(c);
    const int nv = static_cast<int>(T - t0 < 64 ? T - t0 : 64);
    const int64_t kvs = static_cast<int64_t>(p.H_kv) * D;
    const int tid = threadIdx.x;
    stage_f32<D, kST>(sK, FP, p.k + ((b * T + t0) * p.H_kv + hk) * D, kvs, nv);
    {
        const float* src = p.db + ((b * p.H_kv + hk) * T + t0) * D;
        for (int idx = tid; idx < 64 * D; idx += kST) {
            const int t = idx / D, ch = idx % D;
            sS[t * FP + ch] = t < nv ? src[t * D + ch] : 0.f;
        }
    }
    __syncthreads();
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
    __syncthreads();
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
    __syncthreads();
    // sS[t][c] becomes the dk contribution of row t, channel c
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
        __syncthreads();
        for (int i = part; i < D; i += 4) sS[row * FP + i] = ds;
    } else {
        for (int idx = tid; idx < 64 * D; idx += kST) {
            const int t = idx / D, ch = idx % D;
            const int lo = ch > 0 ? ch - 1 : 0, hi = ch + 3 < D ? ch + 3 : D;
            float s = 0.f;
            for (int j = lo; j < hi; ++j) s += sK[t * FP + j];
            const float x = s / static_cast<float>(hi - lo);
            sS[t * FP + ch] *= sigmoidf_stable(-x) / static_cast<float>(hi - lo);
        }
        __syncthreads();
        // pool transpose: channel c'' collects channels c'' - 2 .. c'' + 1
        for (int idx = tid; idx < 64 * D; idx += kST) {
            const int t = idx / D, ch = idx % D;
            float add = 0.f;
#pragma unroll
            for (int j = ch - 2; j <= ch + 1; ++j)
                if (j >= 0 && j < D) add += sS[t * FP + j];
            sK[t * FP + ch] = add;  // raw k no longer needed
        }
    }
    __syncthreads();
    const float* add = GATE == 0 ? sS : sK;
    float* dk = p.dk + ((b * T + t0) * p.H_kv + hk) * D;
    constexpr int PPR = D / 4;
    for (int idx = tid; idx < nv * PPR; idx += kST) {
        const int t = idx / PPR, c4 = (idx % PPR) * 4;
        float4* dst = reinterpret_cast<float4*>(dk + t * kvs + c4);
        const float4 a = *reinterpret_cast<const float4*>(add + t * FP + c4);
        float4 o = *dst;
        o.x += a.x;
        o.y += a.y;
        o.z += a.z;
        o.w += a.w;
        *dst = o;
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
        hipLaunchKernelGGL((bwd_swa_k_kernel<D>), grid, dim3(kST), 0, st, p);
        e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    hipLaunchKernelGGL((bwd_gate_kernel<D, GATE>), grid, dim3(kST), 0, st, p);
    return hipGetLastError();
}

}  // namespace

size_t backward_workspace_bytes(int64_t B, int64_t T, int H_kv, int H_q, int d) {
    if (T <= 0) return 0;
    const int64_t n = (T + 63) / 64;
    const size_t rec = size_t(d) * d + d;
    const size_t floats = 2 * size_t(B) * H_kv * size_t(n - 1) * rec + size_t(B) * H_kv * T * d +
                          size_t(B) * H_kv * n * d + size_t(B) * T * H_q * 2;
    return floats * sizeof(float);
}

hipError_t launch_backward(const BackwardArgs& a) {
    if (a.T == 0 || a.B == 0) return hipSuccess;
    if (a.d == 64) return a.gate ? launch_bwd_t<64, 1>(a) : launch_bwd_t<64, 0>(a);
    return a.gate ? launch_bwd_t<128, 1>(a) : launch_bwd_t<128, 0>(a);
}

}  // namespace liger
