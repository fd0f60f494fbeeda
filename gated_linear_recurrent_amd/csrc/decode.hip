// Liger Attention single-token decode step and ring set-up (gfx950).
//
// One workgroup per (sequence n, key/value head h). Per step it
//   - derives the gate g = sigmoid(pool(k)) and phi(k) = softmax(k) (the key
//     projection reused as a parameter-free gate; softmax feature map),
//   - reads the d x d float32 state once, applies S <- G (.) S + phi(k)^T v
//     (the gated recurrence of the unified framework) and writes it back,
//   - forms phi(q) S for the n_rep query heads that share this kv head,
//   - attends over the `window` most recent tokens held in the KV ring, the
//     new token included (sliding-window softmax, scale 1/sqrt(d)),
//   - mixes alpha * GRM + (1 - alpha) * SWA and stores o,
//   - writes the new key/value to ring slot pos mod window,
//   - and the last workgroup of the sequence to finish advances pos.
// The state row-major read-modify-write is the dominant HBM traffic
// (2 * d * d * 4 bytes per (n, h)); every float4 of S is touched once.
#include <type_traits>

#include "device_common.h"
#include "kernels.h"

namespace liger {

constexpr int kDecThreads = 256;
constexpr int kMaxSinks = 16;  // meta-memory tokens per key/value head

// 64-lane reductions: DPP inside rows of 16, then two cross-row exchanges.
__device__ __forceinline__ float dec_wave_max(float v) {
    v = fmaxf(v, dpp<kDppXor1>(v));
    v = fmaxf(v, dpp<kDppXor2>(v));
    v = fmaxf(v, dpp<kDppHalfMirror>(v));
    v = fmaxf(v, dpp<kDppMirror>(v));
    return xor32_max(xor16_max(v));
}
__device__ __forceinline__ float dec_wave_sum(float v) {
    v += dpp<kDppXor1>(v);
    v += dpp<kDppXor2>(v);
    v += dpp<kDppHalfMirror>(v);
    v += dpp<kDppMirror>(v);
    return xor32_sum(xor16_sum(v));
}

// Per 4-lane block of a wave (lanes 4b .. 4b+3), register i of lane 4b+j
// accumulates a[lane 4b+i] * b[lane 4b+j]: sixteen independent 4 x 4 outer
// products in one fp32 matrix instruction.
typedef float f32x4 __attribute__((ext_vector_type(4)));
__device__ __forceinline__ f32x4 outer4(float a, float b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_4x4x1f32(a, b, c, 0, 0, 0);
}

template <typename T, int D, int GATE, int NREP, bool SINK>
__global__ __launch_bounds__(kDecThreads, (NREP >= 8 || sizeof(T) == 4) ? 1 : 2) void decode_step_kernel(
    const T* __restrict__ q, const T* __restrict__ k, const T* __restrict__ v,
    float* __restrict__ S, T* __restrict__ ring_k, T* __restrict__ ring_v,
    int64_t* __restrict__ pos, uint32_t* __restrict__ sync, T* __restrict__ o,
    int H_kv, int window, float alpha, const T* __restrict__ sink_k, const T* __restrict__ sink_v, int n_sink) {
    constexpr int CG = D / 4;             // float4 column groups of a state row
    constexpr int RG = kDecThreads / CG;  // row groups
    constexpr int RPT = D / RG;           // state rows per thread
    constexpr int SPT = 64 / RG;          // ring slots per thread in the value pass
    constexpr int VPL = 16 / sizeof(T);   // elements per 16-byte load
    constexpr int LPR = D / VPL;          // lanes per key row in the logit pass (16-byte pieces)
    constexpr int SPI = kDecThreads / LPR;  // ring slots per key load instruction
    constexpr int KPT = 64 / SPI;         // key loads (slots) per thread in the logit pass
    constexpr int NR4 = (NREP + 3) / 4;   // float4 groups of the per-head values
    constexpr int NRP = 4 * NR4;          // per-head values padded to a float4 multiple
    static_assert(kDecThreads == 256 && LPR >= 8 && LPR <= 32, "key rows of 8 to 32 pieces");

    __shared__ float s_k[D], s_v[D], s_phik[D], s_g[D];
    __shared__ __align__(16) uint32_t s_kraw[D * sizeof(T) / 4];  // the new key, input bits
    __shared__ int64_t s_pos;
    __shared__ __align__(16) float s_q[D][NRP];      // raw q, head-minor
    __shared__ __align__(16) float s_phiq[D][NRP];   // phi(q), head-minor
    constexpr int NS = SINK ? kMaxSinks : 0;         // sink rows (meta-memory tokens)
    __shared__ __align__(16) float s_p[64 + NS][NRP];  // window weights (then sinks), head-minor
    __shared__ __align__(16) float s_red[RG][NREP][D];

    const int h = blockIdx.x;
    const int n = blockIdx.y;
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int H_q = H_kv * NREP;
    const int cg = tid % CG;
    const int rg = tid / CG;

    const size_t kv_off = (static_cast<size_t>(n) * H_kv + h) * D;
    const T* kp = k + kv_off;
    const T* vp = v + kv_off;
    const T* qp = q + (static_cast<size_t>(n) * H_q + static_cast<size_t>(h) * NREP) * D;
    float* Sp = S + (static_cast<size_t>(n) * H_kv + h) * D * D;
    const T* rk = ring_k + (static_cast<size_t>(n) * H_kv + h) * window * D;
    const T* rv = ring_v + (static_cast<size_t>(n) * H_kv + h) * window * D;

    // ---- loads (memory returns in issue order): the new token, the ring
    // keys and values, then the state rows last, so that the whole window
    // attention runs while the state is still arriving. None depends on pos.
    // raw element pairs, converted only after every load has been issued:
    // threads 0 .. D/2-1 read k, D/2 .. D-1 read v, all threads read q
    typedef typename std::conditional<sizeof(T) == 2, uint32_t, float2>::type Pair;
    constexpr int QPT = (NREP * D / 2 + kDecThreads - 1) / kDecThreads;
    Pair kvin;
    if (tid < D) kvin = *reinterpret_cast<const Pair*>((tid < D / 2 ? kp : vp) + 2 * (tid % (D / 2)));
    Pair qin[QPT];
#pragma unroll
    for (int i = 0; i < QPT; ++i) {
        const int pidx = tid + i * kDecThreads;
        if (pidx < NREP * D / 2) qin[i] = *reinterpret_cast<const Pair*>(qp + 2 * pidx);
    }
    // ring keys: consecutive lanes read consecutive 16-byte pieces; thread
    // tid holds piece kl of the rows of slots ks0 + i * SPI
    const int ks0 = tid / LPR;
    const int kl = tid % LPR;
    uint4 kr[KPT];
#pragma unroll
    for (int i = 0; i < KPT; ++i)
        kr[i] = ks0 + i * SPI < window ? *reinterpret_cast<const uint4*>(rk + ((ks0 + i * SPI) * D + kl * VPL))
                                       : make_uint4(0, 0, 0, 0);
    // ring values stay packed in registers until they are used
    typedef typename std::conditional<sizeof(T) == 2, uint2, float4>::type VRaw;
    VRaw vraw[SPT];
#pragma unroll
    for (int i = 0; i < SPT; ++i) {
        const int s = rg + i * RG;
        if (s < window) {
            vraw[i] = *reinterpret_cast<const VRaw*>(rv + (s * D + cg * 4));
        } else {
            if constexpr (sizeof(T) == 2) vraw[i] = make_uint2(0, 0);
            else vraw[i] = make_float4(0.f, 0.f, 0.f, 0.f);
        }
    }
    // sink tokens (rows past n_sink repeat the last one; their weight is 0)
    constexpr int SKI = SINK ? (kMaxSinks + SPI - 1) / SPI : 0;   // sink key loads per thread
    constexpr int SVI = SINK ? (kMaxSinks + RG - 1) / RG : 0;     // sink value loads per thread
    uint4 skr[SKI > 0 ? SKI : 1];
    VRaw svr[SVI > 0 ? SVI : 1];
    if constexpr (SINK) {
        const T* skp = sink_k + static_cast<size_t>(h) * n_sink * D;
        const T* svp = sink_v + static_cast<size_t>(h) * n_sink * D;
#pragma unroll
        for (int i = 0; i < SKI; ++i)
            skr[i] = *reinterpret_cast<const uint4*>(skp + (min(ks0 + i * SPI, n_sink - 1) * D + kl * VPL));
#pragma unroll
        for (int i = 0; i < SVI; ++i)
            svr[i] = *reinterpret_cast<const VRaw*>(svp + (min(rg + i * RG, n_sink - 1) * D + cg * 4));
    }
    float4 sv[RPT];
#pragma unroll
    for (int i = 0; i < RPT; ++i)
        sv[i] = *reinterpret_cast<const float4*>(Sp + ((rg + i * RG) * D + cg * 4));
    // every load is in flight before the first use waits on one
    __builtin_amdgcn_sched_barrier(0);

    // pos[n] is read by thread 0 alone and handed to the other waves through
    // LDS. Its arrival on sync[n] depends on the value read, so it is counted
    // only after that read; the last of the H_kv workgroups of sequence n to
    // arrive advances pos[n] at its end, when every workgroup has read it.
    uint32_t prev = 0;
    if (tid == 0) {
        const int64_t p0 = pos[n];
        s_pos = p0;
        prev = __hip_atomic_fetch_add(&sync[n], 1u + static_cast<uint32_t>(p0 >> 62), __ATOMIC_RELAXED,
                                      __HIP_MEMORY_SCOPE_AGENT);
    }

    auto unpair = [](const Pair& p2, float& lo, float& hi) {
        if constexpr (sizeof(T) == 2) {
            lo = __uint_as_float(p2 << 16);
            hi = __uint_as_float(p2 & 0xffff0000u);
        } else {
            lo = p2.x;
            hi = p2.y;
        }
    };
    if (tid < D / 2) s_kraw[tid * sizeof(T) / 2] = *reinterpret_cast<const uint32_t*>(&kvin);
    if constexpr (sizeof(T) == 4) {
        if (tid < D / 2) s_kraw[tid * 2 + 1] = *(reinterpret_cast<const uint32_t*>(&kvin) + 1);
    }
    if (tid < D) {
        float lo, hi;
        unpair(kvin, lo, hi);
        float* dst = tid < D / 2 ? s_k : s_v;
        const int c = 2 * (tid % (D / 2));
        dst[c] = lo;
        dst[c + 1] = hi;
    }
#pragma unroll
    for (int i = 0; i < QPT; ++i) {
        const int pidx = tid + i * kDecThreads;
        if (pidx < NREP * D / 2) {
            float lo, hi;
            unpair(qin[i], lo, hi);
            const int idx = 2 * pidx;  // element of the NREP x D query block; D is even
            s_q[idx % D][idx / D] = lo;
            s_q[(idx + 1) % D][idx / D] = hi;
        }
    }
    __syncthreads();
    const int64_t p = s_pos;
    const int slot = static_cast<int>(p % window);
    const int nvalid = static_cast<int>(p + 1 < window ? p + 1 : window);

    // ---- softmax over d of k (row 0) and of each query head (stored times
    // alpha, the GRM weight), one row per half wave; the gate on the last wave
    {
        constexpr int EPH = D / 32;  // elements per lane of a half-wave row
        const int hl = lane & 31;
        for (int row = 2 * wave + (lane >> 5); row <= NREP; row += kDecThreads / 32) {
            float x[EPH];
            float mx = -INFINITY;
#pragma unroll
            for (int e = 0; e < EPH; ++e) {
                const int c = hl + 32 * e;
                x[e] = row == 0 ? s_k[c] : s_q[c][row - 1];
                mx = fmaxf(mx, x[e]);
            }
            mx = group8_max(mx);
            mx = fmaxf(mx, dpp<kDppMirror>(mx));
            mx = xor16_max(mx);
            float se = 0.f;
#pragma unroll
            for (int e = 0; e < EPH; ++e) {
                x[e] = fast_exp2((x[e] - mx) * kLog2e);
                se += x[e];
            }
            se = group8_sum(se);
            se += dpp<kDppMirror>(se);
            se = xor16_sum(se);
            const float inv = fast_rcp(se) * (row == 0 ? 1.0f : alpha);
#pragma unroll
            for (int e = 0; e < EPH; ++e) {
                const int c = hl + 32 * e;
                if (row == 0) s_phik[c] = x[e] * inv;
                else s_phiq[c][row - 1] = x[e] * inv;
            }
        }
        if (wave == kDecThreads / 64 - 1) {
            constexpr int EPL = D / 64;
            if (GATE == 0) {
                float sm = 0.f;
#pragma unroll
                for (int e = 0; e < EPL; ++e) sm += s_k[lane + 64 * e];
                const float g = sigmoidf_stable(dec_wave_sum(sm) * (1.0f / D));
#pragma unroll
                for (int e = 0; e < EPL; ++e) s_g[lane + 64 * e] = g;
            } else {
#pragma unroll
                for (int e = 0; e < EPL; ++e) {
                    const int c = lane + 64 * e;
                    int n;
                    const float sm = pool4_taps<D>(s_k, c, n);
                    s_g[c] = sigmoidf_stable(sm * (c == 0 || c == D - 2 ? (1.0f / 3.0f) : c == D - 1 ? 0.5f : 0.25f));
                }
            }
        }
    }

    // ---- window logits q . k_s: this thread's piece of KPT slots, summed over
    // the LPR lanes of each row (the new token's key from LDS)
    {
        float qv[VPL][NRP];
#pragma unroll
        for (int t = 0; t < VPL; ++t)
#pragma unroll
            for (int j4 = 0; j4 < NR4; ++j4) {
                const float4 q4 = *reinterpret_cast<const float4*>(&s_q[kl * VPL + t][4 * j4]);
                qv[t][4 * j4 + 0] = q4.x;
                qv[t][4 * j4 + 1] = q4.y;
                qv[t][4 * j4 + 2] = q4.z;
                qv[t][4 * j4 + 3] = q4.w;
            }
        const uint4 knew = reinterpret_cast<const uint4*>(s_kraw)[kl];
        const float scale = kLog2e * rsqrtf(static_cast<float>(D));
        // logit of one key row (all LPR lanes of the row take part); row
        // `prow` of s_p, -inf where the key is not valid
        auto logit_row = [&](const uint4& kk, int prow, bool valid) {
            const T* e = reinterpret_cast<const T*>(&kk);
            float dot[NRP];
#pragma unroll
            for (int j = 0; j < NRP; ++j) dot[j] = 0.f;
#pragma unroll
            for (int t = 0; t < VPL; ++t) {
                const float kv = to_f32(e[t]);
#pragma unroll
                for (int j = 0; j < NREP; ++j) dot[j] += qv[t][j] * kv;
            }
#pragma unroll
            for (int j = 0; j < NREP; ++j) {
                dot[j] += dpp<kDppXor1>(dot[j]);
                dot[j] += dpp<kDppXor2>(dot[j]);
                dot[j] += dpp<kDppHalfMirror>(dot[j]);
                if constexpr (LPR >= 16) dot[j] += dpp<kDppMirror>(dot[j]);
                if constexpr (LPR >= 32) dot[j] = xor16_sum(dot[j]);
                dot[j] = valid ? dot[j] * scale : -INFINITY;
            }
            if (kl == 0) {
#pragma unroll
                for (int j4 = 0; j4 < NR4; ++j4)
                    *reinterpret_cast<float4*>(&s_p[prow][4 * j4]) =
                        make_float4(dot[4 * j4], dot[4 * j4 + 1], dot[4 * j4 + 2], dot[4 * j4 + 3]);
            }
        };
#pragma unroll
        for (int i = 0; i < KPT; ++i) {
            const int s_i = ks0 + i * SPI;
            logit_row(s_i == slot ? knew : kr[i], s_i, s_i < nvalid);
        }
        if constexpr (SINK) {
#pragma unroll
            for (int i = 0; i < SKI; ++i) {
                const int r = ks0 + i * SPI;
                if (r < kMaxSinks) logit_row(skr[i], 64 + r, r < n_sink);
            }
        }
    }
    __syncthreads();
    // window softmax per head, weights times (1 - alpha)
    for (int j = wave; j < NREP; j += kDecThreads / 64) {
        const float l = s_p[lane][j];
        // lane < kMaxSinks also takes sink `lane` (logit -inf past n_sink)
        const float ls = (SINK && lane < kMaxSinks) ? s_p[64 + (lane & (kMaxSinks - 1))][j] : -INFINITY;
        const float m = dec_wave_max(fmaxf(l, ls));
        const float e = lane < nvalid ? fast_exp2(l - m) : 0.f;
        const float es = fast_exp2(ls - m);  // exp2(-inf) = 0
        const float inv = fast_rcp(dec_wave_sum(e + es));
        s_p[lane][j] = e * inv * (1.0f - alpha);
        if (SINK && lane < kMaxSinks) s_p[64 + (lane & (kMaxSinks - 1))][j] = es * inv * (1.0f - alpha);
    }
    __syncthreads();

    // ---- sum_s p_s v_s (the new token's value from LDS). Both this and
    // phi(q) S below are head x column outer products summed over a slot or a
    // state row, on the matrix cores: in 4-lane block b (four consecutive
    // column groups of one row group) lane 4b+i brings the weight of head
    // 4 hg + i, lane 4b+j the value of its own column, so register i of acc[hg][e]
    // collects head 4 hg + i at this thread's column 4 cg + e.
    const int hq = tid & 3;
    f32x4 acc[NR4][4];
#pragma unroll
    for (int hg = 0; hg < NR4; ++hg)
#pragma unroll
        for (int e = 0; e < 4; ++e) acc[hg][e] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int i = 0; i < SPT; ++i) {
        const int s = rg + i * RG;
        float vr[4];
        if constexpr (sizeof(T) == 2) {
            vr[0] = __uint_as_float(vraw[i].x << 16);
            vr[1] = __uint_as_float(vraw[i].x & 0xffff0000u);
            vr[2] = __uint_as_float(vraw[i].y << 16);
            vr[3] = __uint_as_float(vraw[i].y & 0xffff0000u);
        } else {
            vr[0] = vraw[i].x;
            vr[1] = vraw[i].y;
            vr[2] = vraw[i].z;
            vr[3] = vraw[i].w;
        }
        if (s == slot) {
#pragma unroll
            for (int e = 0; e < 4; ++e) vr[e] = s_v[cg * 4 + e];
        }
#pragma unroll
        for (int hg = 0; hg < NR4; ++hg) {
            const float a = s_p[s][4 * hg + hq];  // 0 outside the window
#pragma unroll
            for (int e = 0; e < 4; ++e) acc[hg][e] = outer4(a, vr[e], acc[hg][e]);
        }
    }
    if constexpr (SINK) {
#pragma unroll
        for (int i = 0; i < SVI; ++i) {
            const int r = rg + i * RG;
            if (r >= kMaxSinks) continue;
            float vr[4];
            if constexpr (sizeof(T) == 2) {
                vr[0] = __uint_as_float(svr[i].x << 16);
                vr[1] = __uint_as_float(svr[i].x & 0xffff0000u);
                vr[2] = __uint_as_float(svr[i].y << 16);
                vr[3] = __uint_as_float(svr[i].y & 0xffff0000u);
            } else {
                vr[0] = svr[i].x;
                vr[1] = svr[i].y;
                vr[2] = svr[i].z;
                vr[3] = svr[i].w;
            }
#pragma unroll
            for (int hg = 0; hg < NR4; ++hg) {
                const float a = s_p[64 + r][4 * hg + hq];  // 0 past n_sink
#pragma unroll
                for (int e = 0; e < 4; ++e) acc[hg][e] = outer4(a, vr[e], acc[hg][e]);
            }
        }
    }

    // ---- state read-modify-write, row by row as the rows arrive, and
    // alpha phi(q) S_t
    const float4 v4 = *reinterpret_cast<const float4*>(s_v + cg * 4);
#pragma unroll
    for (int i = 0; i < RPT; ++i) {
        const int r = rg + i * RG;
        const float g = s_g[r];
        const float pk = s_phik[r];
        float4 st = sv[i];
        st.x = g * st.x + pk * v4.x;
        st.y = g * st.y + pk * v4.y;
        st.z = g * st.z + pk * v4.z;
        st.w = g * st.w + pk * v4.w;
        *reinterpret_cast<float4*>(Sp + (r * D + cg * 4)) = st;
#pragma unroll
        for (int hg = 0; hg < NR4; ++hg) {
            const float a = s_phiq[r][4 * hg + hq];
            acc[hg][0] = outer4(a, st.x, acc[hg][0]);
            acc[hg][1] = outer4(a, st.y, acc[hg][1]);
            acc[hg][2] = outer4(a, st.z, acc[hg][2]);
            acc[hg][3] = outer4(a, st.w, acc[hg][3]);
        }
    }
#pragma unroll
    for (int j = 0; j < NREP; ++j)
        *reinterpret_cast<float4*>(&s_red[rg][j][cg * 4]) =
            make_float4(acc[j / 4][0][j % 4], acc[j / 4][1][j % 4], acc[j / 4][2][j % 4], acc[j / 4][3][j % 4]);
    __syncthreads();
    T* op = o + (static_cast<size_t>(n) * H_q + static_cast<size_t>(h) * NREP) * D;
    for (int idx = 2 * tid; idx < NREP * D; idx += 2 * kDecThreads) {
        const int j = idx / D, c = idx % D;  // c is even: the pair stays in one head
        float s0 = 0.f, s1 = 0.f;
#pragma unroll
        for (int r = 0; r < RG; ++r) {
            const float2 x = *reinterpret_cast<const float2*>(&s_red[r][j][c]);
            s0 += x.x;
            s1 += x.y;
        }
        if constexpr (sizeof(T) == 2)
            *reinterpret_cast<uint32_t*>(op + idx) =
                static_cast<uint32_t>(from_f32<T>(s0)) | (static_cast<uint32_t>(from_f32<T>(s1)) << 16);
        else
            *reinterpret_cast<float2*>(op + idx) = make_float2(s0, s1);
    }

    // ---- ring slot <- (k, v), bit copy of the inputs
    T* rkw = ring_k + ((static_cast<size_t>(n) * H_kv + h) * window + slot) * D;
    T* rvw = ring_v + ((static_cast<size_t>(n) * H_kv + h) * window + slot) * D;
    if (tid < D) *reinterpret_cast<Pair*>((tid < D / 2 ? rkw : rvw) + 2 * (tid % (D / 2))) = kvin;

    // ---- the last of the H_kv workgroups of sequence n to arrive advances
    // pos[n] and clears the count. A count that was not zero on entry (a
    // counter never reset, or a step that did not complete) shows up as an
    // arrival numbered H_kv or more: that workgroup sets bit 31 of sync[n],
    // which then stays set (every later arrival sees it and none advances
    // pos[n]) until the caller resets the counter.
    if (tid == 0) {
        if (prev >= static_cast<uint32_t>(H_kv)) {
            __hip_atomic_fetch_or(&sync[n], 0x80000000u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        } else if (prev == static_cast<uint32_t>(H_kv - 1)) {
            __hip_atomic_fetch_and(&sync[n], 0x80000000u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            pos[n] = p + 1;
        }
    }
}

template <typename T, int D>
__global__ __launch_bounds__(64) void ring_fill_kernel(
    const T* __restrict__ k, const T* __restrict__ v, T* __restrict__ ring_k,
    T* __restrict__ ring_v, int64_t* __restrict__ pos, uint32_t* __restrict__ sync,
    int64_t Tlen, int H_kv, int window) {
    const int slot = blockIdx.x;
    const int h = blockIdx.y;
    const int64_t b = blockIdx.z;
    const int64_t t0 = Tlen > window ? Tlen - window : 0;
    const int64_t t = t0 + ((slot - t0 % window) % window + window) % window;
    const bool valid = t < Tlen;
    const size_t src = ((static_cast<size_t>(b) * Tlen + (valid ? t : 0)) * H_kv + h) * D;
    const size_t dst = ((static_cast<size_t>(b) * H_kv + h) * window + slot) * D;
    for (int i = threadIdx.x; i < D; i += 64) {
        ring_k[dst + i] = valid ? k[src + i] : T(0);
        ring_v[dst + i] = valid ? v[src + i] : T(0);
    }
    if (slot == 0 && h == 0 && threadIdx.x == 0) {
        pos[b] = Tlen;
        sync[b] = 0u;
    }
}

// Continuation: the ring after T more tokens. Slot s receives the new token at
// absolute position P = s (mod window) among the last `window` positions when
// P >= pos (a new token); otherwise it keeps the older token it holds.
template <typename T, int D>
__global__ __launch_bounds__(64) void ring_append_kernel(
    const T* __restrict__ k, const T* __restrict__ v, T* __restrict__ ring_k,
    T* __restrict__ ring_v, const int64_t* __restrict__ pos, int64_t Tlen, int H_kv, int window) {
    const int slot = blockIdx.x;
    const int h = blockIdx.y;
    const int64_t b = blockIdx.z;
    const int64_t pos0 = pos[b];
    const int64_t first = pos0 + Tlen - window;  // oldest position the ring keeps
    const int64_t P = first + (((slot - first) % window) + window) % window;
    if (P < pos0) return;
    const size_t src = ((static_cast<size_t>(b) * Tlen + (P - pos0)) * H_kv + h) * D;
    const size_t dst = ((static_cast<size_t>(b) * H_kv + h) * window + slot) * D;
    for (int i = threadIdx.x; i < D; i += 64) {
        ring_k[dst + i] = k[src + i];
        ring_v[dst + i] = v[src + i];
    }
}

// pos[b] += T and the arrival counters cleared, after the ring append has read pos.
__global__ void ring_advance_kernel(int64_t* __restrict__ pos, uint32_t* __restrict__ sync, int64_t B, int64_t Tlen) {
    const int64_t b = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
    if (b < B) {
        pos[b] += Tlen;
        sync[b] = 0u;
    }
}

// ------------------------------------------------------------------ launchers
template <typename T, int D, int GATE, int NREP>
static hipError_t launch_dec_t(const DecodeArgs& a) {
    dim3 grid(a.H_kv, static_cast<unsigned>(a.N));
    if (a.n_sink > 0)
        hipLaunchKernelGGL((decode_step_kernel<T, D, GATE, NREP, true>), grid, dim3(kDecThreads), 0,
                           static_cast<hipStream_t>(a.stream),
                           static_cast<const T*>(a.q), static_cast<const T*>(a.k), static_cast<const T*>(a.v),
                           a.S, static_cast<T*>(a.ring_k), static_cast<T*>(a.ring_v), a.pos, a.sync,
                           static_cast<T*>(a.o), a.H_kv, a.window, a.alpha, static_cast<const T*>(a.sink_k),
                           static_cast<const T*>(a.sink_v), a.n_sink);
    else
        hipLaunchKernelGGL((decode_step_kernel<T, D, GATE, NREP, false>), grid, dim3(kDecThreads), 0,
                           static_cast<hipStream_t>(a.stream),
                           static_cast<const T*>(a.q), static_cast<const T*>(a.k), static_cast<const T*>(a.v),
                           a.S, static_cast<T*>(a.ring_k), static_cast<T*>(a.ring_v), a.pos, a.sync,
                           static_cast<T*>(a.o), a.H_kv, a.window, a.alpha, nullptr, nullptr, 0);
    return hipGetLastError();
}

template <typename T, int D, int GATE>
static hipError_t launch_dec_rep(const DecodeArgs& a) {
    switch (a.n_rep) {
        case 1: return launch_dec_t<T, D, GATE, 1>(a);
        case 2: return launch_dec_t<T, D, GATE, 2>(a);
        case 4: return launch_dec_t<T, D, GATE, 4>(a);
        case 8: return launch_dec_t<T, D, GATE, 8>(a);
        default: return hipErrorInvalidValue;
    }
}

template <typename T>
static hipError_t launch_dec_dtype(const DecodeArgs& a) {
    if (a.d == 64) return a.gate ? launch_dec_rep<T, 64, 1>(a) : launch_dec_rep<T, 64, 0>(a);
    return a.gate ? launch_dec_rep<T, 128, 1>(a) : launch_dec_rep<T, 128, 0>(a);
}

hipError_t launch_decode_step(const DecodeArgs& a) {
    return a.bf16 ? launch_dec_dtype<bf16_t>(a) : launch_dec_dtype<float>(a);
}

template <typename T, int D>
static hipError_t launch_fill_t(const RingFillArgs& a) {
    dim3 grid(a.window, a.H_kv, static_cast<unsigned>(a.B));
    hipLaunchKernelGGL((ring_fill_kernel<T, D>), grid, dim3(64), 0, static_cast<hipStream_t>(a.stream),
                       static_cast<const T*>(a.k), static_cast<const T*>(a.v), static_cast<T*>(a.ring_k),
                       static_cast<T*>(a.ring_v), a.pos, a.sync, a.T, a.H_kv, a.window);
    return hipGetLastError();
}

template <typename T, int D>
static hipError_t launch_append_t(const RingFillArgs& a) {
    hipStream_t st = static_cast<hipStream_t>(a.stream);
    dim3 grid(a.window, a.H_kv, static_cast<unsigned>(a.B));
    hipLaunchKernelGGL((ring_append_kernel<T, D>), grid, dim3(64), 0, st, static_cast<const T*>(a.k),
                       static_cast<const T*>(a.v), static_cast<T*>(a.ring_k), static_cast<T*>(a.ring_v), a.pos, a.T,
                       a.H_kv, a.window);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(ring_advance_kernel, dim3(static_cast<unsigned>((a.B + 255) / 256)), dim3(256), 0, st, a.pos,
                       a.sync, a.B, a.T);
    return hipGetLastError();
}

hipError_t launch_ring_append(const RingFillArgs& a) {
    if (a.bf16) return a.d == 64 ? launch_append_t<bf16_t, 64>(a) : launch_append_t<bf16_t, 128>(a);
    return a.d == 64 ? launch_append_t<float, 64>(a) : launch_append_t<float, 128>(a);
}

hipError_t launch_ring_fill(const RingFillArgs& a) {
    if (a.bf16) return a.d == 64 ? launch_fill_t<bf16_t, 64>(a) : launch_fill_t<bf16_t, 128>(a);
    return a.d == 64 ? launch_fill_t<float, 64>(a) : launch_fill_t<float, 128>(a);
}

}  // namespace liger
