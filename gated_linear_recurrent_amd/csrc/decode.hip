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
#include "device_common.h"
#include "kernels.h"

namespace liger {

constexpr int kDecThreads = 256;

template <typename T, int D, int GATE, int NREP>
__global__ __launch_bounds__(kDecThreads) void decode_step_kernel(
    const T* __restrict__ q, const T* __restrict__ k, const T* __restrict__ v,
    float* __restrict__ S, T* __restrict__ ring_k, T* __restrict__ ring_v,
    int64_t* __restrict__ pos, uint32_t* __restrict__ sync, T* __restrict__ o,
    int H_kv, int window, float alpha) {
    constexpr int CG = D / 4;             // float4 column groups of a state row
    constexpr int RG = kDecThreads / CG;  // row groups
    constexpr int RPT = D / RG;           // state rows per thread
    constexpr int SPT = 64 / RG;          // ring slots per thread (<= 64 slots)

    __shared__ float s_k[D], s_v[D], s_phik[D], s_g[D];
    __shared__ float s_q[NREP][D];
    __shared__ float s_phiq[NREP][D];
    __shared__ float s_p[NREP][64];
    __shared__ float s_red[RG][NREP][D];

    const int h = blockIdx.x;
    const int n = blockIdx.y;
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int H_q = H_kv * NREP;

    const int64_t p = pos[n];
    const int slot = static_cast<int>(p % window);
    const int nvalid = static_cast<int>(p + 1 < window ? p + 1 : window);

    const size_t kv_off = (static_cast<size_t>(n) * H_kv + h) * D;
    const T* kp = k + kv_off;
    const T* vp = v + kv_off;
    const T* qp = q + (static_cast<size_t>(n) * H_q + static_cast<size_t>(h) * NREP) * D;

    for (int i = tid; i < D; i += kDecThreads) {
        s_k[i] = to_f32(kp[i]);
        s_v[i] = to_f32(vp[i]);
    }
    for (int i = tid; i < NREP * D; i += kDecThreads) s_q[i / D][i % D] = to_f32(qp[i]);
    __syncthreads();

    // softmax over d of k (row 0) and of each query head (rows 1..NREP); gate.
    constexpr int EPL = D / 64;
    for (int row = wave; row <= NREP; row += kDecThreads / 64) {
        const float* src = row == 0 ? s_k : s_q[row - 1];
        float x[EPL];
        float mx = -INFINITY, sum_raw = 0.f;
#pragma unroll
        for (int e = 0; e < EPL; ++e) {
            x[e] = src[lane + 64 * e];
            mx = fmaxf(mx, x[e]);
            sum_raw += x[e];
        }
        mx = wave_max(mx);
        float se = 0.f;
#pragma unroll
        for (int e = 0; e < EPL; ++e) {
            x[e] = fast_exp2((x[e] - mx) * kLog2e);
            se += x[e];
        }
        const float inv = 1.0f / wave_sum(se);
        float* dst = row == 0 ? s_phik : s_phiq[row - 1];
#pragma unroll
        for (int e = 0; e < EPL; ++e) dst[lane + 64 * e] = x[e] * inv;
        if (row == 0) {
            if (GATE == 0) {
                const float g = sigmoidf_stable(wave_sum(sum_raw) * (1.0f / D));
#pragma unroll
                for (int e = 0; e < EPL; ++e) s_g[lane + 64 * e] = g;
            } else {
#pragma unroll
                for (int e = 0; e < EPL; ++e) {
                    const int c = lane + 64 * e;
                    const int lo = c > 0 ? c - 1 : 0;
                    const int hi = c + 3 < D ? c + 3 : D;
                    float s = 0.f;
                    for (int m = lo; m < hi; ++m) s += s_k[m];
                    s_g[c] = sigmoidf_stable(s / static_cast<float>(hi - lo));
                }
            }
        }
    }
    __syncthreads();

    // ---- state read-modify-write and GRM output phi(q) S_t
    const int cg = tid % CG;
    const int rg = tid / CG;
    float* Sp = S + (static_cast<size_t>(n) * H_kv + h) * D * D;
    float4 sv[RPT];
#pragma unroll
    for (int i = 0; i < RPT; ++i)
        sv[i] = *reinterpret_cast<const float4*>(Sp + static_cast<size_t>(rg + i * RG) * D + cg * 4);
    const float4 v4 = *reinterpret_cast<const float4*>(s_v + cg * 4);
    float acc[NREP][4];
#pragma unroll
    for (int j = 0; j < NREP; ++j) acc[j][0] = acc[j][1] = acc[j][2] = acc[j][3] = 0.f;
#pragma unroll
    for (int i = 0; i < RPT; ++i) {
        const int r = rg + i * RG;
        const float g = s_g[r];
        const float pk = s_phik[r];
        float4 s = sv[i];
        s.x = g * s.x + pk * v4.x;
        s.y = g * s.y + pk * v4.y;
        s.z = g * s.z + pk * v4.z;
        s.w = g * s.w + pk * v4.w;
        *reinterpret_cast<float4*>(Sp + static_cast<size_t>(r) * D + cg * 4) = s;
#pragma unroll
        for (int j = 0; j < NREP; ++j) {
            const float pq = s_phiq[j][r];
            acc[j][0] += pq * s.x;
            acc[j][1] += pq * s.y;
            acc[j][2] += pq * s.z;
            acc[j][3] += pq * s.w;
        }
    }

    // ---- sliding-window logits over the ring (current token from registers)
    const float scale = kLog2e * rsqrtf(static_cast<float>(D));
    const T* rk = ring_k + (static_cast<size_t>(n) * H_kv + h) * window * D;
    const T* rv = ring_v + (static_cast<size_t>(n) * H_kv + h) * window * D;
    {
        const int s = tid >> 2;       // ring slot
        const int part = tid & 3;     // quarter of the head dimension
        float dot[NREP];
#pragma unroll
        for (int j = 0; j < NREP; ++j) dot[j] = 0.f;
        if (s < nvalid) {
            const int c0 = part * (D / 4);
            if (s == slot) {
                for (int c = c0; c < c0 + D / 4; ++c) {
                    const float kv = s_k[c];
#pragma unroll
                    for (int j = 0; j < NREP; ++j) dot[j] += s_q[j][c] * kv;
                }
            } else {
                const T* kr = rk + static_cast<size_t>(s) * D;
                for (int c = c0; c < c0 + D / 4; ++c) {
                    const float kv = to_f32(kr[c]);
#pragma unroll
                    for (int j = 0; j < NREP; ++j) dot[j] += s_q[j][c] * kv;
                }
            }
        }
#pragma unroll
        for (int j = 0; j < NREP; ++j) {
            dot[j] += __shfl_xor(dot[j], 1, 64);
            dot[j] += __shfl_xor(dot[j], 2, 64);
        }
        if (part == 0) {
#pragma unroll
            for (int j = 0; j < NREP; ++j) s_p[j][s] = s < nvalid ? dot[j] * scale : -INFINITY;
        }
    }
    __syncthreads();
    for (int j = wave; j < NREP; j += kDecThreads / 64) {
        const float l = s_p[j][lane];
        const float m = wave_max(l);
        const float e = lane < nvalid ? fast_exp2(l - m) : 0.f;
        const float inv = 1.0f / wave_sum(e);
        s_p[j][lane] = e * inv * (1.0f - alpha);
    }
    __syncthreads();

    // ---- mix: alpha * GRM + sum_s p_s v_s
#pragma unroll
    for (int j = 0; j < NREP; ++j) {
        acc[j][0] *= alpha;
        acc[j][1] *= alpha;
        acc[j][2] *= alpha;
        acc[j][3] *= alpha;
    }
#pragma unroll
    for (int i = 0; i < SPT; ++i) {
        const int s = rg + i * RG;
        if (s < nvalid) {
            float vv[4];
            if (s == slot) {
#pragma unroll
                for (int e = 0; e < 4; ++e) vv[e] = s_v[cg * 4 + e];
            } else {
                const T* vr = rv + static_cast<size_t>(s) * D + cg * 4;
#pragma unroll
                for (int e = 0; e < 4; ++e) vv[e] = to_f32(vr[e]);
            }
#pragma unroll
            for (int j = 0; j < NREP; ++j) {
                const float pj = s_p[j][s];
#pragma unroll
                for (int e = 0; e < 4; ++e) acc[j][e] += pj * vv[e];
            }
        }
    }
#pragma unroll
    for (int j = 0; j < NREP; ++j)
        *reinterpret_cast<float4*>(&s_red[rg][j][cg * 4]) = make_float4(acc[j][0], acc[j][1], acc[j][2], acc[j][3]);
    __syncthreads();
    T* op = o + (static_cast<size_t>(n) * H_q + static_cast<size_t>(h) * NREP) * D;
    for (int idx = tid; idx < NREP * D; idx += kDecThreads) {
        const int j = idx / D, c = idx % D;
        float sum = 0.f;
#pragma unroll
        for (int r = 0; r < RG; ++r) sum += s_red[r][j][c];
        op[idx] = from_f32<T>(sum);
    }

    // ---- ring slot <- (k, v), bit copy of the inputs
    T* rkw = ring_k + ((static_cast<size_t>(n) * H_kv + h) * window + slot) * D;
    T* rvw = ring_v + ((static_cast<size_t>(n) * H_kv + h) * window + slot) * D;
    for (int i = tid; i < D; i += kDecThreads) {
        rkw[i] = kp[i];
        rvw[i] = vp[i];
    }

    // ---- the last of the H_kv workgroups of sequence n advances pos[n].
    // Every workgroup has read pos before it arrives, so the write is safe.
    __syncthreads();
    if (tid == 0) {
        __threadfence();
        const uint32_t prev = __hip_atomic_fetch_add(&sync[n], 1u, __ATOMIC_ACQ_REL, __HIP_MEMORY_SCOPE_AGENT);
        if (prev == static_cast<uint32_t>(H_kv - 1)) {
            sync[n] = 0u;
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

// ------------------------------------------------------------------ launchers
template <typename T, int D, int GATE, int NREP>
static hipError_t launch_dec_t(const DecodeArgs& a) {
    dim3 grid(a.H_kv, static_cast<unsigned>(a.N));
    hipLaunchKernelGGL((decode_step_kernel<T, D, GATE, NREP>), grid, dim3(kDecThreads), 0,
                       static_cast<hipStream_t>(a.stream),
                       static_cast<const T*>(a.q), static_cast<const T*>(a.k), static_cast<const T*>(a.v),
                       a.S, static_cast<T*>(a.ring_k), static_cast<T*>(a.ring_v), a.pos, a.sync,
                       static_cast<T*>(a.o), a.H_kv, a.window, a.alpha);
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

hipError_t launch_ring_fill(const RingFillArgs& a) {
    if (a.bf16) return a.d == 64 ? launch_fill_t<bf16_t, 64>(a) : launch_fill_t<bf16_t, 128>(a);
    return a.d == 64 ? launch_fill_t<float, 64>(a) : launch_fill_t<float, 128>(a);
}

}  // namespace liger
