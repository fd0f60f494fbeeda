// Full causal softmax attention for gfx950: the standard softmax attention
// layer that the inter-layer hybrid places between Liger blocks (paper-notes
// page "Liger: Linearizing Large Language Models to Gated Recurrent
// Structures", section "Liger 整体架构"):
//   o_i = sum_{j <= i} softmax_j(q_i . k_j / sqrt(d)) v_j ,
// query head h reading key/value head h / n_rep. bf16 in and out, fp32
// accumulation.
//
// One workgroup per (64-query block, group of up to four query heads that
// share a key/value head): two waves per head, 32 queries each, so every
// 64-key K/V tile staged in LDS serves all the heads of the group. Key
// blocks 0 .. the diagonal are walked with an online softmax (running row
// maximum in log2 units, running sum kept per lane and reduced once at the
// end). Scores are formed as S^T = K Q^T, so a lane holds four keys of one
// query and the probabilities pack straight into the key-indexed operand of
// O^T += V^T P (V^T read from the token-major tile with transposing loads).
// The key loop is software-pipelined: K runs one block ahead of V, so the
// next block's scores (MFMA) are issued beside this block's softmax (VALU).
// Query blocks are launched heaviest (last) first.
#include <type_traits>

#include "device_common.h"
#include "kernels.h"

namespace liger {

template <int D, int HPW>
__global__ __launch_bounds__(128 * HPW) void full_attn_kernel(FullAttnArgs p) {
    typedef Mfma<bf16_t> M;
    typedef M::frag Frag;
    constexpr int NW = 2 * HPW;         // waves
    constexpr int NTH = 64 * NW;        // threads
    constexpr int KS = D / M::KSTEP;    // k-steps over the head dimension
    constexpr int NT = D / 16;          // 16-wide output column tiles
    constexpr int DP = D + 8;           // pitch of the K tile (rows 4 banks apart)
    constexpr int VP = D + 16;          // pitch of the V tile (transposing reads)
    constexpr int PPR = D / 8;          // 16-byte pieces per row
    constexpr int NPC = 64 * PPR / NTH;  // pieces of each tile per thread
    static_assert(NPC * NTH == 64 * PPR, "tile pieces must divide over the threads");

    __shared__ __align__(16) bf16_t sK[2][64 * DP];
    __shared__ __align__(16) bf16_t sV[2][64 * VP];

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int col = lane & 15, g = lane >> 4;
    const int64_t T = p.T;
    const int nqb = static_cast<int>((T + 63) / 64);
    // Workgroup L runs on XCD L mod 8 (round-robin dispatch). When the
    // (sequence, head group) count is a multiple of 8, each group stays on one
    // XCD, so its K/V (T x d per tensor) is shared in that XCD's L2; query
    // blocks go heaviest (last) first.
    const int L = static_cast<int>(blockIdx.x);
    int grp, qi;
    if (p.ngroups % 8 == 0) {
        const int per = p.ngroups / 8, j = L / 8;
        grp = (L % 8) + 8 * (j % per);
        qi = j / per;
    } else {
        grp = L % p.ngroups;
        qi = L / p.ngroups;
    }
    const int qb = nqb - 1 - qi;
    const int hgrp = grp % (p.H_q / HPW);
    const int64_t b = grp / (p.H_q / HPW);
    const int hq = hgrp * HPW + wave / 2;
    const int hk = hgrp * HPW / p.n_rep;
    const int qoff = 32 * (wave & 1);   // this wave's queries within the block
    const bf16_t* q = static_cast<const bf16_t*>(p.q);
    const bf16_t* kg = static_cast<const bf16_t*>(p.k) + (b * T * p.H_kv + hk) * D;
    const bf16_t* vg = static_cast<const bf16_t*>(p.v) + (b * T * p.H_kv + hk) * D;
    const int64_t kv_stride = static_cast<int64_t>(p.H_kv) * D;

    // query fragments: query 64 qb + qoff + 16 s + col, channels 32 k + 8 g ..
    Frag qf[2][KS];
#pragma unroll
    for (int s = 0; s < 2; ++s) {
        const int64_t row = 64 * static_cast<int64_t>(qb) + qoff + 16 * s + col;
        const bf16_t* qr = q + ((b * T + (row < T ? row : 0)) * p.H_q + hq) * D + 8 * g;
#pragma unroll
        for (int k = 0; k < KS; ++k) qf[s][k] = row < T ? M::load(qr + M::KSTEP * k) : M::zero();
    }

    // K/V tiles staged through registers: K runs one key block ahead of V,
    // so the scores of block j + 1 are formed while block j's probabilities
    // are computed (independent MFMA and VALU work in one wave). During
    // iteration j the waves read K(j + 1) and V(j); at its end K(j + 2) and
    // V(j + 1) are stored into the buffers last read one iteration earlier.
    uint4 kr[NPC], vr[NPC];
    auto issue_k = [&](int kb) {
#pragma unroll
        for (int n = 0; n < NPC; ++n) {
            const int idx = tid + n * NTH;
            const int64_t row = 64 * static_cast<int64_t>(kb) + idx / PPR;
            kr[n] = row < T ? *reinterpret_cast<const uint4*>(kg + row * kv_stride + (idx % PPR) * 8)
                            : make_uint4(0, 0, 0, 0);
        }
    };
    auto issue_v = [&](int kb) {
#pragma unroll
        for (int n = 0; n < NPC; ++n) {
            const int idx = tid + n * NTH;
            const int64_t row = 64 * static_cast<int64_t>(kb) + idx / PPR;
            vr[n] = row < T ? *reinterpret_cast<const uint4*>(vg + row * kv_stride + (idx % PPR) * 8)
                            : make_uint4(0, 0, 0, 0);
        }
    };
    auto commit_k = [&](int buf) {
#pragma unroll
        for (int n = 0; n < NPC; ++n) {
            const int idx = tid + n * NTH;
            *reinterpret_cast<uint4*>(&sK[buf][(idx / PPR) * DP + (idx % PPR) * 8]) = kr[n];
        }
    };
    auto commit_v = [&](int buf) {
#pragma unroll
        for (int n = 0; n < NPC; ++n) {
            const int idx = tid + n * NTH;
            *reinterpret_cast<uint4*>(&sV[buf][(idx / PPR) * VP + (idx % PPR) * 8]) = vr[n];
        }
    };

    f32x4_t acc[2][NT];
#pragma unroll
    for (int s = 0; s < 2; ++s)
#pragma unroll
        for (int t = 0; t < NT; ++t) acc[s][t] = zero4();
    float m[2] = {-INFINITY, -INFINITY};  // running maximum, log2 units
    float l[2] = {0.f, 0.f};              // running sum of this lane's keys
    const float c = kLog2e * rsqrtf(static_cast<float>(D));

    // ---- S^T = K Q^T on the K tile in buffer kbuf: lane (col, g) holds keys
    // 16 kt + 4 g + r of query col; on the diagonal block a key tile past a
    // query tile is skipped whole
    auto scores = [&](int kbuf, auto diag_c, f32x4_t (&sc)[2][4]) {
        constexpr bool diag = decltype(diag_c)::value;
#pragma unroll
        for (int kt = 0; kt < 4; ++kt) {
            sc[0][kt] = zero4();
            sc[1][kt] = zero4();
            const bool live0 = !diag || kt <= 2 * (wave & 1);
            const bool live1 = !diag || kt <= 2 * (wave & 1) + 1;
            if (!live1) continue;
            const bf16_t* krow = &sK[kbuf][(16 * kt + col) * DP + 8 * g];
#pragma unroll
            for (int k = 0; k < KS; ++k) {
                const Frag a = M::load(krow + M::KSTEP * k);
                if (live0) sc[0][kt] = M::mma(a, qf[0][k], sc[0][kt]);
                sc[1][kt] = M::mma(a, qf[1][k], sc[1][kt]);
            }
        }
    };
    // ---- online softmax of one block's scores -> packed probabilities
    auto softmax = [&](f32x4_t (&sc)[2][4], auto diag_c, Frag (&pf)[2][2]) {
        constexpr bool diag = decltype(diag_c)::value;
#pragma unroll
        for (int s = 0; s < 2; ++s) {
            float mx = -INFINITY;
#pragma unroll
            for (int kt = 0; kt < 4; ++kt)
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    float x = sc[s][kt][r];
                    if (diag && 16 * kt + 4 * g + r > qoff + 16 * s + col) x = -INFINITY;
                    sc[s][kt][r] = x;
                    mx = fmaxf(mx, x);
                }
            // Every query keeps at least one key (itself) on the diagonal
            // block. The running maximum moves only when the block's exceeds
            // it by more than 8 (log2 units): probabilities up to 2^8 are
            // exact enough in fp32 sums and bf16 operands, and the O rescale
            // is skipped whenever no query of the wave moved.
            const float mblk = group4_max(mx) * c;
            const bool grow = mblk > m[s] + 8.0f;
            const float mnew = grow ? mblk : m[s];
            const float alpha = fast_exp2(m[s] - mnew);
            m[s] = mnew;
            float ls = 0.f;
            float pv[4][4];
#pragma unroll
            for (int kt = 0; kt < 4; ++kt)
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const float e = fast_exp2(fmaf(sc[s][kt][r], c, -mnew));  // exp2(-inf) = 0 when masked
                    pv[kt][r] = e;
                    ls += e;
                }
            l[s] = fmaf(l[s], alpha, ls);
            if (__any(grow)) {
#pragma unroll
                for (int t = 0; t < NT; ++t) acc[s][t] *= alpha;
            }
#pragma unroll
            for (int G = 0; G < 2; ++G) {
                const float v8[8] = {pv[2 * G][0], pv[2 * G][1], pv[2 * G][2], pv[2 * G][3],
                                     pv[2 * G + 1][0], pv[2 * G + 1][1], pv[2 * G + 1][2], pv[2 * G + 1][3]};
                pf[s][G] = M::pack(v8);
            }
        }
    };
    // ---- O^T += V^T P over the two 32-key groups of the V tile in buffer vbuf
    auto values = [&](int vbuf, const Frag (&pf)[2][2]) {
#pragma unroll
        for (int t = 0; t < NT; ++t)
#pragma unroll
            for (int G = 0; G < 2; ++G) {
                const Frag a = load_key_frag(sV[vbuf], VP, 32 * G, 16 * t, lane);
                acc[0][t] = M::mma(a, pf[0][G], acc[0][t]);
                acc[1][t] = M::mma(a, pf[1][G], acc[1][t]);
            }
    };

    // prologue: K(0), V(0) and K(1) in LDS, the scores of block 0
    issue_k(0);
    issue_v(0);
    commit_k(0);
    if (qb >= 1) issue_k(1);
    commit_v(0);
    if (qb >= 1) commit_k(1);
    __syncthreads();
    f32x4_t sc[2][4];
    if (qb == 0) scores(0, std::true_type{}, sc);
    else scores(0, std::false_type{}, sc);
    // iteration 0 stores K(2) over K(0): every wave has read K(0) first
    if (qb >= 1) __syncthreads();
    // iteration j: K(j + 2) and V(j + 1) in flight, probabilities of block j,
    // scores of block j + 1, values of block j, then the two stores
    auto step = [&](int j, auto next_c) {
        constexpr int NEXT = decltype(next_c)::value;  // 2: full next block, 1: diagonal next block
        const bool issue_next_k = NEXT == 2 && j + 2 <= qb;
        if (issue_next_k) issue_k(j + 2);
        issue_v(j + 1);
        Frag pf[2][2];
        softmax(sc, std::false_type{}, pf);
        f32x4_t scn[2][4];
        if constexpr (NEXT == 2) scores((j + 1) & 1, std::false_type{}, scn);
        else scores((j + 1) & 1, std::true_type{}, scn);
        values(j & 1, pf);
        if (issue_next_k) commit_k(j & 1);
        commit_v((j + 1) & 1);
        __syncthreads();
#pragma unroll
        for (int s = 0; s < 2; ++s)
#pragma unroll
            for (int kt = 0; kt < 4; ++kt) sc[s][kt] = scn[s][kt];
    };
    for (int j = 0; j + 1 < qb; ++j) step(j, std::integral_constant<int, 2>{});
    if (qb >= 1) step(qb - 1, std::integral_constant<int, 1>{});
    {
        Frag pf[2][2];
        softmax(sc, std::true_type{}, pf);
        values(qb & 1, pf);
    }

    // ---- normalise and store: lane (col, g) holds channels 16 t + 4 g + r of query col
    bf16_t* o = static_cast<bf16_t*>(p.o);
#pragma unroll
    for (int s = 0; s < 2; ++s) {
        const int64_t row = 64 * static_cast<int64_t>(qb) + qoff + 16 * s + col;
        const float inv = fast_rcp(group4_sum(l[s]));
        if (row >= T) continue;
        bf16_t* orow = o + ((b * T + row) * p.H_q + hq) * D + 4 * g;
#pragma unroll
        for (int t = 0; t < NT; ++t)
            *reinterpret_cast<uint2*>(orow + 16 * t) =
                make_uint2(pack_bf16x2(acc[s][t][0] * inv, acc[s][t][1] * inv),
                           pack_bf16x2(acc[s][t][2] * inv, acc[s][t][3] * inv));
    }
}

template <int D, int HPW>
static hipError_t launch_full_t(const FullAttnArgs& a) {
    FullAttnArgs p = a;
    p.ngroups = static_cast<int>(a.B * (a.H_q / HPW));
    const int64_t nwg = ((a.T + 63) / 64) * p.ngroups;
    if (nwg > 2147483647LL) return hipErrorInvalidValue;
    hipLaunchKernelGGL((full_attn_kernel<D, HPW>), dim3(static_cast<unsigned>(nwg)), dim3(128 * HPW), 0,
                       static_cast<hipStream_t>(a.stream), p);
    return hipGetLastError();
}

template <int D>
static hipError_t launch_full_d(const FullAttnArgs& a) {
    switch (a.n_rep) {
        case 1: return launch_full_t<D, 1>(a);
        case 2: return launch_full_t<D, 2>(a);
        case 4:
        case 8: return launch_full_t<D, 4>(a);
        default: return hipErrorInvalidValue;
    }
}

hipError_t launch_full_attn(const FullAttnArgs& a) {
    if (a.T == 0) return hipSuccess;
    return a.d == 64 ? launch_full_d<64>(a) : launch_full_d<128>(a);
}

}  // namespace liger
