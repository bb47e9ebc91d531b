// gdn_recurrent.h -- token-by-token (recurrent) form of the gated delta rule
// on gfx950, for short sequences such as a decode step.
//
// Per token ("从零开始的 GDN 推导", recurrent form, transposed to the
// d_v x d_k state; "RNN的复兴03", section 1, with write strength = beta):
//     u   = S_{t-1} k_t
//     S_t = alpha_t (S_{t-1} - beta_t u k_t^T) + beta_t v_t k_t^T
//         = alpha_t S_{t-1} + beta_t (v_t - alpha_t u) k_t^T
//     o_t = S_t q_t
// Each row i of S evolves on its own (it needs only v_t[i] besides the shared
// k_t, q_t, alpha_t, beta_t), so a group of LPR lanes owns one row: lane m
// keeps columns 4 m + 4 LPR j + e (j < J, e < 4) of that row in registers for
// all T tokens, and the two row dot products are reduced across the group.
// The state is read once and written once (in place when S_final == S0);
// with T = 1 the kernel streams the state through HBM.
#pragma once
#include "gdn_device.h"

namespace gdn {

struct RecParams {
    const void* q;
    const void* k;
    const void* v;
    const float* alpha;     // may be null (alpha = 1)
    const float* beta;
    const float* S0;        // may be null (zero state)
    void* O;
    float* S_final;
    int T, dv;
    int blocks_per_head;
    int o_bf16;
};

// Lanes per state row: the largest power of two <= 32 with d_k = 4 * LPR * J.
constexpr int rec_lanes_per_row(int dk) {
    int l = 32;
    while (l > 1 && dk % (4 * l) != 0) l /= 2;
    return l;
}

constexpr int kRecThreads = 256;

template <int DK, bool BF>
__global__ __launch_bounds__(kRecThreads) void gdn_recurrent_kernel(RecParams p) {
    constexpr int LPR = rec_lanes_per_row(DK);
    constexpr int J = DK / (4 * LPR);
    constexpr int RPW = 64 / LPR;                     // rows per wave
    constexpr int RPB = (kRecThreads / 64) * RPW;     // rows per workgroup
    static_assert(DK == 4 * LPR * J, "d_k must be a multiple of 4");

    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int m = lane % LPR;
    const long bh = blockIdx.x / p.blocks_per_head;
    const int row = (blockIdx.x % p.blocks_per_head) * RPB + wave * RPW + lane / LPR;
    const bool valid = row < p.dv;   // uniform over a row's lane group
    const int T = p.T, dv = p.dv;

    f32x4 S[J];
    const size_t srow = ((size_t)bh * dv + row) * DK;
#pragma unroll
    for (int j = 0; j < J; ++j)
        S[j] = (valid && p.S0) ? *reinterpret_cast<const f32x4*>(p.S0 + srow + 4 * m + 4 * LPR * j)
                               : zero4();

    for (int t = 0; t < T; ++t) {
        const size_t tok = (size_t)bh * T + t;
        f32x4 kk[J], qq[J];
#pragma unroll
        for (int j = 0; j < J; ++j) {
            const size_t off = tok * DK + 4 * m + 4 * LPR * j;
            if constexpr (BF) {
                kk[j] = __builtin_convertvector(
                    *reinterpret_cast<const bf16x4*>(reinterpret_cast<const __bf16*>(p.k) + off), f32x4);
                qq[j] = __builtin_convertvector(
                    *reinterpret_cast<const bf16x4*>(reinterpret_cast<const __bf16*>(p.q) + off), f32x4);
            } else {
                kk[j] = *reinterpret_cast<const f32x4*>(reinterpret_cast<const float*>(p.k) + off);
                qq[j] = *reinterpret_cast<const f32x4*>(reinterpret_cast<const float*>(p.q) + off);
            }
        }
        const float a = p.alpha ? p.alpha[tok] : 1.f;
        const float b = p.beta[tok];
        float vv = 0.f;
        if (valid) {
            vv = BF ? (float)reinterpret_cast<const __bf16*>(p.v)[tok * dv + row]
                    : reinterpret_cast<const float*>(p.v)[tok * dv + row];
        }
        // u = S_{t-1} k_t over the row
        float u = 0.f;
#pragma unroll
        for (int j = 0; j < J; ++j)
#pragma unroll
            for (int e = 0; e < 4; ++e) u = fmaf(S[j][e], kk[j][e], u);
#pragma unroll
        for (int o = LPR / 2; o > 0; o >>= 1) u += __shfl_xor(u, o, 64);
        const float coef = b * (vv - a * u);
        float ot = 0.f;
#pragma unroll
        for (int j = 0; j < J; ++j) {
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                S[j][e] = fmaf(coef, kk[j][e], a * S[j][e]);
                ot = fmaf(S[j][e], qq[j][e], ot);
            }
        }
#pragma unroll
        for (int o = LPR / 2; o > 0; o >>= 1) ot += __shfl_xor(ot, o, 64);
        if (valid && m == 0) {
            if (p.o_bf16) reinterpret_cast<__bf16*>(p.O)[tok * dv + row] = (__bf16)ot;
            else reinterpret_cast<float*>(p.O)[tok * dv + row] = ot;
        }
    }
    if (valid) {
#pragma unroll
        for (int j = 0; j < J; ++j)
            *reinterpret_cast<f32x4*>(p.S_final + srow + 4 * m + 4 * LPR * j) = S[j];
    }
}

}  // namespace gdn
