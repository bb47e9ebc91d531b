// gdn_recurrent.h -- token-by-token (recurrent) form of the gated delta rule
// on gfx950, for short sequences such as a decode step.
//
// Per token ("从零开始的 GDN 推导", recurrent form, transposed to the
// d_v x d_k state):
//     u   = S_{t-1} k_t
//     S_t = alpha_t (S_{t-1} - beta_t u k_t^T) + eta_t v_t k_t^T
//         = alpha_t S_{t-1} + (eta_t v_t - alpha_t beta_t u) k_t^T
//     o_t = S_t q_t
// with the write strength eta_t = beta_t unless it is given separately
// ("RNN的复兴03", section 1).
// Each row i of S evolves on its own (it needs only v_t[i] besides the shared
// k_t, q_t, alpha_t, beta_t, eta_t), so a group of LPR lanes owns one row: lane m
// keeps columns 4 m + 4 LPR j + e (j < J, e < 4) of that row in registers for
// all T tokens, and the two row dot products are reduced across the group.
// The state is read once and written once (in place when S_final == S0);
// with T = 1 the kernel streams the state through HBM, so its loads and
// stores carry the non-temporal hint (measured ≈8 % faster on a 64 MiB state).
#pragma once
#include "gdn_device.h"

namespace gdn {

struct RecParams {
    const void* q;
    const void* k;
    const void* v;
    const float* alpha;     // may be null (alpha = 1)
    const float* beta;
    const float* eta;       // may be null (eta = beta)
    const float* S0;        // may be null (zero state)
    void* O;
    float* S_final;
    int T, dv;
    int blocks_per_head;
    int o_bf16;
};

// Lanes per state row: 8 (4 when d_k = 16), so that a row's sum over its
// lanes is three DPP steps within a row of 16 lanes, and each lane streams
// d_k / 32 16-byte pieces of its row (many bytes in flight per wave).
constexpr int rec_lanes_per_row(int dk) { return dk % 32 == 0 ? 8 : 4; }

template <int CTRL>
__device__ __forceinline__ float dpp_f32(float v) {
    return __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v), CTRL, 0xf, 0xf, false));
}

// Sum over aligned groups of LPR (4 or 8) lanes, result in every lane:
// quad_perm [1,0,3,2] and [2,3,0,1] sum each quad of lanes, then
// row_half_mirror (lane i <-> 7 - i within 8 lanes) adds the other quad.
template <int LPR>
__device__ __forceinline__ float group_sum(float x) {
    x += dpp_f32<0xB1>(x);
    x += dpp_f32<0x4E>(x);
    if constexpr (LPR == 8) x += dpp_f32<0x141>(x);
    return x;
}

constexpr int kRecThreads = 128;

// Rows per lane group: each group keeps R rows (RPB / R apart), so k_t and
// q_t are loaded once per token for R rows and R times the state bytes are
// in flight per lane.
constexpr int kRecRows = 4;

template <int DK, bool BF>
__global__ __launch_bounds__(kRecThreads) void gdn_recurrent_kernel(RecParams p) {
    constexpr int LPR = rec_lanes_per_row(DK);
    constexpr int J = DK / (4 * LPR);
    constexpr int R = kRecRows;
    constexpr int RPW = 64 / LPR;                     // row groups per wave
    constexpr int GPB = (kRecThreads / 64) * RPW;     // row groups per workgroup
    static_assert(DK == 4 * LPR * J, "d_k must be a multiple of 4");

    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int m = lane % LPR;
    const long bh = blockIdx.x / p.blocks_per_head;
    const int row0 = (blockIdx.x % p.blocks_per_head) * GPB * R + wave * RPW + lane / LPR;
    const int T = p.T, dv = p.dv;

    // rows row0 + GPB * r, r < R; validity is uniform over a lane group
    f32x4 S[R][J];
#pragma unroll
    for (int r = 0; r < R; ++r) {
        const int row = row0 + GPB * r;
        const size_t srow = ((size_t)bh * dv + row) * DK;
#pragma unroll
        for (int j = 0; j < J; ++j)
            S[r][j] = (row < dv && p.S0)
                          ? __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(p.S0 + srow + 4 * m + 4 * LPR * j))
                          : zero4();
    }

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
        const float et = p.eta ? p.eta[tok] : b;
#pragma unroll
        for (int r = 0; r < R; ++r) {
            const int row = row0 + GPB * r;
            const bool valid = row < dv;
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
                for (int e = 0; e < 4; ++e) u = fmaf(S[r][j][e], kk[j][e], u);
            u = group_sum<LPR>(u);
            const float coef = et * vv - a * b * u;
            float ot = 0.f;
#pragma unroll
            for (int j = 0; j < J; ++j) {
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    S[r][j][e] = fmaf(coef, kk[j][e], a * S[r][j][e]);
                    ot = fmaf(S[r][j][e], qq[j][e], ot);
                }
            }
            ot = group_sum<LPR>(ot);
            if (valid && m == 0) {
                if (p.o_bf16) reinterpret_cast<__bf16*>(p.O)[tok * dv + row] = (__bf16)ot;
                else reinterpret_cast<float*>(p.O)[tok * dv + row] = ot;
            }
        }
    }
#pragma unroll
    for (int r = 0; r < R; ++r) {
        const int row = row0 + GPB * r;
        if (row < dv) {
            const size_t srow = ((size_t)bh * dv + row) * DK;
#pragma unroll
            for (int j = 0; j < J; ++j)
                __builtin_nontemporal_store(S[r][j], reinterpret_cast<f32x4*>(p.S_final + srow + 4 * m + 4 * LPR * j));
        }
    }
}

}  // namespace gdn
