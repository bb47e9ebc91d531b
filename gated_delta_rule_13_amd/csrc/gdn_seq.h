// gdn_seq.h -- the kernel that completes a sequence-parallel run of the
// fused chunk kernel.
//
// The state recurrence is linear in the state ("Параллельность RNN?",
// section "Уровень 2": a linear recurrence is associative, so it can be
// evaluated by a parallel scan).  Over a segment of tokens that starts from
// state X, the end state and the outputs are affine in X:
//     end state  = X M + E0,      o_t = o0_t + X qm_t,
// where, with S of shape d_v x d_k (S_t = S_{t-1} A_t + eta_t v_t k_t^T,
// A_t = alpha_t (I - beta_t k_t k_t^T)):
//     M    = A_first ... A_last                     (d_k x d_k transition)
//     E0   = the segment's end state from a zero state
//     o0_t = the segment's outputs from a zero state
//     qm_t = (A_first ... A_t) q_t                  (the query carried through
//                                                    the transitions up to t)
// The fused kernel computes all of them at once for every segment (M and qm
// as the state and outputs of d_k extra rows that start from the identity
// with zero values).  Then, in one more launch,
//   combine: X_1 = end state of segment 0 (from the true S0),
//            X_{i+1} = X_i M_i + E0_i          (sequential over segments,
//                                               independent over state rows)
//   correct: o_t = o0_t + X_j qm_t              (every token of segment j >= 1)
// Each workgroup of that launch forms the X_j its tokens need from the
// segment end states itself (a short chain of small products), so no launch
// waits on another.
#pragma once

#include "gdn_device.h"

namespace gdn {

struct SeqParams {
    int BH, nseg, seg_len, T, dv;
    const float* seg_state;  // [BH][nseg][dv + dk][dk]: each segment's end state from zero
                             // (the first from S0), then its transition transposed,
                             // W[c][k] = M[k][c]
    const float* seg_q;    // [BH*T][dk] transformed queries (tokens of segments >= 1)
    const float* seg_o;    // [BH*T][dv] fp32 zero-state outputs, or null: they are in O
    void* O;               // [BH*T][dv], fp32 or bf16
    int o_bf16;
    float* S_final;        // [BH][dv][dk]
};

// Split-bf16 product of 16 x 32 by 32 x 16 fp32 slices: each operand as a
// bf16 hi + lo pair (about 16 significant bits), three MFMAs (hi hi, hi lo,
// lo hi) accumulated in fp32.  The A operand arrives split (it is shared by
// several products).
struct SplitA {
    bf16x8 hi, lo;
};
// The B operand is pinned where it is used (an empty asm that the compiler
// must treat as redefining it), so that its conversion, and with it the wait
// for its load, is not hoisted ahead of earlier work.
__device__ __forceinline__ f32x4 mfma_split(const SplitA& a, f32x4 b0, f32x4 b1, f32x4 acc) {
    asm volatile("" : "+v"(b0), "+v"(b1));
    bf16x8 bh, bl;
    split8(b0, b1, bh, bl);
    acc = mfma_bf16(a.hi, bh, acc);
    acc = mfma_bf16(a.hi, bl, acc);
    return mfma_bf16(a.lo, bh, acc);
}

// finish: one workgroup per (head, 16 value rows, segment j >= 1, group of
// G tokens of it), four waves.
//   chain:   X_1 = rows of segment 0's end state, then X_{i+1} = X_i M_i +
//            E0_i for i < j (and i = j for the workgroup that also writes
//            S_final: segment n_seg - 1, first group).  The rows stay in LDS;
//            16 x 16 output tile ct of a step is formed by wave ct % 4 with
//            split-bf16 MFMAs (16 x 16 x 32: lane (n, h) gives A[n][8h..+7]
//            and B[8h..+7][n] and receives D[4h + i][n]).  M_i is stored
//            transposed, W_i[c][k] = M_i[k][c], so that both operands are
//            read as rows.
//   correct: o_t += X_j qm_t for the group's tokens: the 16 x 16 tiles
//            O^T[rows][16 tokens] = X_j qm^T, TPW token tiles per wave.
// Every operand is loaded at the start (the chain's in blocks of PF steps),
// in one memory round trip, and the compiler is kept from sinking the loads
// towards their uses: the kernel is bound by memory latency, not work.
// Workgroup ids are grouped so that the row blocks of one (head, segment,
// group) share an XCD (ids congruent mod 8) and its L2 copy of qm.
template <int DK>
struct FinishShape {
    static constexpr int NC = DK / 16;                  // 16-column tiles of a row block
    static constexpr int NCW = (NC + 3) / 4;            // tiles per wave (at most)
    static constexpr int NKS = DK / 32;                 // 32-wide k-steps
    static constexpr int TPW = DK <= 128 ? 2 : 1;       // token tiles per wave
    static constexpr int G = 64 * TPW;                  // tokens per workgroup
    static constexpr int REGS = NCW * NKS * 8 + NCW * 4;   // chain operand floats per step and lane
    static constexpr int PF0 = 100 / REGS;
    static constexpr bool BLOCKED = PF0 >= 1;           // else (d_k 256) per-tile loads
    static constexpr int PF = PF0 < 1 ? 1 : PF0 > 8 ? 8 : PF0;   // steps loaded at once
};

// tokens per finishing workgroup, by d_k (host side)
inline int seq_group_tokens(int dk) { return 64 * (dk <= 128 ? 2 : 1); }

template <int DK>
__global__ __launch_bounds__(256) void gdn_seq_finish_kernel(SeqParams p) {
    using Sh = FinishShape<DK>;
    constexpr int NC = Sh::NC, NCW = Sh::NCW, NKS = Sh::NKS, PF = Sh::PF, TPW = Sh::TPW, G = Sh::G;
    // the rows' current end state in LDS, already split into its bf16 hi and
    // lo parts (the A operand of every product): split once where it is
    // produced, not by every reader
    constexpr int XP = DK + 8;   // row stride (bf16): the 16 rows' 16-byte reads spread over the banks
    __shared__ __bf16 Xh[16][XP], Xl[16][XP];
    const int dv = p.dv, nseg = p.nseg, L = p.seg_len, T = p.T;
    const int nrb = dv / 16;
    const int ngps = (L + G - 1) / G;
    const long per_head = (long)(nseg - 1) * ngps;
    const int xcd = blockIdx.x & 7, slot = blockIdx.x >> 3;
    const long unit = xcd + 8L * (slot / nrb);
    const int rb = slot % nrb;
    if (unit >= (long)p.BH * per_head) return;   // padding of the grid (before any barrier)
    const int bh = (int)(unit / per_head);
    const int rem = (int)(unit - (long)bh * per_head);
    const int j = 1 + rem / ngps, grp = rem % ngps;
    const int tb = j * L + grp * G;
    if (tb >= T) return;                         // a group past the end (whole workgroup)
    const int te = min(T, min((j + 1) * L, tb + G));
    const bool fin = j == nseg - 1 && grp == 0;  // also forms the final state
    const int nsteps = j - 1 + (fin ? 1 : 0);
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    const int n = lane & 15, h = lane >> 4;
    auto x_put = [&](int r, int c, float v) __attribute__((always_inline)) {
        __bf16 hi, lo;
        split_bf16(v, hi, lo);
        Xh[r][c] = hi;
        Xl[r][c] = lo;
    };
    auto x_get = [&](int ks) __attribute__((always_inline)) {
        SplitA a;
        a.hi = *reinterpret_cast<const bf16x8*>(&Xh[n][32 * ks + 8 * h]);
        a.lo = *reinterpret_cast<const bf16x8*>(&Xl[n][32 * ks + 8 * h]);
        return a;
    };
    const size_t slot_sz = (size_t)(dv + DK) * DK;
    const float* E = p.seg_state + (size_t)bh * nseg * slot_sz;

    // Every load is issued up front in the order of use, unconditionally (a
    // token past the end reads the last valid row; its output is not stored), so
    // that each use waits only for its own loads: X_1, then the chain's
    // operands, then the correction's.
    // X_1: rows 16 rb .. of segment 0's end state, in 16-byte pieces
    constexpr int XN = 16 * DK / 4, XV = (XN + 255) / 256;
    f32x4 xin[XV];
#pragma unroll
    for (int v = 0; v < XV; ++v) {
        const int e = min((int)threadIdx.x + 256 * v, XN - 1);
        const int r = e / (DK / 4), c = 4 * (e - r * (DK / 4));
        xin[v] = *reinterpret_cast<const f32x4*>(E + (size_t)(16 * rb + r) * DK + c);
    }
    // chain operands of steps i0 .. i0 + PF - 1: rows 16 ct + n of W_i
    // (k-slices 32 ks + 8 h ..) and E0_i in accumulator layout (rows 4 h + r,
    // column n); past the last step the last one's again (unused)
    f32x4 bw[Sh::BLOCKED ? PF : 1][NCW][NKS][2], e0[Sh::BLOCKED ? PF : 1][NCW];
    auto load_block = [&](int i0) __attribute__((always_inline)) {
        if constexpr (Sh::BLOCKED) {
#pragma unroll
            for (int s = 0; s < PF; ++s) {
                // (segment 1 exists whenever this kernel runs)
                const int i = max(1, min(i0 + s, nsteps));
                const float* Ei = E + (size_t)i * slot_sz;
                const float* W = Ei + (size_t)dv * DK;
#pragma unroll
                for (int cw = 0; cw < NCW; ++cw) {
                    const int ct = min(w + 4 * cw, NC - 1);
                    const float* wrow = W + (size_t)(16 * ct + n) * DK + 8 * h;
#pragma unroll
                    for (int ks = 0; ks < NKS; ++ks)
#pragma unroll
                        for (int q = 0; q < 2; ++q)
                            bw[s][cw][ks][q] = *reinterpret_cast<const f32x4*>(wrow + 32 * ks + 4 * q);
#pragma unroll
                    for (int r = 0; r < 4; ++r)
                        e0[s][cw][r] = Ei[(size_t)(16 * rb + 4 * h + r) * DK + 16 * ct + n];
                }
            }
        }
    };
    load_block(1);
    // correction operands: for token tile u of this wave, lane (n, h) holds
    // qm[t][32 ks + 8 h .. + 7] of token t = t0 + n, and its zero-state
    // outputs o0[t][16 rb + 4 h .. + 3]
    f32x4 qa[TPW][NKS][2], o0[TPW];
#pragma unroll
    for (int u = 0; u < TPW; ++u) {
        const int t = min(tb + 16 * (w + 4 * u) + n, te - 1);
        const float* qrow = p.seg_q + ((size_t)bh * T + t) * DK + 8 * h;
#pragma unroll
        for (int ks = 0; ks < NKS; ++ks)
#pragma unroll
            for (int q = 0; q < 2; ++q) qa[u][ks][q] = *reinterpret_cast<const f32x4*>(qrow + 32 * ks + 4 * q);
        const size_t off = ((size_t)bh * T + t) * dv + 16 * rb + 4 * h;
        const float* src = p.seg_o ? p.seg_o + off : reinterpret_cast<const float*>(p.O) + off;
        o0[u] = *reinterpret_cast<const f32x4*>(src);
    }
    __builtin_amdgcn_sched_barrier(0);   // every load above is issued before any use
#pragma unroll
    for (int v = 0; v < XV; ++v) {
        const int e = threadIdx.x + 256 * v;
        const int r = e / (DK / 4), c = 4 * (e - r * (DK / 4));
        if (e < XN) {
#pragma unroll
            for (int q = 0; q < 4; ++q) x_put(r, c + q, xin[v][q]);
        }
    }
    __syncthreads();

    // correction with X_j: O^T[16 rb + 4 h + r][t0 + n] += sum_k X_j[4 h + r][k] qm[t0 + n][k]
    auto correct = [&]() __attribute__((always_inline)) {
        SplitA xa[NKS];
#pragma unroll
        for (int ks = 0; ks < NKS; ++ks) xa[ks] = x_get(ks);
#pragma unroll
        for (int u = 0; u < TPW; ++u) {
            const int t = tb + 16 * (w + 4 * u) + n;
            f32x4 acc = o0[u];
#pragma unroll
            for (int ks = 0; ks < NKS; ++ks) acc = mfma_split(xa[ks], qa[u][ks][0], qa[u][ks][1], acc);
            // lane (n, h): token t, value columns 16 rb + 4 h .. + 3
            if (t < te) {
                const size_t off = ((size_t)bh * T + t) * dv + 16 * rb + 4 * h;
                if (p.o_bf16)
                    *reinterpret_cast<bf16x4*>(reinterpret_cast<__bf16*>(p.O) + off) =
                        __builtin_convertvector(acc, bf16x4);
                else
                    *reinterpret_cast<f32x4*>(reinterpret_cast<float*>(p.O) + off) = acc;
            }
        }
    };
    // one chain step: acc (per owned tile) from X_i in LDS, then X_{i+1} (or
    // the final state) written back
    auto finish_step = [&](int i, f32x4* acc) __attribute__((always_inline)) {
        __syncthreads();   // every wave is done reading X_i
        const bool to_final = fin && i == j;
#pragma unroll
        for (int cw = 0; cw < NCW; ++cw) {
            const int ct = w + 4 * cw;
            if (ct < NC) {
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    if (to_final)
                        p.S_final[((size_t)bh * dv + 16 * rb + 4 * h + r) * DK + 16 * ct + n] = acc[cw][r];
                    else
                        x_put(4 * h + r, 16 * ct + n, acc[cw][r]);
                }
            }
        }
        __syncthreads();   // X holds X_{i+1}
    };
    if constexpr (Sh::BLOCKED) {
        for (int i0 = 1; i0 <= nsteps; i0 += PF) {
            if (i0 > 1) {
                load_block(i0);
                __builtin_amdgcn_sched_barrier(0);
            }
#pragma unroll
            for (int s = 0; s < PF; ++s) {
                const int i = i0 + s;
                if (i > nsteps) break;   // uniform over the workgroup
                if (i == j) correct();   // (the final-state workgroup: X holds X_j)
                SplitA xa[NKS];
#pragma unroll
                for (int ks = 0; ks < NKS; ++ks) xa[ks] = x_get(ks);
                f32x4 acc[NCW];
#pragma unroll
                for (int cw = 0; cw < NCW; ++cw) {
                    acc[cw] = e0[s][cw];
#pragma unroll
                    for (int ks = 0; ks < NKS; ++ks)
                        acc[cw] = mfma_split(xa[ks], bw[s][cw][ks][0], bw[s][cw][ks][1], acc[cw]);
                }
                finish_step(i, acc);
            }
        }
    } else {
        // (one step's operands would not fit in registers: each tile's are
        // loaded just before its products)
        for (int i = 1; i <= nsteps; ++i) {
            if (i == j) correct();
            const float* Ei = E + (size_t)i * slot_sz;
            const float* W = Ei + (size_t)dv * DK;
            f32x4 acc[NCW];
#pragma unroll
            for (int cw = 0; cw < NCW; ++cw) {
                const int ct = min(w + 4 * cw, NC - 1);
                const float* wrow = W + (size_t)(16 * ct + n) * DK + 8 * h;
#pragma unroll
                for (int r = 0; r < 4; ++r) acc[cw][r] = Ei[(size_t)(16 * rb + 4 * h + r) * DK + 16 * ct + n];
#pragma unroll
                for (int ks = 0; ks < NKS; ++ks) {
                    const f32x4 b0 = *reinterpret_cast<const f32x4*>(wrow + 32 * ks);
                    const f32x4 b1 = *reinterpret_cast<const f32x4*>(wrow + 32 * ks + 4);
                    acc[cw] = mfma_split(x_get(ks), b0, b1, acc[cw]);
                }
            }
            finish_step(i, acc);
        }
    }
    if (!fin) correct();   // X holds X_j after steps 1 .. j - 1
}

}  // namespace gdn
