// gdn_kernels.h -- gfx950 kernels of the chunkwise-parallel gated delta rule.
//
// Orientation: state S is d_v x d_k, o_t = S_t q_t (inclusive), as on
// "RNN的复兴03:现代RNN的并行计算" (section 4) and the circuit-complexity page.
// "从零开始的 GDN 推导" writes the transpose; its chunk formulas, transposed,
// are (chunk input state S, chunk-local positions r = 0..C-1):
//   g_r     = sum_{j<=r} log alpha_j         gamma_{r+1} = exp(g_r)
//   A_ri    = -beta_r exp(g_r - g_i) k_r.k_i  (i < r)   T = (I - A)^{-1}
//   W = T diag(beta) diag(exp g) K,  U = T diag(beta) V          (WY / UT)
//   V'      = U - W S^T                                  (pseudo-values)
//   O       = diag(exp g) Q S^T + (Q K^T o D) V',  D_ri = exp(g_r - g_i), i <= r
//   S_next  = exp(g_last) S + V'^T diag(exp(g_last - g)) K
// The fused kernel evaluates V' re-associated as
//   V' = T diag(beta) (V - diag(exp g) (K S^T))
// which is the same product (W S^T = T diag(beta) diag(exp g) K S^T) without
// forming W: it saves 2 C d_k flops per token and keeps K exact in bf16.
//
// Precision plan (bf16 inputs): q, k, v are exact bf16 MFMA operands; every
// derived operand (S, T diag(beta), the pseudo-value input, V', the decayed
// V', the masked scores) is split into bf16 hi + lo and multiplied with
// 2 or 3 MFMAs, so each product carries about 16 significant bits and fp32
// accumulation.  fp32 inputs use fp32 MFMA throughout.
#pragma once
#include <type_traits>

#include "gdn_device.h"

namespace gdn {

// Prep waves per workgroup of the fp16-operand fused kernel (gdn_fast.h):
// six beside one or two scan waves, five beside three, and beside four six
// at chunks of up to 32 tokens with d_k up to 128 (ten waves, whose
// registers still fit three waves on a SIMD), else four (eight waves in
// all, two per SIMD).
constexpr int fast_prep_waves(int ns, int C, int dk) {
    return ns == 3 ? 5 : (ns == 4 && (C > 32 || dk > 128)) ? 4 : 6;
}

struct FwdParams {
    const void* q;
    const void* k;
    const void* v;
    const float* alpha;   // may be null: alpha = 1
    const float* beta;
    const float* S0;      // may be null: zero state
    void* O;
    float* S_final;
    float* T_out;         // prep kernel outputs (each may be null)
    float* W_out;
    float* U_out;
    int B, H, T, dv;
    int n_tiles;          // value-column tiles per head
    int o_bf16;           // O stored as bf16 (else fp32)
    int xcd_groups;       // pipelined kernel: place a head's tiles on one XCD
                          // (the grid then covers B * H rounded up to a multiple of 8)
    int o_wt;             // fp32 output written through (else non-temporal only)
    const float* eta;     // write strength; may be null: eta = beta
    float* dbg_T;         // fast kernel, stage output: T per chunk [B,H,NT,C,C] (may be null)
    float* dbg_V;         // fast kernel, stage output: pseudo-values V' [B,H,T,d_v] (may be null)
    // Sequence-parallel launch of the fast kernel (nseg > 1).  Each sequence
    // is cut into nseg segments of seg_len tokens (a multiple of the chunk
    // size), all run at once.  The first segment starts from S0 and its
    // outputs are final; every later one starts from a zero state, and its
    // tiles from n_tiles_v on carry the d_k rows of the segment's transition
    // (identity state, zero values), whose outputs are the segment's queries
    // carried through its transitions.
    int nseg;             // segments per sequence (1: the whole sequence)
    int seg_len;          // tokens per segment
    int n_tiles_v;        // value-column tiles (tiles past them: transition rows)
    float* seg_state;     // [B*H][nseg][d_v + d_k][d_k]: each segment's end state (the first
                          // from S0, the others from zero), then its transition M
                          // transposed (d_k x d_k, element (r, k) of M at k * d_k + r)
    float* seg_q;         // [B*H*T][d_k]: transformed queries of the later segments
    float* seg_o;         // [B*H*T][d_v]: fp32 outputs of the later segments from a zero
                          // state when O is bf16 (null: they are written to O)
};

// LDS layout of one workgroup.  Rows are padded by 16 bytes.
template <int C, int DK, int NW, bool BF>
struct alignas(16) Lds {
    using In = typename std::conditional<BF, __bf16, float>::type;
    static constexpr int DVT = 16 * NW;
    static constexpr int PAD = 16 / (int)sizeof(In);
    In K[C][DK + PAD];              // keys, row-major
    In Kt[BF ? DK : 1][C + PAD];    // keys transposed (bf16 operand loads)
    In Q[C][DK + PAD];
    In V[C][DVT + PAD];             // value columns of this tile
    float A[C][C + 1];              // strictly lower A
    float Tm[C][C + 1];             // T = (I - A)^{-1}
    float M[16][C + 1];             // block-row scratch of the solve
    In Tt[C][C + PAD];              // T diag(beta)       (bf16: hi part)
    In Ttl[BF ? C : 1][C + PAD];    //                    (bf16: lo part)
    In P[C][C + PAD];               // masked, decayed scores (hi)
    In Pl[BF ? C : 1][C + PAD];     //                         (lo)
    float g2[C];                    // chunk-local inclusive cumsum of log2(alpha)
    float eg[C];                    // exp(g_r)
    float dec[C];                   // exp(g_last - g_r)
    float beta[C];
    float eta[C];                   // write strength (= beta unless given)
    float glast;                    // exp(g_last)
};

// Register staging of one chunk's inputs (prefetched a chunk ahead).
template <int C, int DK, int NW, bool BF>
struct Stage {
    using In = typename std::conditional<BF, __bf16, float>::type;
    static constexpr int NTHR = NW * 64;
    static constexpr int EPV = 16 / (int)sizeof(In);      // elements per 16-byte vector
    static constexpr int DVT = 16 * NW;
    static constexpr int KVEC = C * DK / EPV;
    static constexpr int VVEC = C * DVT / EPV;
    static constexpr int NKV = (KVEC + NTHR - 1) / NTHR;
    static constexpr int NVV = (VVEC + NTHR - 1) / NTHR;
    uint4 k[NKV], q[NKV], v[NVV];
    float a, b, e;
};

template <int C, int DK, int NW, bool BF>
struct ChunkCtx {
    using In = typename std::conditional<BF, __bf16, float>::type;
    const In* kb;      // this sequence's k [T, DK]
    const In* qb;
    const In* vb;      // this sequence's v [T, dv]
    const float* ab;   // alpha [T] or null
    const float* bb;   // beta [T]
    const float* eb;   // eta [T] or null (eta = beta)
    int T, dv, col0;   // col0: first value column of this tile
};

template <int C, int DK, int NW, bool BF>
__device__ __forceinline__ void load_chunk(Stage<C, DK, NW, BF>& st,
                                           const ChunkCtx<C, DK, NW, BF>& cx,
                                           int t0, int Lc, int tid, bool want_q) {
    using S = Stage<C, DK, NW, BF>;
    const uint4 z = make_uint4(0, 0, 0, 0);
#pragma unroll
    for (int i = 0; i < S::NKV; ++i) {
        const int vi = tid + i * S::NTHR;
        st.k[i] = z;
        st.q[i] = z;
        if (vi < S::KVEC) {
            const int r = vi / (DK / S::EPV);
            const int c = vi % (DK / S::EPV);
            if (r < Lc) {
                const size_t off = (size_t)(t0 + r) * DK + (size_t)c * S::EPV;
                st.k[i] = *reinterpret_cast<const uint4*>(cx.kb + off);
                if (want_q) st.q[i] = *reinterpret_cast<const uint4*>(cx.qb + off);
            }
        }
    }
#pragma unroll
    for (int i = 0; i < S::NVV; ++i) {
        const int vi = tid + i * S::NTHR;
        st.v[i] = z;
        if (vi < S::VVEC) {
            const int r = vi / (S::DVT / S::EPV);
            const int c = vi % (S::DVT / S::EPV);
            if (r < Lc)
                st.v[i] = *reinterpret_cast<const uint4*>(
                    cx.vb + (size_t)(t0 + r) * cx.dv + cx.col0 + (size_t)c * S::EPV);
        }
    }
    // padding tokens: alpha = 1, beta = eta = 0 (identity transition)
    st.a = 1.f;
    st.b = 0.f;
    st.e = 0.f;
    if (tid < Lc) {
        st.a = cx.ab ? cx.ab[t0 + tid] : 1.f;
        st.b = cx.bb[t0 + tid];
        st.e = cx.eb ? cx.eb[t0 + tid] : st.b;
    }
}

// Registers -> LDS, and the chunk-local decay prefix (wave 0).
template <int C, int DK, int NW, bool BF>
__device__ __forceinline__ void store_chunk(const Stage<C, DK, NW, BF>& st,
                                            Lds<C, DK, NW, BF>& s, int tid, int lane) {
    using S = Stage<C, DK, NW, BF>;
    using In = typename S::In;
#pragma unroll
    for (int i = 0; i < S::NKV; ++i) {
        const int vi = tid + i * S::NTHR;
        if (vi < S::KVEC) {
            const int r = vi / (DK / S::EPV);
            const int c = (vi % (DK / S::EPV)) * S::EPV;
            *reinterpret_cast<uint4*>(&s.K[r][c]) = st.k[i];
            *reinterpret_cast<uint4*>(&s.Q[r][c]) = st.q[i];
            if constexpr (BF) {
                const In* e = reinterpret_cast<const In*>(&st.k[i]);
#pragma unroll
                for (int x = 0; x < S::EPV; ++x) s.Kt[c + x][r] = e[x];
            }
        }
    }
#pragma unroll
    for (int i = 0; i < S::NVV; ++i) {
        const int vi = tid + i * S::NTHR;
        if (vi < S::VVEC) {
            const int r = vi / (S::DVT / S::EPV);
            const int c = (vi % (S::DVT / S::EPV)) * S::EPV;
            *reinterpret_cast<uint4*>(&s.V[r][c]) = st.v[i];
        }
    }
    if (tid < 64) {
        // g_r = sum_{j<=r} log alpha_j, kept in base 2; lanes >= C carry alpha = 1.
        const float l2 = (tid < C) ? __log2f(st.a) : 0.f;
        const float g = wave_inclusive_scan(l2, lane);
        const float gl = __shfl(g, C - 1, 64);
        if (tid < C) {
            s.g2[tid] = g;
            s.eg[tid] = exp2f(g);
            s.dec[tid] = exp2f(gl - g);
            s.beta[tid] = st.b;
            s.eta[tid] = st.e;
        }
        if (tid == 0) s.glast = exp2f(gl);
    }
}

// Decay-masked Gram matrix A and masked scores P of the chunk, on MFMA.
//   A_ri = -beta_r exp(g_r - g_i) k_r.k_i   (i < r)
//   P_ri =          exp(g_r - g_i) q_r.k_i  (i <= r)
template <int C, int DK, int NW, bool BF>
__device__ __forceinline__ void gram_phase(Lds<C, DK, NW, BF>& s, int wave, int n, int h,
                                           bool want_p) {
    constexpr int NT = C / 16;
    constexpr int NPAIR = NT * (NT + 1) / 2;
    const int njobs = want_p ? 2 * NPAIR : NPAIR;
    for (int job = wave; job < njobs; job += NW) {
        const bool isP = job >= NPAIR;
        int ct = isP ? job - NPAIR : job;
        int rt = 0;
        while (ct > rt) { ct -= rt + 1; ++rt; }
        const auto* arow = isP ? &s.Q[16 * rt + n][0] : &s.K[16 * rt + n][0];
        const auto* brow = &s.K[16 * ct + n][0];
        f32x4 acc = zero4();
        if constexpr (BF) {
#pragma unroll
            for (int ss = 0; ss < DK / 32; ++ss)
                acc = mfma_bf16(ld_nat8(arow, ss, h), ld_nat8(brow, ss, h), acc);
        } else {
#pragma unroll
            for (int kk = 0; kk < DK / 4; ++kk)
                acc = mfma_f32(arow[4 * kk + h], brow[4 * kk + h], acc);
        }
        const int i = 16 * ct + n;
        const float g2i = s.g2[i];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int r = 16 * rt + 4 * h + j;
            const float d = exp2f(s.g2[r] - g2i);
            if (!isP) {
                s.A[r][i] = (i < r) ? -s.beta[r] * d * acc[j] : 0.f;
            } else {
                const float pv = (i <= r) ? d * acc[j] : 0.f;
                if constexpr (BF) {
                    __bf16 hi, lo;
                    split_bf16(pv, hi, lo);
                    s.P[r][i] = hi;
                    s.Pl[r][i] = lo;
                } else {
                    s.P[r][i] = pv;
                }
            }
        }
    }
}

// T = (I - A)^{-1} by forward substitution ("RNN的复兴03", section 2.3.1:
// T[i,j] = sum_{k=j}^{i-1} A[i,k] T[k,j]), blocked by 16:
//   diagonal 16 x 16 blocks: one lane per column, sequential over rows;
//   block row R:  T_{R,c} = T_RR (sum_{m<R} A_{R,m} T_{m,c})  for c < R,
// which is the same recurrence grouped by blocks.  All on VALU, fp32.
// Then T diag(beta) (FOLD_BETA) or T is written (bf16: as hi + lo).
template <bool FOLD_BETA, int C, int DK, int NW, bool BF>
__device__ __forceinline__ void solve_phase(Lds<C, DK, NW, BF>& s, int tid, int wave, int lane) {
    constexpr int NT = C / 16;
    constexpr int NTHR = NW * 64;
    if (wave == 0 && lane < 16 * NT) {
        const int b = lane >> 4, j = lane & 15;
        float t[16];
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            float acc = (i == j) ? 1.f : 0.f;
            const float* arow = &s.A[16 * b + i][16 * b];
#pragma unroll
            for (int k = 0; k < i; ++k) acc = fmaf(arow[k], t[k], acc);
            t[i] = acc;
        }
#pragma unroll
        for (int i = 0; i < 16; ++i) s.Tm[16 * b + i][16 * b + j] = t[i];
    }
#pragma unroll
    for (int R = 1; R < NT; ++R) {
        __syncthreads();
        const int ncol = 16 * R;
        for (int idx = tid; idx < 16 * ncol; idx += NTHR) {
            const int i = idx / ncol, c = idx % ncol;
            const float* arow = &s.A[16 * R + i][0];
            float acc = 0.f;
            for (int m = c & ~15; m < ncol; ++m) acc = fmaf(arow[m], s.Tm[m][c], acc);
            s.M[i][c] = acc;
        }
        __syncthreads();
        for (int idx = tid; idx < 16 * ncol; idx += NTHR) {
            const int i = idx / ncol, c = idx % ncol;
            const float* trow = &s.Tm[16 * R + i][16 * R];
            float acc = s.M[i][c];
            for (int m = 0; m < i; ++m) acc = fmaf(trow[m], s.M[m][c], acc);
            s.Tm[16 * R + i][c] = acc;
        }
    }
    __syncthreads();
    for (int idx = tid; idx < C * C; idx += NTHR) {
        const int r = idx / C, i = idx % C;
        if ((i >> 4) <= (r >> 4)) {
            const float x = FOLD_BETA ? s.Tm[r][i] * s.beta[i] : s.Tm[r][i];
            if constexpr (BF) {
                __bf16 hi, lo;
                split_bf16(x, hi, lo);
                s.Tt[r][i] = hi;
                s.Ttl[r][i] = lo;
            } else {
                s.Tt[r][i] = x;
            }
        }
    }
}

template <int C, int DK, int NW, bool BF>
__device__ __forceinline__ void zero_upper(Lds<C, DK, NW, BF>& s, int tid) {
    using In = typename Lds<C, DK, NW, BF>::In;
    constexpr int NTHR = NW * 64;
    for (int idx = tid; idx < C * C; idx += NTHR) {
        const int r = idx / C, i = idx % C;
        s.Tt[r][i] = (In)0.f;
        s.P[r][i] = (In)0.f;
        if constexpr (BF) {
            s.Ttl[r][i] = (In)0.f;
            s.Pl[r][i] = (In)0.f;
        }
    }
}

// ---------------------------------------------------------------------------
// Fused forward kernel.  One workgroup per (b, h, value-column tile of 16*NW
// columns); wave w owns 16 value columns and that slice of the state
// (S^T[d_k, 16] as MFMA accumulators).  Chunks are processed in order; the
// next chunk's inputs are prefetched into registers during the current one.
// ---------------------------------------------------------------------------
template <int C, int DK, int NW, bool BF>
__global__ __launch_bounds__(NW * 64) void gdn_fwd_kernel(FwdParams p) {
    using L = Lds<C, DK, NW, BF>;
    using St = Stage<C, DK, NW, BF>;
    using In = typename L::In;
    constexpr int NT = C / 16;
    constexpr int NK = DK / 16;
    static_assert(sizeof(L) <= 160 * 1024, "LDS budget");
    __shared__ L s;

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int n = lane & 15;
    const int h = lane >> 4;

    const int tile = blockIdx.x % p.n_tiles;
    const int bh = blockIdx.x / p.n_tiles;
    const int T = p.T, dv = p.dv;
    const int col_tile = tile * L::DVT;
    const int col = col_tile + 16 * wave + n;   // this lane's value column

    ChunkCtx<C, DK, NW, BF> cx;
    cx.kb = reinterpret_cast<const In*>(p.k) + (size_t)bh * T * DK;
    cx.qb = reinterpret_cast<const In*>(p.q) + (size_t)bh * T * DK;
    cx.vb = reinterpret_cast<const In*>(p.v) + (size_t)bh * T * dv;
    cx.ab = p.alpha ? p.alpha + (size_t)bh * T : nullptr;
    cx.bb = p.beta + (size_t)bh * T;
    cx.eb = p.eta ? p.eta + (size_t)bh * T : nullptr;
    cx.T = T;
    cx.dv = dv;
    cx.col0 = col_tile;

    // State slice: Sacc[t][j] = S[col][16 t + 4 h + j]
    f32x4 Sacc[NK];
    const size_t sbase = (size_t)bh * dv * DK + (size_t)col * DK;
#pragma unroll
    for (int t = 0; t < NK; ++t)
#pragma unroll
        for (int j = 0; j < 4; ++j)
            Sacc[t][j] = p.S0 ? p.S0[sbase + 16 * t + 4 * h + j] : 0.f;

    zero_upper(s, tid);

    const int nchunks = (T + C - 1) / C;
    St st;
    load_chunk(st, cx, 0, min(C, T), tid, true);

    for (int c = 0; c < nchunks; ++c) {
        const int t0 = c * C;
        const int Lc = min(C, T - t0);
        __syncthreads();                       // previous chunk done with LDS
        store_chunk(st, s, tid, lane);
        __syncthreads();
        if (c + 1 < nchunks) load_chunk(st, cx, t0 + C, min(C, T - t0 - C), tid, true);

        gram_phase(s, wave, n, h, true);
        __syncthreads();
        solve_phase<false>(s, tid, wave, lane);
        __syncthreads();

        // ---- X = K S^T, Z = Q S^T (this wave's 16 columns) ----
        f32x4 X[NT], Z[NT];
#pragma unroll
        for (int rt = 0; rt < NT; ++rt) { X[rt] = zero4(); Z[rt] = zero4(); }
        if constexpr (BF) {
#pragma unroll
            for (int ss = 0; ss < DK / 32; ++ss) {
                bf16x8 shi, slo;
                split8(Sacc[2 * ss], Sacc[2 * ss + 1], shi, slo);
#pragma unroll
                for (int rt = 0; rt < NT; ++rt) {
                    const bf16x8 kf = ld_perm8(&s.K[16 * rt + n][0], ss, h);
                    X[rt] = mfma_bf16(kf, shi, X[rt]);
                    X[rt] = mfma_bf16(kf, slo, X[rt]);
                    const bf16x8 qf = ld_perm8(&s.Q[16 * rt + n][0], ss, h);
                    Z[rt] = mfma_bf16(qf, shi, Z[rt]);
                    Z[rt] = mfma_bf16(qf, slo, Z[rt]);
                }
            }
        } else {
#pragma unroll
            for (int t = 0; t < NK; ++t)
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    const float sb = Sacc[t][j];
#pragma unroll
                    for (int rt = 0; rt < NT; ++rt) {
                        X[rt] = mfma_f32(s.K[16 * rt + n][16 * t + 4 * h + j], sb, X[rt]);
                        Z[rt] = mfma_f32(s.Q[16 * rt + n][16 * t + 4 * h + j], sb, Z[rt]);
                    }
                }
        }

        // ---- pseudo-value input Y = diag(eta) V - diag(beta) diag(exp g) X ----
        f32x4 Y[NT];
#pragma unroll
        for (int rt = 0; rt < NT; ++rt)
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int r = 16 * rt + 4 * h + j;
                Y[rt][j] = s.eta[r] * (float)s.V[r][16 * wave + n] - s.beta[r] * s.eg[r] * X[rt][j];
            }

        // ---- V' = T Y ----
        f32x4 Vp[NT];
#pragma unroll
        for (int rt = 0; rt < NT; ++rt) Vp[rt] = zero4();
        if constexpr (BF) {
#pragma unroll
            for (int ss = 0; ss < C / 32; ++ss) {
                bf16x8 yhi, ylo;
                split8(Y[2 * ss], Y[2 * ss + 1], yhi, ylo);
#pragma unroll
                for (int rt = 0; rt < NT; ++rt) {
                    if (32 * ss > 16 * rt + 15) continue;   // above the diagonal
                    const bf16x8 th = ld_perm8(&s.Tt[16 * rt + n][0], ss, h);
                    const bf16x8 tl = ld_perm8(&s.Ttl[16 * rt + n][0], ss, h);
                    Vp[rt] = mfma_bf16(th, yhi, Vp[rt]);
                    Vp[rt] = mfma_bf16(th, ylo, Vp[rt]);
                    Vp[rt] = mfma_bf16(tl, yhi, Vp[rt]);
                }
            }
        } else {
#pragma unroll
            for (int t = 0; t < NT; ++t)
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    const float yb = Y[t][j];
#pragma unroll
                    for (int rt = t; rt < NT; ++rt)
                        Vp[rt] = mfma_f32(s.Tt[16 * rt + n][16 * t + 4 * h + j], yb, Vp[rt]);
                }
        }

        // ---- O = diag(exp g) Z + P V' ----
        f32x4 PV[NT];
#pragma unroll
        for (int rt = 0; rt < NT; ++rt) PV[rt] = zero4();
        if constexpr (BF) {
#pragma unroll
            for (int ss = 0; ss < C / 32; ++ss) {
                bf16x8 vhi, vlo;
                split8(Vp[2 * ss], Vp[2 * ss + 1], vhi, vlo);
#pragma unroll
                for (int rt = 0; rt < NT; ++rt) {
                    if (32 * ss > 16 * rt + 15) continue;
                    const bf16x8 ph = ld_perm8(&s.P[16 * rt + n][0], ss, h);
                    const bf16x8 pl = ld_perm8(&s.Pl[16 * rt + n][0], ss, h);
                    PV[rt] = mfma_bf16(ph, vhi, PV[rt]);
                    PV[rt] = mfma_bf16(ph, vlo, PV[rt]);
                    PV[rt] = mfma_bf16(pl, vhi, PV[rt]);
                }
            }
        } else {
#pragma unroll
            for (int t = 0; t < NT; ++t)
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    const float vb = Vp[t][j];
#pragma unroll
                    for (int rt = t; rt < NT; ++rt)
                        PV[rt] = mfma_f32(s.P[16 * rt + n][16 * t + 4 * h + j], vb, PV[rt]);
                }
        }
        {
            const size_t obase = ((size_t)bh * T + t0) * dv + col;
#pragma unroll
            for (int rt = 0; rt < NT; ++rt)
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    const int r = 16 * rt + 4 * h + j;
                    if (r < Lc) {
                        const float o = s.eg[r] * Z[rt][j] + PV[rt][j];
                        if (p.o_bf16)
                            reinterpret_cast<__bf16*>(p.O)[obase + (size_t)r * dv] = (__bf16)o;
                        else
                            reinterpret_cast<float*>(p.O)[obase + (size_t)r * dv] = o;
                    }
                }
        }

        // ---- S^T <- exp(g_last) S^T + K^T diag(exp(g_last - g)) V' ----
        const float gl = s.glast;
#pragma unroll
        for (int t = 0; t < NK; ++t)
#pragma unroll
            for (int j = 0; j < 4; ++j) Sacc[t][j] *= gl;
        f32x4 Vd[NT];
#pragma unroll
        for (int rt = 0; rt < NT; ++rt)
#pragma unroll
            for (int j = 0; j < 4; ++j) Vd[rt][j] = s.dec[16 * rt + 4 * h + j] * Vp[rt][j];
        if constexpr (BF) {
#pragma unroll
            for (int ss = 0; ss < C / 32; ++ss) {
                bf16x8 vhi, vlo;
                split8(Vd[2 * ss], Vd[2 * ss + 1], vhi, vlo);
#pragma unroll
                for (int t = 0; t < NK; ++t) {
                    const bf16x8 kt = ld_perm8(&s.Kt[16 * t + n][0], ss, h);
                    Sacc[t] = mfma_bf16(kt, vhi, Sacc[t]);
                    Sacc[t] = mfma_bf16(kt, vlo, Sacc[t]);
                }
            }
        } else {
#pragma unroll
            for (int rt = 0; rt < NT; ++rt)
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    const float vb = Vd[rt][j];
#pragma unroll
                    for (int t = 0; t < NK; ++t)
                        Sacc[t] = mfma_f32(s.K[16 * rt + 4 * h + j][16 * t + n], vb, Sacc[t]);
                }
        }
    }

#pragma unroll
    for (int t = 0; t < NK; ++t)
#pragma unroll
        for (int j = 0; j < 4; ++j) p.S_final[sbase + 16 * t + 4 * h + j] = Sacc[t][j];
}

// ---------------------------------------------------------------------------
// Chunk-local stage kernel: T, W = T diag(beta) diag(exp g) K and
// U = T diag(beta) V for every chunk.  One workgroup per (b, h, chunk,
// value-column tile); the same load / Gram / solve phases as the fused kernel.
// ---------------------------------------------------------------------------
template <int C, int DK, int NW, bool BF>
__global__ __launch_bounds__(NW * 64) void gdn_prep_kernel(FwdParams p) {
    using L = Lds<C, DK, NW, BF>;
    using St = Stage<C, DK, NW, BF>;
    using In = typename L::In;
    constexpr int NT = C / 16;
    __shared__ L s;

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int n = lane & 15;
    const int h = lane >> 4;

    const int T = p.T, dv = p.dv;
    const int nchunks = (T + C - 1) / C;
    const int tile = blockIdx.x % p.n_tiles;
    const int c = (blockIdx.x / p.n_tiles) % nchunks;
    const int bh = blockIdx.x / (p.n_tiles * nchunks);
    const int col_tile = tile * L::DVT;
    const int t0 = c * C;
    const int Lc = min(C, T - t0);

    ChunkCtx<C, DK, NW, BF> cx;
    cx.kb = reinterpret_cast<const In*>(p.k) + (size_t)bh * T * DK;
    cx.qb = nullptr;
    cx.vb = reinterpret_cast<const In*>(p.v) + (size_t)bh * T * dv;
    cx.ab = p.alpha ? p.alpha + (size_t)bh * T : nullptr;
    cx.bb = p.beta + (size_t)bh * T;
    cx.eb = p.eta ? p.eta + (size_t)bh * T : nullptr;
    cx.T = T;
    cx.dv = dv;
    cx.col0 = col_tile;

    zero_upper(s, tid);
    St st;
    load_chunk(st, cx, t0, Lc, tid, false);
    __syncthreads();
    store_chunk(st, s, tid, lane);
    __syncthreads();
    gram_phase(s, wave, n, h, false);
    __syncthreads();
    solve_phase<true>(s, tid, wave, lane);
    __syncthreads();

    if (tile == 0 && p.T_out) {
        float* Tb = p.T_out + ((size_t)bh * nchunks + c) * C * C;
        for (int idx = tid; idx < C * C; idx += NW * 64) {
            const int r = idx / C, i = idx % C;
            Tb[idx] = (i <= r) ? s.Tm[r][i] : 0.f;
        }
    }
    // W: output tiles (rt, 16-column d_k tile) spread over the waves.
    if (tile == 0 && p.W_out) {
        for (int job = wave; job < NT * (DK / 16); job += NW) {
            const int rt = job % NT, dt = job / NT;
            f32x4 acc = zero4();
            if constexpr (BF) {
#pragma unroll
                for (int ss = 0; ss < C / 32; ++ss) {
                    float x[8];
#pragma unroll
                    for (int e = 0; e < 8; ++e) {
                        const int r = 32 * ss + 8 * h + e;
                        x[e] = s.eg[r] * (float)s.Kt[16 * dt + n][r];
                    }
                    bf16x8 bhi, blo;
#pragma unroll
                    for (int e = 0; e < 8; ++e) {
                        __bf16 a, b;
                        split_bf16(x[e], a, b);
                        bhi[e] = a;
                        blo[e] = b;
                    }
                    const bf16x8 th = ld_nat8(&s.Tt[16 * rt + n][0], ss, h);
                    const bf16x8 tl = ld_nat8(&s.Ttl[16 * rt + n][0], ss, h);
                    acc = mfma_bf16(th, bhi, acc);
                    acc = mfma_bf16(th, blo, acc);
                    acc = mfma_bf16(tl, bhi, acc);
                }
            } else {
#pragma unroll
                for (int kk = 0; kk < C / 4; ++kk) {
                    const int r = 4 * kk + h;
                    acc = mfma_f32(s.Tt[16 * rt + n][r], s.eg[r] * s.K[r][16 * dt + n], acc);
                }
            }
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int r = 16 * rt + 4 * h + j;
                if (r < Lc) p.W_out[((size_t)bh * T + t0 + r) * DK + 16 * dt + n] = acc[j];
            }
        }
    }
    // U: wave w owns 16 value columns of this tile.
    if (p.U_out) {
        const int col = col_tile + 16 * wave + n;
#pragma unroll
        for (int rt = 0; rt < NT; ++rt) {
            f32x4 acc = zero4();
            if constexpr (BF) {
#pragma unroll
                for (int ss = 0; ss < C / 32; ++ss) {
                    bf16x8 vb;
#pragma unroll
                    for (int e = 0; e < 8; ++e) vb[e] = s.V[32 * ss + 8 * h + e][16 * wave + n];
                    acc = mfma_bf16(ld_nat8(&s.Tt[16 * rt + n][0], ss, h), vb, acc);
                    acc = mfma_bf16(ld_nat8(&s.Ttl[16 * rt + n][0], ss, h), vb, acc);
                }
            } else {
#pragma unroll
                for (int kk = 0; kk < C / 4; ++kk)
                    acc = mfma_f32(s.Tt[16 * rt + n][4 * kk + h], s.V[4 * kk + h][16 * wave + n], acc);
            }
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int r = 16 * rt + 4 * h + j;
                if (r < Lc) p.U_out[((size_t)bh * T + t0 + r) * dv + col] = acc[j];
            }
        }
    }
}

}  // namespace gdn
