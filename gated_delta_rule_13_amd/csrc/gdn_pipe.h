// gdn_pipe.h -- software-pipelined fused kernel (bf16 inputs) for the
// chunkwise gated delta rule on gfx950.
//
// Same chunk algebra as gdn_kernels.h ("从零开始的 GDN 推导": A, U and W, S
// update, O update; transposed to the d_v x d_k state).  Two changes of
// evaluation order, both exact in real arithmetic:
//
// 1. T = (I - A)^{-1} is never formed.  The pseudo-values solve the unit
//    lower-triangular system (I - A) V' = Y with
//    Y = diag(eta) V - diag(beta) diag(exp g) K S^T (so that V' = U - W S^T;
//    eta, the write strength, equals beta unless given), by forward
//    substitution over 16-row blocks ("RNN的复兴03", section 2.3.1, grouped
//    by blocks):
//        V'_b = T_bb (Y_b + sum_{c<b} A_bc V'_c),
//    where T_bb = (I - A_bb)^{-1} are the 16 x 16 diagonal blocks, solved by
//    substitution on VALU (one lane per row of T_bb).  The coupling terms
//    A_bc V'_c are dense 16 x 16 x 16 contractions; each one's bf16 hi / lo
//    products run as two 16 x 16 x 32 MFMAs (operands concatenated along k).
// 2. Work is split by role inside the workgroup: NS "scan" waves each own 16
//    value columns and that slice of the fp32 state (S^T in MFMA
//    accumulators); NP = 4 "prep" waves build the next chunk's chunk-local
//    quantities (decay prefix, Gram matrix, masked scores, diagonal-block
//    solves) while the scan waves consume the current chunk.  Prep wave 0
//    owns the per-token gates and the diagonal blocks, with the keys it
//    needs for them in registers; prep waves 1..3 stage keys and queries in
//    LDS and own the off-diagonal and score tiles.  Per chunk c:
//       phase A: scan    X = K S^T, Z^T = S Q^T, block substitution for V'
//                prep 0  decay vectors and diagonal blocks A_bb of chunk c + 1
//                prep 1+ masked scores P of chunk c; stage chunk c + 1
//       phase B: scan    O^T = Z^T + V'^T P^T, state update
//                prep 0  diagonal-block solves T_bb of chunk c + 1; with one
//                        or two scan waves also chunk c + 1's values, written
//                        transposed into LDS for the scan's next phase A
//                prep 1+ Gram tiles of chunk c + 1 (MFMA), off-diagonal A blocks
//    Keys, queries, transposed keys and the block matrices are double-buffered
//    in LDS.  The output products are taken transposed (operands swapped) so
//    that each lane ends with four consecutive columns of one output row.
//
// Precision: as in gdn_kernels.h -- inputs exact in bf16, every derived MFMA
// operand split into bf16 hi + lo, fp32 accumulation and fp32 state.
#pragma once
#include <type_traits>

#include "gdn_device.h"
#include "gdn_kernels.h"

namespace gdn {

__device__ __forceinline__ bf16x8 cat8(bf16x4 a, bf16x4 b) {
    return __builtin_shufflevector(a, b, 0, 1, 2, 3, 4, 5, 6, 7);
}

__device__ __forceinline__ void split4(f32x4 x, bf16x4& hi, bf16x4& lo) {
    hi = __builtin_convertvector(x, bf16x4);
    const f32x4 back = __builtin_convertvector(hi, f32x4);
    lo = __builtin_convertvector(x - back, bf16x4);
}

// Order LDS traffic of this wave (cross-lane exchange through LDS).
__device__ __forceinline__ void wave_lds_sync() {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_s_waitcnt(0xc07f);   // lgkmcnt(0)
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

template <int I, int N, typename F>
__device__ __forceinline__ void static_for(F&& f) {
    if constexpr (I < N) {
        f(std::integral_constant<int, I>{});
        static_for<I + 1, N>(f);
    }
}

constexpr int kPrepWaves = 4;

typedef __attribute__((ext_vector_type(2))) float f32x2;

// An integer whose value the compiler may not reason about (no instruction
// is emitted): used to keep it from proving 16-byte alignment of an offset.
__device__ __forceinline__ int lds_opaque(int v) {
    asm volatile("" : "+v"(v));
    return v;
}

// Four floats at base + o (o a multiple of 4) read as two 8-byte halves.
// For the scan's per-token vectors, which the 16 lanes of a row group read
// at one address (a broadcast), a pair of 8-byte reads (ds_read2_b64)
// measured faster than one 16-byte read (about 5 % of the kernel).
__device__ __forceinline__ f32x4 lds_bcast4(const float* base, int o) {
    o = lds_opaque(o);
    const f32x2 a = *reinterpret_cast<const f32x2*>(base + o);
    const f32x2 b = *reinterpret_cast<const f32x2*>(base + o + 2);
    return f32x4{a[0], a[1], b[0], b[1]};
}

// Whether prep wave 0 stages the value tile in LDS (VT) for the scan waves;
// with four scan waves the tile is twice as large and the scan waves load
// their values themselves.
constexpr bool pipe_stages_values(int ns) { return ns <= 2; }

// Position in an LDS key / query row of natural element k (a multiple of 4):
// within each 32-element block, group g = (k mod 32) / 4 of four elements
// goes to 8 g for g < 4 and to 8 (g - 4) + 4 for g >= 4.
__device__ __forceinline__ int kq_pos(int k) {
    const int g = (k & 31) >> 2;
    return (k & ~31) + (g < 4 ? 8 * g : 8 * (g - 4) + 4);
}

template <int C, int DK, int NS, bool ETA>
struct alignas(16) PipeLds {
    static constexpr int NT = C / 16;
    // Key / query rows: each 32-element block stored in the scan's k-order
    // (elements 4h..4h+3 then 16+4h..16+4h+3 for h = 0..3), so that any MFMA
    // operand slice is one aligned 16-byte read; row stride d_k + 8 (an odd
    // multiple of 16 bytes modulo 128: 16-byte reads of 8 rows hit distinct banks).
    static constexpr int KP = DK + 8;
    // Row strides against LDS bank conflicts (32 banks of 4 bytes; an 8-byte
    // access serves 16 lanes per pass): 8-byte column slices of 16
    // consecutive rows hit distinct banks when the stride is an odd multiple
    // of 8 bytes modulo 128, as for C + 4 bf16 (C = 32, 64) and 20 bf16;
    // 16-byte slices of 8 rows when it is an odd multiple of 16, as for
    // 20 floats and d_k + 8 bf16.
    static constexpr int CP = C + 4;    // row stride of C-wide rows (bf16)
    static constexpr int BP = 20;       // row stride of 16 x 16 blocks (bf16 and fp32)
    __bf16 K[2][C][KP];
    __bf16 Q[2][C][KP];
    __bf16 Kt[2][DK][CP];
    __bf16 Ph[C][CP];                   // masked decayed scores, hi
    __bf16 Pl[C][CP];                   //                        lo
    static constexpr int NB = NT * (NT + 1) / 2;   // blocks on and below the diagonal
    static constexpr int bidx(int b, int cb) { return b * (b + 1) / 2 + cb; }
    // block matrices by chunk parity: block (b, c<b) holds A_bc, block (b, b) holds T_bb
    __bf16 Bh[2][NB][16][BP];           // hi
    __bf16 Bl[2][NB][16][BP];           // lo
    float Ad[NT][16][BP];               // diagonal blocks of A, fp32
    float g2[2][C];                     // inclusive cumsum of log2 alpha
    float er[2][C];                     // 2^(g2_r - g2_ref): row factor of exp(g_r - g_i)
    float fi[2][C];                     // 2^(g2_ref - g2_i): column factor
    int sep[2];                         // row x column factors safe in fp32 for this chunk
    float eg[2][C];                     // 2^g2 = exp(g)
    float dec[2][C];                    // exp(g_last - g)
    float beta[2][C];
    float glast[2];                     // exp(g_last)
    // with a separate write strength only: eta and beta exp(g)
    float eta[ETA ? 2 : 1][ETA ? C : 4];
    float bge[ETA ? 2 : 1][ETA ? C : 4];
    // the workgroup's 16 NS value columns of one chunk, transposed (a row per
    // column, C + 4 row stride as for the scores): a scan lane reads its four
    // consecutive tokens of one column as one 8-byte read.  Last, so that the
    // offsets of the members above do not depend on it.
    static constexpr bool VST = pipe_stages_values(NS);
    __bf16 VT[VST ? 16 * NS : 1][VST ? CP : 8];
};

// Chunk-local tile jobs of prep waves 1..NP-1, round-robin.  Kinds:
// 1 = off-diagonal block of A, 2 = block of the masked scores P (kind 0,
// the diagonal blocks of A, belongs to prep wave 0, which computes them from
// registers and solves them).  Encoding: (kind << 16) | (rt << 8) | ct for
// tile (rt, ct), ct <= rt.
template <int NT, int NP>
struct PrepJobs {
    static constexpr int NPAIR = NT * (NT + 1) / 2;
    static constexpr int NOFF = NT * (NT - 1) / 2;
    static constexpr int NREST = NOFF + NPAIR;
    static constexpr int pair_rt(int p) {
        int rt = 0, ct = p;
        while (ct > rt) { ct -= rt + 1; ++rt; }
        return rt;
    }
    static constexpr int pair_ct(int p) {
        int rt = 0, ct = p;
        while (ct > rt) { ct -= rt + 1; ++rt; }
        return ct;
    }
    static constexpr int off_pair(int j) {
        int cnt = 0;
        for (int q = 0; q < NPAIR; ++q)
            if (pair_rt(q) != pair_ct(q)) {
                if (cnt == j) return q;
                ++cnt;
            }
        return 0;
    }
    // k-th job of the round-robin list (off-diagonal A blocks, then P blocks)
    static constexpr int rest(int k) {
        if (k < NOFF) {
            const int q = off_pair(k);
            return (1 << 16) | (pair_rt(q) << 8) | pair_ct(q);
        }
        const int q = k - NOFF;
        return (2 << 16) | (pair_rt(q) << 8) | pair_ct(q);
    }
    static constexpr int owner(int k) { return 1 + k % (NP - 1); }
    static constexpr int count(int w) {
        if (w == 0) return 0;
        int n = 0;
        for (int k = 0; k < NREST; ++k) n += owner(k) == w;
        return n;
    }
    static constexpr int job(int w, int j) {
        for (int k = 0; k < NREST; ++k)
            if (owner(k) == w) {
                if (j == 0) return rest(k);
                --j;
            }
        return -1;
    }
    static constexpr int maxjobs() {
        int m = 1;
        for (int w = 0; w < NP; ++w) m = count(w) > m ? count(w) : m;
        return m;
    }
};

// ETA: a separate write strength is given (p.eta); otherwise eta = beta and
// the substitution's right-hand side keeps the factored form
// diag(beta) (V - diag(exp g) K S^T).
template <int C, int DK, int NS, bool ETA>
__global__ __launch_bounds__((NS + kPrepWaves) * 64) void gdn_fwd_pipe_kernel(FwdParams p) {
    constexpr int NP = kPrepWaves;
    using L = PipeLds<C, DK, NS, ETA>;
    constexpr bool VST = L::VST;
    using J = PrepJobs<C / 16, NP>;
    constexpr int NT = C / 16;
    constexpr int NK = DK / 16;
    constexpr int DVT = 16 * NS;
    constexpr int NTHR = (NS + NP) * 64;
    constexpr int KV = C * DK / 8;        // 16-byte vectors in a key tile
    constexpr int NSTG = NP - 1;          // prep waves 1..NP-1 stage keys and queries
    constexpr int NKV = (KV + 64 * NSTG - 1) / (64 * NSTG);   // per staging lane
    constexpr int NDS = DK / 32;          // k-steps of a Gram tile
    constexpr int MAXJ = J::maxjobs();
    static_assert(sizeof(L) <= 160 * 1024, "LDS budget");
    __shared__ L s;

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    // wave index as a scalar: role branches below are uniform per wave
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int n = lane & 15;
    const int h = lane >> 4;
    const bool scan = wave < NS;
    const int pw = wave - NS;             // prep wave 0..NP-1
    const int plane = tid - (NS + 1) * 64;  // 0..64*NSTG-1 on prep waves 1..NP-1

    // Workgroups are dispatched round-robin over the 8 XCDs (L2 domains);
    // when the head count allows it, all value tiles of one head get block
    // ids congruent mod 8, so they share that XCD's L2 copy of K and Q.
    int tile, bh;
    if (p.xcd_groups) {
        const int xcd = blockIdx.x & 7, slot = blockIdx.x >> 3;
        tile = slot % p.n_tiles;
        bh = xcd + 8 * (slot / p.n_tiles);
    } else {
        tile = blockIdx.x % p.n_tiles;
        bh = blockIdx.x / p.n_tiles;
    }
    // padding workgroups of an XCD-grouped grid (B * H rounded up to a
    // multiple of 8) have no head: they leave before any barrier
    if (bh >= p.B * p.H) return;
    const int T = p.T, dv = p.dv;
    const int nchunks = (T + C - 1) / C;
    const __bf16* kb = reinterpret_cast<const __bf16*>(p.k) + (size_t)bh * T * DK;
    const __bf16* qb = reinterpret_cast<const __bf16*>(p.q) + (size_t)bh * T * DK;
    const __bf16* vb = reinterpret_cast<const __bf16*>(p.v) + (size_t)bh * T * dv;
    const float* ab = p.alpha ? p.alpha + (size_t)bh * T : nullptr;
    const float* bb = p.beta + (size_t)bh * T;
    const float* eb = p.eta ? p.eta + (size_t)bh * T : nullptr;
    // per-head buffers: rows past the end of the sequence read as zero
    const buf_t kbuf = buffer_over(kb, (uint32_t)T * DK * 2);
    const buf_t qbuf = buffer_over(qb, (uint32_t)T * DK * 2);
    const int col0 = tile * DVT + 16 * wave;  // scan waves: first value column of this wave

    // the upper part of the score matrix stays zero
    for (int i = tid; i < C * L::CP; i += NTHR) {
        (&s.Ph[0][0])[i] = (__bf16)0.f;
        (&s.Pl[0][0])[i] = (__bf16)0.f;
    }

    // Each role runs its own loop; both execute two workgroup barriers per
    // chunk (plus two in the prologue), so the barriers pair up by count.
    if (!scan) {
        // ============================ prep waves ============================
        // Prep waves 1..NP-1 stage keys and queries: registers, two sets by
        // chunk parity (chunk cc is loaded into set cc & 1 two iterations
        // before it is written to LDS).  Keys are assigned row-fastest (one
        // row per lane) so that the transposed copy is written in contiguous
        // runs; queries use the row-major order.  Prep wave 0 stages the
        // per-token gates (same two sets) and keeps the next chunk's keys in
        // registers in MFMA operand order for its diagonal Gram tiles.
        uint4 stK[2][NKV], stQ[2][NKV];
        // prep wave 0 (VST): the next chunk's value tile (16 NS columns),
        // loaded one chunk ahead and written transposed in phase B
        constexpr int VV = C * 2 * NS;          // 16-byte vectors in a value tile
        constexpr int NVV = VST ? (VV + 63) / 64 : 1;
        uint4 stV[NVV];
        const buf_t vbuf_p = buffer_over(vb, (uint32_t)T * dv * 2);
        const int vcol0 = tile * DVT;
        // rows past the end of the sequence read as zero
        auto v_load = [&](int cc) __attribute__((always_inline)) {
            const int t0 = cc * C;
            static_for<0, NVV>([&](auto I) {
                constexpr int i = decltype(I)::value;
                const int vi = lane + i * 64;
                if (i + 1 < NVV || vi < VV) {
                    const int r = vi % C, c8 = (vi / C) * 8;
                    stV[i] = buf_load_16B(vbuf_p, 2u * ((t0 + r) * dv + vcol0 + c8));
                }
            });
        };
        auto v_store = [&]() __attribute__((always_inline)) {
            static_for<0, NVV>([&](auto I) {
                constexpr int i = decltype(I)::value;
                const int vi = lane + i * 64;
                if (i + 1 < NVV || vi < VV) {
                    const int r = vi % C, c8 = (vi / C) * 8;
                    const uint4 vv = stV[i];
                    static_for<0, 8>([&](auto X) {
                        constexpr int x = decltype(X)::value;
                        const unsigned word = x < 2 ? vv.x : x < 4 ? vv.y : x < 6 ? vv.z : vv.w;
                        *reinterpret_cast<unsigned short*>(&s.VT[c8 + x][r]) =
                            (unsigned short)(word >> (16 * (x & 1)));
                    });
                }
            });
        };
        float stA[2] = {1.f, 1.f}, stB[2] = {0.f, 0.f}, stE[2] = {0.f, 0.f};
        f32x4 gacc[MAXJ];
        uint4 dK[NT][NDS];   // prep wave 0: keys of rows 16 rt + n, columns 32 ss + 8 h .. + 7

        auto prep_load = [&](auto PAR, int cc) __attribute__((always_inline)) {
            constexpr int par = decltype(PAR)::value;
            const int t0 = cc * C, Lc = min(C, T - t0);
            if (pw == 0) {
                const int tt = t0 + min(lane, Lc - 1);
                stA[par] = ab ? ab[tt] : 1.f;
                stB[par] = bb[tt];
                if constexpr (ETA) stE[par] = eb[tt];
                return;
            }
            static_for<0, NKV>([&](auto I) {
                constexpr int i = decltype(I)::value;
                const int vi = plane + i * 64 * NSTG;
                if (i + 1 < NKV || vi < KV) {
                    {
                        const int r = vi % C, c8 = (vi / C) * 8;
                        stK[par][i] = buf_load_16B(kbuf, 2u * ((t0 + r) * DK + c8));
                    }
                    {
                        const int r = vi / (DK / 8), c8 = (vi % (DK / 8)) * 8;
                        stQ[par][i] = buf_load_16B(qbuf, 2u * ((t0 + r) * DK + c8));
                    }
                }
            });
        };
        // keys of chunk cc for prep wave 0's diagonal Gram tiles (rows past
        // the end of the sequence read as zero)
        auto diag_load = [&](int cc) __attribute__((always_inline)) {
            const int t0 = cc * C;
#pragma unroll
            for (int rt = 0; rt < NT; ++rt)
#pragma unroll
                for (int ss = 0; ss < NDS; ++ss)
                    dK[rt][ss] = buf_load_16B(kbuf, 2u * ((t0 + 16 * rt + n) * DK + 32 * ss + 8 * h));
        };
        auto prep_store = [&](auto PAR, int cc) __attribute__((always_inline)) {
            constexpr int par = decltype(PAR)::value;
            const int buf = cc & 1;
            const int Lc = min(C, T - cc * C);
            if (pw != 0) {
                static_for<0, NKV>([&](auto I) {
                    constexpr int i = decltype(I)::value;
                    const int vi = plane + i * 64 * NSTG;
                    if (i + 1 < NKV || vi < KV) {
                        {
                            // rows past the end of the sequence were loaded as zeros
                            const int r = vi % C, c8 = (vi / C) * 8;
                            const uint4 kv = stK[par][i];
                            *reinterpret_cast<uint2*>(&s.K[buf][r][kq_pos(c8)]) = make_uint2(kv.x, kv.y);
                            *reinterpret_cast<uint2*>(&s.K[buf][r][kq_pos(c8 + 4)]) = make_uint2(kv.z, kv.w);
                            static_for<0, 8>([&](auto X) {
                                constexpr int x = decltype(X)::value;
                                const unsigned word = x < 2 ? kv.x : x < 4 ? kv.y : x < 6 ? kv.z : kv.w;
                                *reinterpret_cast<unsigned short*>(&s.Kt[buf][c8 + x][r]) =
                                    (unsigned short)(word >> (16 * (x & 1)));
                            });
                        }
                        {
                            const int r = vi / (DK / 8), c8 = (vi % (DK / 8)) * 8;
                            const uint4 qv = stQ[par][i];
                            *reinterpret_cast<uint2*>(&s.Q[buf][r][kq_pos(c8)]) = make_uint2(qv.x, qv.y);
                            *reinterpret_cast<uint2*>(&s.Q[buf][r][kq_pos(c8 + 4)]) = make_uint2(qv.z, qv.w);
                        }
                    }
                });
            } else {
                // padding tokens: alpha = 1, beta = eta = 0 (identity transitions)
                const float a = lane < Lc ? stA[par] : 1.f;
                const float l2 = (lane < C) ? __builtin_amdgcn_logf(a) : 0.f;
                const float g = wave_inclusive_scan(l2, lane);
                const float gl = lane_value(g, C - 1);
                // exp(g_r - g_i) = 2^(g2_r - ref) * 2^(ref - g2_i) with ref the middle
                // of the chunk; used when the chunk's decay range keeps both factors
                // far inside fp32 (else the formation exponentiates each ratio).
                const float ref = lane_value(g, C / 2);
                const float g0 = lane_value(g, 0);
                if (lane < C) {
                    s.g2[buf][lane] = g;
                    s.eg[buf][lane] = __builtin_amdgcn_exp2f(g);
                    s.dec[buf][lane] = __builtin_amdgcn_exp2f(gl - g);
                    s.beta[buf][lane] = lane < Lc ? stB[par] : 0.f;
                    if constexpr (ETA) {
                        s.eta[buf][lane] = lane < Lc ? stE[par] : 0.f;
                        s.bge[buf][lane] = lane < Lc ? stB[par] * __builtin_amdgcn_exp2f(g) : 0.f;
                    }
                    s.er[buf][lane] = __builtin_amdgcn_exp2f(g - ref);
                    s.fi[buf][lane] = __builtin_amdgcn_exp2f(ref - g);
                }
                if (lane == 0) {
                    s.glast[buf] = __builtin_amdgcn_exp2f(gl);
                    s.sep[buf] = (g0 - gl) <= 96.f;
                }
            }
        };
        // Gram / score tiles: lane holds row r = 16 rt + n, columns 16 ct + 4 h + e.
        auto gram = [&](auto W, int cc) __attribute__((always_inline)) {
            constexpr int w = decltype(W)::value;
            const int buf = cc & 1;
            static_for<0, J::count(w)>([&](auto JJ) {
                constexpr int j = decltype(JJ)::value;
                constexpr int code = J::job(w, j);
                constexpr int kind = code >> 16;
                constexpr int rt = (code >> 8) & 255, ct = code & 255;
                const __bf16* arow = &s.K[buf][16 * ct + n][0];
                const __bf16* brow = kind == 2 ? &s.Q[buf][16 * rt + n][0] : &s.K[buf][16 * rt + n][0];
                f32x4 acc = zero4();
#pragma unroll
                for (int ss = 0; ss < DK / 32; ++ss)
                    acc = mfma_bf16(*reinterpret_cast<const bf16x8*>(arow + 32 * ss + 8 * h),
                                    *reinterpret_cast<const bf16x8*>(brow + 32 * ss + 8 * h), acc);
                gacc[j] = acc;
            });
        };
        // A_ri = -beta_r exp(g_r - g_i) k_r.k_i (i < r), P_ri = exp(g_r - g_i) q_r.k_i (i <= r).
        // SEP: exp(g_r - g_i) from the separable row / column factors.
        // SCORES: form the P blocks (else the A blocks) of this wave's jobs.
        auto form = [&](auto W, auto SEP, auto SCORES, int cc) __attribute__((always_inline)) {
            constexpr int w = decltype(W)::value;
            constexpr bool sep = decltype(SEP)::value;
            constexpr bool scores = decltype(SCORES)::value;
            const int buf = cc & 1;
            static_for<0, J::count(w)>([&](auto JJ) {
                constexpr int j = decltype(JJ)::value;
                constexpr int code = J::job(w, j);
                constexpr int kind = code >> 16;
                constexpr int rt = (code >> 8) & 255, ct = code & 255;
                if constexpr ((kind == 2) == scores) {
                const int r = 16 * rt + n;
                const int i0 = 16 * ct + 4 * h;
                const float br = s.beta[buf][r];
                f32x4 d;
                if constexpr (sep) {
                    d = s.er[buf][r] * *reinterpret_cast<const f32x4*>(&s.fi[buf][i0]);
                } else {
                    const float g2r = s.g2[buf][r];
                    const f32x4 g2i = *reinterpret_cast<const f32x4*>(&s.g2[buf][i0]);
#pragma unroll
                    for (int e = 0; e < 4; ++e) d[e] = __builtin_amdgcn_exp2f(g2r - g2i[e]);
                }
                f32x4 v;
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const int i = i0 + e;
                    if constexpr (kind == 2) v[e] = (i <= r) ? d[e] * gacc[j][e] : 0.f;
                    else if constexpr (kind == 0) v[e] = (i < r) ? -br * d[e] * gacc[j][e] : 0.f;
                    else v[e] = -br * d[e] * gacc[j][e];
                }
                if constexpr (kind == 2) {
                    bf16x4 hi, lo;
                    split4(v, hi, lo);
                    *reinterpret_cast<bf16x4*>(&s.Ph[r][i0]) = hi;
                    *reinterpret_cast<bf16x4*>(&s.Pl[r][i0]) = lo;
                } else if constexpr (kind == 0) {
                    // row n, columns 4h .. 4h + 3 of diagonal block rt
                    *reinterpret_cast<f32x4*>(&s.Ad[rt][n][4 * h]) = v;
                } else {
                    bf16x4 hi, lo;
                    split4(v, hi, lo);
                    *reinterpret_cast<bf16x4*>(&s.Bh[buf][L::bidx(rt, ct)][n][4 * h]) = hi;
                    *reinterpret_cast<bf16x4*>(&s.Bl[buf][L::bidx(rt, ct)][n][4 * h]) = lo;
                }
                }
            });
        };
        // Prep wave 0: the diagonal blocks A_bb of chunk cc, Gram tiles from the
        // keys held in registers (the same register is both MFMA operands),
        // formed in fp32 for the solve.  Lane holds row r = 16 rt + n,
        // columns 16 rt + 4 h + e.
        auto diag_blocks = [&](int cc) __attribute__((always_inline)) {
            const int buf = cc & 1;
            auto run = [&](auto SEP) __attribute__((always_inline)) {
                constexpr bool sep = decltype(SEP)::value;
                static_for<0, NT>([&](auto RT) {
                    constexpr int rt = decltype(RT)::value;
                    f32x4 acc = zero4();
#pragma unroll
                    for (int ss = 0; ss < NDS; ++ss) {
                        const bf16x8 kv = __builtin_bit_cast(bf16x8, dK[rt][ss]);
                        acc = mfma_bf16(kv, kv, acc);
                    }
                    const int r = 16 * rt + n;
                    const int i0 = 16 * rt + 4 * h;
                    const float br = s.beta[buf][r];
                    f32x4 d;
                    if constexpr (sep) {
                        d = s.er[buf][r] * *reinterpret_cast<const f32x4*>(&s.fi[buf][i0]);
                    } else {
                        const float g2r = s.g2[buf][r];
                        const f32x4 g2i = *reinterpret_cast<const f32x4*>(&s.g2[buf][i0]);
#pragma unroll
                        for (int e = 0; e < 4; ++e) d[e] = __builtin_amdgcn_exp2f(g2r - g2i[e]);
                    }
                    f32x4 v;
#pragma unroll
                    for (int e = 0; e < 4; ++e) v[e] = (i0 + e < r) ? -br * d[e] * acc[e] : 0.f;
                    *reinterpret_cast<f32x4*>(&s.Ad[rt][n][4 * h]) = v;
                });
            };
            if (s.sep[buf]) run(std::true_type{});
            else run(std::false_type{});
        };
        // T_bb = (I - A_bb)^{-1}, all diagonal blocks at once: lane (b, i)
        // computes row i of T_bb from T = I + T A, i.e. the transposed
        // unit triangular system, by substitution from the last column down:
        //     T[i][k] = [i == k] + sum_{m > k} T[i][m] A[m][k].
        // Right-looking: once T[i][m] is final it is added into every
        // earlier column's partial sum, so one multiply-add per step sits on
        // the dependency chain.  Rows of A are read as broadcasts (lanes of
        // one block read the same words), two steps ahead of their use.
        auto diag_solve = [&](int cc) __attribute__((always_inline)) {
            const int buf = cc & 1;
            if (lane < 16 * NT) {
                const int b = lane >> 4, i = lane & 15;
                float part[16];
#pragma unroll
                for (int k = 0; k < 16; ++k) part[k] = (k == i) ? 1.f : 0.f;
                float x[16];
                f32x4 abuf[3][4];
                auto load_row = [&](auto M) __attribute__((always_inline)) {
                    constexpr int m = decltype(M)::value;
#pragma unroll
                    for (int q = 0; 4 * q < m; ++q)
                        abuf[m % 3][q] = *reinterpret_cast<const f32x4*>(&s.Ad[b][m][4 * q]);
                };
                load_row(std::integral_constant<int, 15>{});
                load_row(std::integral_constant<int, 14>{});
                static_for<0, 16>([&](auto J) {
                    constexpr int m = 15 - decltype(J)::value;
                    if constexpr (m - 2 > 0) load_row(std::integral_constant<int, m - 2>{});
                    x[m] = part[m];
#pragma unroll
                    for (int q = 0; 4 * q < m; ++q) {
                        const f32x4 a = abuf[m % 3][q];
#pragma unroll
                        for (int e = 0; e < 4; ++e)
                            if (4 * q + e < m) part[4 * q + e] = fmaf(x[m], a[e], part[4 * q + e]);
                    }
                });
                bf16x4 hi[4], lo[4];
#pragma unroll
                for (int q = 0; q < 4; ++q)
                    split4(f32x4{x[4 * q], x[4 * q + 1], x[4 * q + 2], x[4 * q + 3]}, hi[q], lo[q]);
                __bf16* th = &s.Bh[buf][L::bidx(b, b)][i][0];
                __bf16* tl = &s.Bl[buf][L::bidx(b, b)][i][0];
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    *reinterpret_cast<bf16x4*>(th + 4 * q) = hi[q];
                    *reinterpret_cast<bf16x4*>(tl + 4 * q) = lo[q];
                }
            }
        };
        // The whole prep loop is specialised per prep wave so that every tile
        // job index is a compile-time constant within one loop.
        auto prep_role = [&](auto W) __attribute__((always_inline)) {
            constexpr int w = decltype(W)::value;
            // waves 1..NP-1: Gram tiles of chunk cc and its off-diagonal A
            // blocks; the score tiles stay in registers until the next phase A
            auto chunk_matrices = [&](int cc) __attribute__((always_inline)) {
                gram(W, cc);
                if (s.sep[cc & 1]) form(W, std::true_type{}, std::false_type{}, cc);
                else form(W, std::false_type{}, std::false_type{}, cc);
            };
            // wave 0: decay vectors of chunk cc and its diagonal blocks A_bb;
            // then the keys of chunk cc + 1 into registers
            auto diag_work = [&](auto PAR, int cc) __attribute__((always_inline)) {
                prep_store(PAR, cc);
                wave_lds_sync();
                diag_blocks(cc);
                if (cc + 1 < nchunks) diag_load(cc + 1);
            };
            // one pipeline step; PAR = parity of chunk c
            auto step = [&](auto PAR, int c) __attribute__((always_inline)) {
                constexpr int nxt = decltype(PAR)::value ^ 1;
                // ---- phase A: scores of chunk c; stage chunk c + 1; its
                //      decay vectors and diagonal blocks ----
                if constexpr (w == 0) {
                    if (c + 1 < nchunks) {
                        diag_work(std::integral_constant<int, nxt>{}, c + 1);
                        if (c + 3 < nchunks) prep_load(std::integral_constant<int, nxt>{}, c + 3);
                    }
                } else {
                    if (s.sep[c & 1]) form(W, std::true_type{}, std::true_type{}, c);
                    else form(W, std::false_type{}, std::true_type{}, c);
                    if (c + 1 < nchunks) {
                        prep_store(std::integral_constant<int, nxt>{}, c + 1);
                        if (c + 3 < nchunks) prep_load(std::integral_constant<int, nxt>{}, c + 3);
                    }
                }
                __syncthreads();
                // ---- phase B: chunk c + 1's Gram tiles and off-diagonal A
                //      blocks (waves 1..), T_bb of its diagonal blocks (wave 0) ----
                if (c + 1 < nchunks) {
                    if constexpr (w != 0) {
                        chunk_matrices(c + 1);
                    } else {
                        if constexpr (VST) {
                            v_store();
                            if (c + 2 < nchunks) v_load(c + 2);
                        }
                        diag_solve(c + 1);
                    }
                }
                __syncthreads();
            };
            constexpr auto P0 = std::integral_constant<int, 0>{};
            constexpr auto P1 = std::integral_constant<int, 1>{};
            if constexpr (w == 0 && VST) v_load(0);
            prep_load(P0, 0);
            if (nchunks > 1) prep_load(P1, 1);
            if constexpr (w == 0) {
                diag_load(0);
                diag_work(P0, 0);
                if constexpr (VST) {
                    v_store();
                    if (nchunks > 1) v_load(1);
                }
                wave_lds_sync();
                diag_solve(0);
            } else {
                prep_store(P0, 0);
            }
            if (nchunks > 2) prep_load(P0, 2);
            __syncthreads();
            if constexpr (w != 0) chunk_matrices(0);
            __syncthreads();
            for (int c = 0; c < nchunks; c += 2) {
                step(P0, c);
                if (c + 1 < nchunks) step(P1, c + 1);
            }
        };
        switch (pw) {
            case 0: prep_role(std::integral_constant<int, 0>{}); break;
            case 1: prep_role(std::integral_constant<int, 1>{}); break;
            case 2: prep_role(std::integral_constant<int, 2>{}); break;
            default: prep_role(std::integral_constant<int, 3>{}); break;
        }
    } else {
        // ============================ scan waves ============================
        f32x4 Sacc[NK];           // Sacc[t][j] = S[col0 + n][16 t + 4 h + j]
        // without VST: this lane's values of the next chunk, bf16 bits (zero past the end)
        uint32_t vnext[VST ? 1 : NT][4];
        const buf_t vbuf = buffer_over(vb, (uint32_t)T * dv * 2);
        const uint32_t vlane = 2u * (4 * h * dv + col0 + n);
        auto load_v = [&](int cc) __attribute__((always_inline)) {
            if constexpr (!VST) {
                const int t0 = cc * C;
                static_for<0, NT>([&](auto RT) {
                    constexpr int rt = decltype(RT)::value;
                    static_for<0, 4>([&](auto JJ) {
                        constexpr int j = decltype(JJ)::value;
                        vnext[rt][j] = buf_load_bf16_bits(vbuf, vlane + 2u * (t0 + 16 * rt + j) * dv);
                    });
                });
            }
        };
        const int osz = p.o_bf16 ? 2 : 4;
        const buf_t obuf = buffer_over(reinterpret_cast<const char*>(p.O) + (size_t)bh * T * dv * osz,
                                       (uint32_t)T * dv * osz);
        const size_t sb = (size_t)bh * dv * DK + (size_t)(col0 + n) * DK;
#pragma unroll
        for (int t = 0; t < NK; ++t)
#pragma unroll
            for (int j = 0; j < 4; ++j) Sacc[t][j] = p.S0 ? p.S0[sb + 16 * t + 4 * h + j] : 0.f;
        load_v(0);
        __syncthreads();
        __syncthreads();
        for (int c = 0; c < nchunks; ++c) {
            const int buf = c & 1;
            const int t0 = c * C;
            // ---- phase A: X = K S^T, Z^T = S Q^T ----
            // with VST this chunk's values come from LDS: lane (n, h) reads
            // tokens 16 b + 4 h + j of its column (zero past the end)
            bf16x4 vcur[VST ? NT : 1];
            if constexpr (VST) {
#pragma unroll
                for (int b = 0; b < NT; ++b)
                    vcur[b] = *reinterpret_cast<const bf16x4*>(&s.VT[16 * wave + n][16 * b + 4 * h]);
            }
            f32x4 X[NT], Zt[NT];
#pragma unroll
            for (int rt = 0; rt < NT; ++rt) { X[rt] = zero4(); Zt[rt] = zero4(); }
#pragma unroll
            for (int ss = 0; ss < DK / 32; ++ss) {
                bf16x8 shi, slo;
                split8(Sacc[2 * ss], Sacc[2 * ss + 1], shi, slo);
                bf16x8 kf[NT], qf[NT];
#pragma unroll
                for (int rt = 0; rt < NT; ++rt) {
                    kf[rt] = *reinterpret_cast<const bf16x8*>(&s.K[buf][16 * rt + n][32 * ss + 8 * h]);
                    qf[rt] = *reinterpret_cast<const bf16x8*>(&s.Q[buf][16 * rt + n][32 * ss + 8 * h]);
                }
#pragma unroll
                for (int rt = 0; rt < NT; ++rt) X[rt] = mfma_bf16(kf[rt], shi, X[rt]);
#pragma unroll
                for (int rt = 0; rt < NT; ++rt) Zt[rt] = mfma_bf16(shi, qf[rt], Zt[rt]);
#pragma unroll
                for (int rt = 0; rt < NT; ++rt) X[rt] = mfma_bf16(kf[rt], slo, X[rt]);
#pragma unroll
                for (int rt = 0; rt < NT; ++rt) Zt[rt] = mfma_bf16(slo, qf[rt], Zt[rt]);
            }
            // ---- block forward substitution for V' ----
            // all operands of the substitution are loaded before the chain starts
            bf16x4 bh_[NT][NT], bl_[NT][NT];
#pragma unroll
            for (int b = 0; b < NT; ++b)
#pragma unroll
                for (int cb = 0; cb <= b; ++cb) {
                    bh_[b][cb] = *reinterpret_cast<const bf16x4*>(&s.Bh[buf][L::bidx(b, cb)][n][4 * h]);
                    bl_[b][cb] = *reinterpret_cast<const bf16x4*>(&s.Bl[buf][L::bidx(b, cb)][n][4 * h]);
                }
            // right-hand side factors: (eta, beta exp g) or (beta, exp g)
            // (the lanes of one row group read the same 16 bytes)
            const float* f1b = ETA ? &s.eta[buf][0] : &s.beta[buf][0];
            const float* f2b = ETA ? &s.bge[buf][0] : &s.eg[buf][0];
            f32x4 f1_[NT], f2_[NT];
#pragma unroll
            for (int b = 0; b < NT; ++b) {
                f1_[b] = lds_bcast4(f1b, 16 * b + 4 * h);
                f2_[b] = lds_bcast4(f2b, 16 * b + 4 * h);
            }
            f32x4 Vp[NT];
            bf16x4 vph[NT], vpl[NT];
#pragma unroll
            for (int b = 0; b < NT; ++b) {
                f32x4 y;
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    float vv;
                    if constexpr (VST) vv = (float)vcur[b][j];
                    else vv = bf16_bits_to_float(vnext[b][j]);
                    y[j] = ETA ? f1_[b][j] * vv - f2_[b][j] * X[b][j]
                               : f1_[b][j] * (vv - f2_[b][j] * X[b][j]);
                }
                // The three hi / lo products of a block pair as two k = 32
                // MFMAs: (Bh, Bl) . (vh, vh) with both operands concatenated
                // along k the same way, and (Bh, 0) . (vl, 0).  Every product
                // on one accumulator is the same k = 32 instruction: chaining a
                // 16 x 16 x 16 MFMA onto a 16 x 16 x 32 result gave wrong sums.
                const bf16x4 z4 = {};
                f32x4 rhs = y;
#pragma unroll
                for (int cb = 0; cb < b; ++cb) {
                    rhs = mfma_bf16(cat8(bh_[b][cb], bl_[b][cb]), cat8(vph[cb], vph[cb]), rhs);
                    rhs = mfma_bf16(cat8(bh_[b][cb], z4), cat8(vpl[cb], z4), rhs);
                }
                bf16x4 rh, rl;
                split4(rhs, rh, rl);
                Vp[b] = mfma_bf16(cat8(bh_[b][b], bl_[b][b]), cat8(rh, rh), zero4());
                Vp[b] = mfma_bf16(cat8(bh_[b][b], z4), cat8(rl, z4), Vp[b]);
                split4(Vp[b], vph[b], vpl[b]);
            }
            __syncthreads();
            // the next chunk's values, consumed by the next phase A (past the
            // last chunk every offset is out of range and reads zero)
            load_v(c + 1);
            // ---- phase B: O^T = diag(exp g) Z^T + V'^T P^T (lane: row 16 rt + n, 4 columns) ----
            f32x4 PVt[NT];
#pragma unroll
            for (int rt = 0; rt < NT; ++rt) PVt[rt] = zero4();
#pragma unroll
            for (int ss = 0; ss < C / 32; ++ss) {
                bf16x8 vhi, vlo;
                split8(Vp[2 * ss], Vp[2 * ss + 1], vhi, vlo);
                bf16x8 ph[NT], pl[NT];
#pragma unroll
                for (int rt = 0; rt < NT; ++rt) {
                    if (32 * ss > 16 * rt + 15) continue;   // above the diagonal
                    ph[rt] = ld_perm8(&s.Ph[16 * rt + n][0], ss, h);
                    pl[rt] = ld_perm8(&s.Pl[16 * rt + n][0], ss, h);
                }
#pragma unroll
                for (int rt = 0; rt < NT; ++rt)
                    if (32 * ss <= 16 * rt + 15) PVt[rt] = mfma_bf16(vhi, ph[rt], PVt[rt]);
#pragma unroll
                for (int rt = 0; rt < NT; ++rt)
                    if (32 * ss <= 16 * rt + 15) PVt[rt] = mfma_bf16(vlo, ph[rt], PVt[rt]);
#pragma unroll
                for (int rt = 0; rt < NT; ++rt)
                    if (32 * ss <= 16 * rt + 15) PVt[rt] = mfma_bf16(vhi, pl[rt], PVt[rt]);
            }
            // ---- S^T <- exp(g_last) S^T + K^T diag(exp(g_last - g)) V' ----
            const float gl = s.glast[buf];
#pragma unroll
            for (int t = 0; t < NK; ++t) Sacc[t] *= gl;
            f32x4 Vd[NT];
#pragma unroll
            for (int rt = 0; rt < NT; ++rt)
#pragma unroll
                for (int j = 0; j < 4; ++j) Vd[rt][j] = s.dec[buf][16 * rt + 4 * h + j] * Vp[rt][j];
#pragma unroll
            for (int ss = 0; ss < C / 32; ++ss) {
                bf16x8 vhi, vlo;
                split8(Vd[2 * ss], Vd[2 * ss + 1], vhi, vlo);
                bf16x8 kt[NK];
#pragma unroll
                for (int t = 0; t < NK; ++t) kt[t] = ld_perm8(&s.Kt[buf][16 * t + n][0], ss, h);
#pragma unroll
                for (int t = 0; t < NK; ++t) Sacc[t] = mfma_bf16(kt[t], vhi, Sacc[t]);
#pragma unroll
                for (int t = 0; t < NK; ++t) Sacc[t] = mfma_bf16(kt[t], vlo, Sacc[t]);
            }
            // output rows past the end of the sequence fall outside the buffer (dropped)
            if (p.o_bf16) {
#pragma unroll
                for (int rt = 0; rt < NT; ++rt) {
                    const int r = 16 * rt + n;
                    const f32x4 o = s.eg[buf][r] * Zt[rt] + PVt[rt];
                    buf_store(obuf, (uint32_t)((t0 + r) * dv + col0 + 4 * h) * 2,
                              __builtin_convertvector(o, bf16x4));
                }
            } else if (p.o_wt) {
#pragma unroll
                for (int rt = 0; rt < NT; ++rt) {
                    const int r = 16 * rt + n;
                    const f32x4 o = s.eg[buf][r] * Zt[rt] + PVt[rt];
                    buf_store_wt(obuf, (uint32_t)((t0 + r) * dv + col0 + 4 * h) * 4, o);
                }
            } else {
#pragma unroll
                for (int rt = 0; rt < NT; ++rt) {
                    const int r = 16 * rt + n;
                    const f32x4 o = s.eg[buf][r] * Zt[rt] + PVt[rt];
                    buf_store(obuf, (uint32_t)((t0 + r) * dv + col0 + 4 * h) * 4, o);
                }
            }
            __syncthreads();
        }
#pragma unroll
        for (int t = 0; t < NK; ++t)
#pragma unroll
            for (int j = 0; j < 4; ++j) p.S_final[sb + 16 * t + 4 * h + j] = Sacc[t][j];
    }
}

}  // namespace gdn
