// gdn_fast.h -- fused chunkwise gated delta rule forward pass for bf16
// inputs on gfx950, with fp16 MFMA operands.
//
// Chunk algebra ("从零开始的 GDN 推导": A, then U and W, then the S update and
// the O update; transposed to the d_v x d_k state of "RNN的复兴03", section 4):
//   g_r  = sum_{j<=r} log alpha_j                  (chunk-local, kept in base 2)
//   A_ri = -beta_r exp(g_r - g_i) k_r.k_i (i < r),  T = (I - A)^{-1}
//   V'   = T diag(beta) (V - diag(exp g) K S^T)      (= U - W S^T, W never formed)
//   O    = diag(exp g) Q S^T + P V',   P_ri = exp(g_r - g_i) q_r.k_i (i <= r)
//   S   <- exp(g_last) S + V'^T diag(exp(g_last - g)) K
// with eta (write strength, "RNN的复兴03" section 1) in place of the first
// beta of V' when given.
//
// T is formed whole, off the serial chain: its 16 x 16 diagonal blocks by
// substitution ("RNN的复兴03", section 2.3.1, row by row from T = I + T A), and
// the blocks below the diagonal by block substitution
//     T_bc = T_bb sum_{c<=k<b} A_bk T_kc
// on MFMA.  The serial chain over chunks then holds three dense products per
// chunk: X = K S^T, V' = T Y and the state update, each one MFMA per tile.
//
// Precision: every MFMA operand is fp16 (11 significant bits) with fp32
// accumulation and an fp32 state.  q, k, v arrive as bf16 and convert to
// fp16 exactly while |x| lies in [2^-14, 65504]; derived operands (the
// state, T, the pseudo-values, the scores) are rounded to fp16 once per
// product.  Operand magnitudes must stay below 65504 (the fp16 range).
//
// Work is split by role inside the workgroup.  NS "scan" waves own 16 value
// columns each and that slice of the fp32 state (S^T in MFMA accumulators);
// six "prep" waves beside one or two scan waves, five beside three, four
// beside four (the roles below are spread over them by FastRoles), build
// chunk-local matrices one or two chunks ahead.  Iteration i (chunk i on
// the scan waves) has two phases separated by workgroup barriers:
//   phase A  scan     X_i = K_i S^T, Z^T_i = S Q_i^T
//            T blocks blocks of T_i below the diagonal (T_bb of chunk i and
//                     its A blocks are from iteration i - 1)
//            strips   row strips of chunk i + 1: Gram and score tiles formed
//                     into the diagonal blocks of A (fp32), the blocks below
//                     them (fp16) and the masked decayed scores P (fp16)
//            values   (up to three scan waves) the values of chunk i + 1
//                     into LDS, on the solve wave
//   phase B  scan     Y, V' = T_i Y, state update, O = diag(exp g) Z + P V'
//            vectors  decay vectors of chunk i + 2
//            solve    diagonal blocks T_bb of chunk i + 1
//            staging  keys and queries of chunk i + 2 into LDS (fp16)
// The loop starts at i = -2 so that the first two iterations only prepare.
// The state update reads K^T straight from the token-major key tile with
// the LDS transposing read, so the keys stay three chunks deep (chunk i for
// the scan, i + 1 for the strips, i + 2 being staged).
#pragma once
#include <type_traits>

#include "gdn_device.h"
#include "gdn_kernels.h"
#include "gdn_pipe.h"

namespace gdn {

typedef __attribute__((ext_vector_type(8))) _Float16 h8;
typedef __attribute__((ext_vector_type(4))) _Float16 h4;
typedef __attribute__((ext_vector_type(2))) _Float16 h2;
typedef __attribute__((ext_vector_type(2))) float f2;

__device__ __forceinline__ f32x4 mfma_h(h8 a, h8 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ h8 cat_h(h4 a, h4 b) {
    return __builtin_shufflevector(a, b, 0, 1, 2, 3, 4, 5, 6, 7);
}
__device__ __forceinline__ h4 to_h4(f32x4 x) { return __builtin_convertvector(x, h4); }
__device__ __forceinline__ h4 zero_h4() { return h4{0, 0, 0, 0}; }

typedef __attribute__((ext_vector_type(4))) short s4;
typedef __attribute__((address_space(3))) const _Float16 lds_h;
// An LDS address held in one register that the compiler may not split into
// a base and a constant: reads at constant offsets from it then use the
// instructions' 16-bit immediate offset, instead of one address register per
// offset once the array lies beyond the immediate's reach.
__device__ __forceinline__ lds_h* lds_opaque(const _Float16* p) {
    lds_h* q = (lds_h*)p;
    asm volatile("" : "+v"(q));
    return q;
}
template <typename V>
__device__ __forceinline__ V lds_at(lds_h* p, int off) {
    return *reinterpret_cast<__attribute__((address_space(3))) const V*>(p + off);
}
// ds_read_b64_tr_b16: each lane addresses four consecutive 16-bit elements;
// within each group of 16 lanes g, lane 16 g + i receives element i % 4 of
// the four that lanes 16 g + 4 e + i / 4 (e = 0..3) addressed, in e order.
__device__ __forceinline__ h4 lds_read_tr(lds_h* p) {
    return __builtin_bit_cast(h4, __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                                      (__attribute__((address_space(3))) s4*)p));
}

// Two bf16 (one 32-bit word) to two fp16.
__device__ __forceinline__ unsigned bf2_to_h2(unsigned w) {
    const f2 f = {__builtin_bit_cast(float, w << 16), __builtin_bit_cast(float, w & 0xffff0000u)};
    return __builtin_bit_cast(unsigned, __builtin_convertvector(f, h2));
}

template <int C, int DK, int NS, bool ETA>
struct alignas(16) FastLds {
    static constexpr int NT = C / 16;                 // 16-token blocks per chunk
    static constexpr int NB = NT * (NT + 1) / 2;      // blocks on and below the diagonal
    static constexpr int NOFF = NT * (NT - 1) / 2;    // blocks below the diagonal
    // Strides chosen against the LDS banks (reads see 64 banks of 4 bytes,
    // 16-byte reads served eight lanes from each half-wave at a time; writes
    // see 32 banks, consecutive lanes together):
    //   key / query rows DK + 16: the 16-byte operand reads of 8 rows by 2
    //     lane groups cover all banks once, and the transposing reads of the
    //     state update meet at most two to a bank;
    //   16 x 16 blocks at row stride 20: conflict-free fp16 row writes;
    //   the fp32 diagonal blocks of A get 4 floats between blocks, so the
    //     solve's broadcast row reads of four blocks fall in distinct banks.
    static constexpr int KP = DK + 16;                // key / query row stride (fp16)
    static constexpr int BP = 20;                     // row stride of 16 x 16 blocks
    static constexpr int ADS = 16 * BP + 4;           // fp32 diagonal-block stride
    static constexpr int bidx(int b, int c) { return b * (b + 1) / 2 + c; }
    static constexpr int oidx(int b, int c) { return b * (b - 1) / 2 + c; }
    // Small arrays first: the scan reads them at fixed offsets that the LDS
    // instructions' 16-bit immediate reaches from one lane base.
    // per-token vectors, three chunks live at a time
    float g2[3][C];    // inclusive cumsum of log2 alpha
    float er[3][C];    // 2^(g2_r - g2_ref): row factor of exp(g_r - g_i)
    float fi[3][C];    // 2^(g2_ref - g2_i): column factor
    float eg[3][C];    // exp(g)
    float dec[3][C];   // exp(g_last - g)
    float beta[3][C];
    float eta[ETA ? 3 : 1][ETA ? C : 4];   // write strength
    float bge[ETA ? 3 : 1][ETA ? C : 4];   // beta exp(g)
    float glast[4];    // exp(g_last)
    int sep[4];        // row x column factors safe in fp32 for this chunk
    _Float16 Tb[2][NB][16][BP];                // T = (I - A)^{-1}, blocks (b, c <= b)
    _Float16 Pb[2][NB][16][BP];                // masked decayed scores, blocks (b, c <= b)
    _Float16 Ao[2][NOFF > 0 ? NOFF : 1][16][BP];   // A below the diagonal blocks
    float Ad[2][NT][ADS];                      // diagonal blocks of A (fp32, for the solve), rows BP apart
    // keys by chunk modulo 3, queries by chunk parity; each 32-element block
    // of a row in the scan's k-order (elements 4h..4h+3 then 16+4h..16+4h+3,
    // h = 0..3), so an MFMA operand slice is one aligned 16-byte read
    _Float16 K[3][C][KP];
    _Float16 Q[2][C][KP];
    // with up to three scan waves, the values of the scan's chunks as raw
    // bf16 by chunk parity (staged by a prep wave), row = token, 16-byte
    // vector u = value columns 8u..8u+7 of the workgroup's tile.  Row stride
    // VS = 2 x odd vectors: a scan wave's 16-byte reads of eight rows by two
    // halves then fall on 16 distinct 16-byte bank groups.
    static constexpr bool VST = fast_prep_waves(NS, C, DK) != 4;
    static constexpr int VU = 2 * NS;                 // 16-byte vectors per row
    static constexpr int VS = NS == 1 ? 2 : NS == 4 ? 10 : 6;   // row stride (16-byte vectors)
    uint4 Vs[VST ? 2 : 1][VST ? C : 1][VS];
};


// Roles of the prep waves.  The waves of a workgroup are spread over the
// four SIMDs of the compute unit so that waves w and w + 4 share one; the
// roles are placed so that the prep waves beside the scan waves (prep waves
// 2 and 3 when there are six, 1, 2 and 3 when there are five) carry the
// latency-bound, issue-light jobs (the blocks of T below the diagonal, the
// decay vectors, the diagonal solves, the value staging) and the
// issue-heavy ones (Gram strips, staging) sit together on the other SIMDs.
// With five, the SIMD that has no scan wave carries two strip waves of 24
// tile products each, and the prep waves beside scan waves 1 and 2 one of
// 16 each.
//   strips: row strip rt holds the tiles (rt, ct), ct = 0..rt, of both A and
//           the scores P;
//   stagers: convert and store the keys and queries of a chunk.
template <int NS, int NT, int DK>
struct FastRoles {
    static constexpr int NP = fast_prep_waves(NS, 16 * NT, DK);
    // six prep waves beside four scan waves: every SIMD holds a scan wave;
    // prep waves 0 to 3 (one per SIMD) stage the keys and queries, 2 and 3
    // also form the Gram strips, and 4 and 5 (on the SIMDs of scan waves 0
    // and 1) carry the blocks of T with the decay vectors, and the diagonal
    // solves with the value staging
    static constexpr bool WIDE = NP == 6 && NS == 4;
    static constexpr int NSTG = NP == 6 ? 4 : 3;
    static constexpr int toff_wave = WIDE ? 4 : NP == 6 ? 2 : NP == 5 ? 1 : 0;
    static constexpr int vec_wave = WIDE ? 4 : NP == 6 ? 2 : NP == 5 ? 1 : 0;
    static constexpr int solve_wave = WIDE ? 5 : NP == 6 ? 3 : NP == 5 ? 2 : 0;
    static constexpr int stager(int pw) {
        if (WIDE) return pw < 4 ? pw : -1;
        if (NP == 6) return pw == 0 ? 0 : pw == 1 ? 1 : pw == 4 ? 2 : pw == 5 ? 3 : -1;
        if (NP == 5) return pw == 0 ? 0 : pw == 3 ? 1 : pw == 4 ? 2 : -1;
        return pw >= 1 ? pw - 1 : -1;
    }
    // Gram segments: (row strip rt, tile columns c0 <= ct < c1), encoded
    // (rt << 16) | (c0 << 8) | c1, at most two per wave.  With six prep
    // waves and four strips the 80 tile products split 24 / 16 / 16 / 24 so
    // that the two SIMDs of the issue-heavy waves carry 40 each.
    static constexpr int seg_code(int rt, int c0, int c1) { return (rt << 16) | (c0 << 8) | c1; }
    static constexpr int seg(int w, int j) {
        if (WIDE) {   // (chunks of at most 32 tokens)
            if (NT == 2) {
                if (w == 2) return j == 0 ? seg_code(1, 0, 2) : -1;
                if (w == 3) return j == 0 ? seg_code(0, 0, 1) : -1;
                return -1;
            }
            return (w == 2 && j == 0) ? seg_code(0, 0, 1) : -1;
        }
        if (NP == 6) {
            if (NT == 4) {
                if (w == 0) return j == 0 ? seg_code(3, 0, 2) : j == 1 ? seg_code(0, 0, 1) : -1;
                if (w == 1) return j == 0 ? seg_code(3, 2, 4) : -1;
                if (w == 4) return j == 0 ? seg_code(1, 0, 2) : -1;
                if (w == 5) return j == 0 ? seg_code(2, 0, 3) : -1;
                return -1;
            }
            if (NT == 2) {
                if (w == 0) return j == 0 ? seg_code(1, 0, 2) : -1;
                if (w == 1) return j == 0 ? seg_code(0, 0, 1) : -1;
                return -1;
            }
            return (w == 0 && j == 0) ? seg_code(0, 0, 1) : -1;
        }
        if (NP == 5) {
            if (NT == 4) {
                if (w == 0) return j == 0 ? seg_code(3, 0, 2) : j == 1 ? seg_code(0, 0, 1) : -1;
                if (w == 2) return j == 0 ? seg_code(1, 0, 2) : -1;
                if (w == 3) return j == 0 ? seg_code(3, 2, 4) : -1;
                if (w == 4) return j == 0 ? seg_code(2, 0, 3) : -1;
                return -1;
            }
            if (NT == 2) {
                if (w == 0) return j == 0 ? seg_code(1, 0, 2) : -1;
                if (w == 4) return j == 0 ? seg_code(0, 0, 1) : -1;
                return -1;
            }
            return (w == 0 && j == 0) ? seg_code(0, 0, 1) : -1;
        }
        if (NT == 4) {
            if (w == 1) return j == 0 ? seg_code(3, 0, 4) : -1;
            if (w == 2) return j == 0 ? seg_code(2, 0, 3) : -1;
            if (w == 3) return j == 0 ? seg_code(1, 0, 2) : j == 1 ? seg_code(0, 0, 1) : -1;
            return -1;
        }
        if (NT == 2) {
            if (w == 1) return j == 0 ? seg_code(1, 0, 2) : -1;
            if (w == 2) return j == 0 ? seg_code(0, 0, 1) : -1;
            return -1;
        }
        return (w == 1 && j == 0) ? seg_code(0, 0, 1) : -1;
    }
    static constexpr int nseg(int w) { return seg(w, 0) < 0 ? 0 : seg(w, 1) < 0 ? 1 : 2; }
};

// SEG: the sequence-parallel launch (segments, transition tiles); without
// it every segment-related quantity folds to the plain form at compile time.
// DKG: the d_k of the tensors in memory when it is smaller than the
// kernel's (d_k 16 runs as 32: the MFMAs take 32 elements per k-step): the
// keys and queries are padded with zeros as they are staged and the state's
// extra rows stay zero, so the products are those of d_k = DKG.
template <int C, int DK, int NS, bool ETA, bool SEG, int DKG = DK>
__global__ __launch_bounds__((NS + fast_prep_waves(NS, C, DK)) * 64) void gdn_fwd_fast_kernel(FwdParams p) {
    using R = FastRoles<NS, C / 16, DK>;
    constexpr int NP = R::NP;
    using L = FastLds<C, DK, NS, ETA>;
    constexpr int NT = C / 16;
    constexpr int NK = DK / 16;              // 16-row tiles of S^T
    constexpr int NSS = DK / 32;             // k-steps over d_k
    constexpr int NTS = (C + 31) / 32;       // k-steps over the tokens of a chunk
    constexpr int DVT = 16 * NS;
    constexpr int KV = C * DK / 8;           // 16-byte vectors in a key tile
    constexpr int NSTG = R::NSTG;
    constexpr int NKV = (KV + 64 * NSTG - 1) / (64 * NSTG);
    constexpr int BP_ = L::BP;
    static_assert(DK % 32 == 0 && C % 16 == 0, "shape");
    static_assert(sizeof(L) <= 160 * 1024, "LDS budget");
    static_assert(!L::VST || L::VU <= L::VS, "value tile row");
    static_assert(!R::WIDE || NT <= 2, "six prep waves beside four scan waves: chunks of at most 32");
    __shared__ L s;

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int n = lane & 15;
    const int h = lane >> 4;
    const bool scan = wave < NS;
    const int pw = wave - NS;
    // staging lane 0..64*NSTG-1 on the stager waves
    const int plane = (pw >= 0 ? R::stager(pw) : 0) * 64 + lane;

    // unit = (head, segment); the tiles of one unit share its keys and queries
    int tile, unit;
    if (p.xcd_groups) {
        const int xcd = blockIdx.x & 7, slot = blockIdx.x >> 3;
        tile = slot % p.n_tiles;
        unit = xcd + 8 * (slot / p.n_tiles);
    } else {
        tile = blockIdx.x % p.n_tiles;
        unit = blockIdx.x / p.n_tiles;
    }
    const int nseg = SEG ? p.nseg : 1;
    // padding workgroups of an XCD-grouped grid (units rounded up to a
    // multiple of 8) have none: they leave before any barrier, and so do the
    // transition tiles of a first segment (it starts from the true state)
    if (unit >= p.B * p.H * nseg) return;
    const int bh = SEG ? unit / nseg : unit, seg = SEG ? unit - bh * nseg : 0;
    const bool trans = SEG && tile >= p.n_tiles_v;
    if (trans && seg == 0) return;
    // this segment's tokens: T from token tbase of the sequence
    const int tbase = SEG ? seg * p.seg_len : 0;
    const int T = SEG ? min(p.T - tbase, p.seg_len) : p.T, dv = p.dv;
    const size_t tok0 = (size_t)bh * p.T + tbase;
    const int nchunks = (T + C - 1) / C;
    static_assert(DKG == DK || (DKG == 16 && DK == 32 && !SEG), "padded d_k");
    const __bf16* kb = reinterpret_cast<const __bf16*>(p.k) + tok0 * DKG;
    const __bf16* qb = reinterpret_cast<const __bf16*>(p.q) + tok0 * DKG;
    const __bf16* vb = reinterpret_cast<const __bf16*>(p.v) + tok0 * dv;
    const float* ab = p.alpha ? p.alpha + tok0 : nullptr;
    const float* bb = p.beta + tok0;
    const float* eb = p.eta ? p.eta + tok0 : nullptr;
    const buf_t kbuf = buffer_over(kb, (uint32_t)T * DKG * 2);
    const buf_t qbuf = buffer_over(qb, (uint32_t)T * DKG * 2);
    // scan waves: first value column (transition tiles: first transition row)
    const int col0 = (trans ? tile - p.n_tiles_v : tile) * DVT + 16 * wave;

    auto mod3 = [](int x) { return (x + 3) % 3; };   // x >= -3

    if (!scan) {
        // ============================== prep ===============================
        // raw bf16 key / query tiles of the next chunk to stage: loaded an
        // iteration ahead, converted into LDS, then reloaded with the next
        uint4 stK[NKV], stQ[NKV];
        float stA = 1.f, stB = 0.f, stE = 0.f;  // vector wave: gates of the next chunk to prepare

        // stagers: global loads of chunk cc's keys and queries (rows past the
        // end of the sequence read as zero).  Staging vector vi is the 16-byte
        // k-order slice u = vi % (DK / 8) of row vi / (DK / 8): d_k
        // 32 (u / 4) + 4 (u % 4) .. + 3 and the four 16 further on, fetched as
        // two 8-byte pieces so that no lane exchange is needed.
        auto kq_load = [&](int cc) __attribute__((always_inline)) {
            const int t0 = cc * C;
            static_for<0, NKV>([&](auto I) {
                constexpr int i = decltype(I)::value;
                const int vi = plane + i * 64 * NSTG;
                if (i + 1 < NKV || vi < KV) {
                    const int r = vi / (DK / 8), u = vi % (DK / 8);
                    const uint32_t off = 2u * ((t0 + r) * DKG + 32 * (u >> 2) + 4 * (u & 3));
                    const uint2 k0 = buf_load_8B(kbuf, off), q0 = buf_load_8B(qbuf, off);
                    // (d_k 16 padded to 32: the second pieces are the zero padding)
                    const uint2 k1 = DKG == DK ? buf_load_8B(kbuf, off + 32) : make_uint2(0, 0);
                    const uint2 q1 = DKG == DK ? buf_load_8B(qbuf, off + 32) : make_uint2(0, 0);
                    stK[i] = make_uint4(k0.x, k0.y, k1.x, k1.y);
                    stQ[i] = make_uint4(q0.x, q0.y, q1.x, q1.y);
                }
            });
        };
        // stagers: chunk cc's keys and queries into LDS as fp16, one k-order
        // slice per staging vector
        auto kq_store = [&](int cc) __attribute__((always_inline)) {
            const int buf = cc & 1, kb3 = mod3(cc);
            auto slice = [&](const uint4 v) __attribute__((always_inline)) {
                return make_uint4(bf2_to_h2(v.x), bf2_to_h2(v.y), bf2_to_h2(v.z), bf2_to_h2(v.w));
            };
            static_for<0, NKV>([&](auto I) {
                constexpr int i = decltype(I)::value;
                const int vi = plane + i * 64 * NSTG;
                if (i + 1 < NKV || vi < KV) {
                    const int r = vi / (DK / 8), u = vi % (DK / 8);
                    *reinterpret_cast<uint4*>(&s.K[kb3][r][8 * u]) = slice(stK[i]);
                    *reinterpret_cast<uint4*>(&s.Q[buf][r][8 * u]) = slice(stQ[i]);
                }
            });
        };
        // solve wave (up to three scan waves): the value tile of chunk cc (rows
        // past the end of the sequence read as zero, and so does every row of
        // a transition tile), loaded an iteration ahead and stored raw into
        // LDS in phase A, where this wave is otherwise idle, so that the scan
        // waves issue no global loads of their own (theirs would also wait for
        // their earlier output stores: loads and stores share one counter)
        constexpr int VU = L::VU;
        constexpr int NVV = (C * VU + 63) / 64;
        uint4 stV[NVV];
        const buf_t vsbuf = buffer_over(vb, trans ? 0u : (uint32_t)T * dv * 2);
        const uint32_t vcol = (uint32_t)((trans ? tile - p.n_tiles_v : tile) * DVT);
        auto val_load = [&](int cc) __attribute__((always_inline)) {
            const uint32_t t0 = (uint32_t)cc * C;
            static_for<0, NVV>([&](auto I) {
                constexpr int i = decltype(I)::value;
                const int vi = lane + 64 * i;
                if (i + 1 < NVV || vi < C * VU) {
                    const uint32_t r = vi / VU, u = vi % VU;
                    stV[i] = buf_load_16B(vsbuf, 2u * ((t0 + r) * dv + vcol + 8 * u));
                }
            });
        };
        auto val_store = [&](int cc) __attribute__((always_inline)) {
            static_for<0, NVV>([&](auto I) {
                constexpr int i = decltype(I)::value;
                const int vi = lane + 64 * i;
                if (i + 1 < NVV || vi < C * VU) s.Vs[cc & 1][vi / VU][vi % VU] = stV[i];
            });
        };
        // vector wave: gates of chunk cc (lane t holds token t of the chunk)
        auto gate_load = [&](int cc) __attribute__((always_inline)) {
            const int t0 = cc * C, Lc = min(C, T - t0);
            const int tt = t0 + min(lane, Lc - 1);
            stA = ab ? ab[tt] : 1.f;
            stB = bb[tt];
            if constexpr (ETA) stE = eb[tt];
        };
        // vector wave: decay vectors of chunk cc into vector buffer mod3(cc);
        // padding tokens are identity transitions (alpha = 1, beta = eta = 0)
        auto vectors = [&](int cc) __attribute__((always_inline)) {
            const int vb3 = mod3(cc);
            const int Lc = min(C, T - cc * C);
            const float a = lane < Lc ? stA : 1.f;
            const float l2 = (lane < C) ? __builtin_amdgcn_logf(a) : 0.f;
            const float g = wave_inclusive_scan(l2, lane);
            const float gl = lane_value(g, C - 1);
            // exp(g_r - g_i) = 2^(g2_r - ref) 2^(ref - g2_i), ref the middle of
            // the chunk, when the chunk's decay range keeps both factors far
            // inside fp32; otherwise each ratio is exponentiated on its own
            const float ref = lane_value(g, C / 2);
            const float g0 = lane_value(g, 0);
            if (lane < C) {
                const float bt = lane < Lc ? stB : 0.f;
                s.g2[vb3][lane] = g;
                s.eg[vb3][lane] = __builtin_amdgcn_exp2f(g);
                s.dec[vb3][lane] = __builtin_amdgcn_exp2f(gl - g);
                s.beta[vb3][lane] = bt;
                if constexpr (ETA) {
                    s.eta[vb3][lane] = lane < Lc ? stE : 0.f;
                    s.bge[vb3][lane] = bt * __builtin_amdgcn_exp2f(g);
                }
                s.er[vb3][lane] = __builtin_amdgcn_exp2f(g - ref);
                s.fi[vb3][lane] = __builtin_amdgcn_exp2f(ref - g);
            }
            if (lane == 0) {
                s.glast[vb3] = __builtin_amdgcn_exp2f(gl);
                s.sep[vb3] = (g0 - gl) <= 96.f;
            }
        };
        // Gram segments of chunk cc owned by this wave.  Segment (rt, c0, c1):
        // key block rt (B operand of A's tiles), query block rt (B operand of
        // the scores) and each key block ct in [c0, c1) (A operand of both)
        // are read from LDS once; then the tiles are formed,
        //   A_ri = -beta_r exp(g_r - g_i) k_r.k_i (i < r),  P_ri = exp(g_r - g_i) q_r.k_i (i <= r),
        // with lane (n, h) holding row r = 16 rt + n, columns 16 ct + 4 h + e.
        auto strips = [&](auto W, int cc) __attribute__((always_inline)) {
            constexpr int w = decltype(W)::value;
            const int buf = cc & 1;
            const int vb3 = mod3(cc);
            const bool sep = s.sep[vb3];
            static_for<0, R::nseg(w)>([&](auto JJ) {
                constexpr int code = R::seg(w, decltype(JJ)::value);
                constexpr int rt = code >> 16, c0 = (code >> 8) & 255, c1 = code & 255;
                const int r = 16 * rt + n;
                h8 kb[NSS], qb[NSS];
#pragma unroll
                for (int ss = 0; ss < NSS; ++ss) {
                    kb[ss] = *reinterpret_cast<const h8*>(&s.K[vb3][r][32 * ss + 8 * h]);
                    qb[ss] = *reinterpret_cast<const h8*>(&s.Q[buf][r][32 * ss + 8 * h]);
                }
                const float nbr = -s.beta[vb3][r];
                const float g2r = s.g2[vb3][r];
                const float err = s.er[vb3][r];
                // every product of the strip before any store: LDS stores
                // would keep the compiler from hoisting the next tile's loads
                f32x4 ga[NT], gp[NT];
                static_for<c0, c1>([&](auto CC) {
                    constexpr int ct = decltype(CC)::value;
                    h8 ka[NSS];
#pragma unroll
                    for (int ss = 0; ss < NSS; ++ss) {
                        if constexpr (ct == rt) ka[ss] = kb[ss];
                        else ka[ss] = *reinterpret_cast<const h8*>(&s.K[vb3][16 * ct + n][32 * ss + 8 * h]);
                    }
                    ga[ct] = zero4();
                    gp[ct] = zero4();
#pragma unroll
                    for (int ss = 0; ss < NSS; ++ss) {
                        ga[ct] = mfma_h(ka[ss], kb[ss], ga[ct]);
                        gp[ct] = mfma_h(ka[ss], qb[ss], gp[ct]);
                    }
                });
                f32x4 fic[NT], g2c[NT];
                static_for<c0, c1>([&](auto CC) {
                    constexpr int ct = decltype(CC)::value;
                    fic[ct] = *reinterpret_cast<const f32x4*>(&s.fi[vb3][16 * ct + 4 * h]);
                    g2c[ct] = *reinterpret_cast<const f32x4*>(&s.g2[vb3][16 * ct + 4 * h]);
                });
                static_for<c0, c1>([&](auto CC) {
                    constexpr int ct = decltype(CC)::value;
                    const int i0 = 16 * ct + 4 * h;
                    f32x4 d;
                    if (sep) {
                        d = err * fic[ct];
                    } else {
#pragma unroll
                        for (int e = 0; e < 4; ++e) d[e] = __builtin_amdgcn_exp2f(g2r - g2c[ct][e]);
                    }
                    f32x4 va, vp;
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        va[e] = (ct < rt || i0 + e < r) ? nbr * d[e] * ga[ct][e] : 0.f;
                        vp[e] = (ct < rt || i0 + e <= r) ? d[e] * gp[ct][e] : 0.f;
                    }
                    *reinterpret_cast<h4*>(&s.Pb[buf][L::bidx(rt, ct)][n][4 * h]) = to_h4(vp);
                    if constexpr (ct == rt)
                        *reinterpret_cast<f32x4*>(&s.Ad[buf][rt][n * BP_ + 4 * h]) = va;
                    else
                        *reinterpret_cast<h4*>(&s.Ao[buf][L::oidx(rt, ct)][n][4 * h]) = to_h4(va);
                });
            });
        };
        // solve wave: T_bb = (I - A_bb)^{-1} for all diagonal blocks of chunk cc:
        // lane (b, i) computes row i of T_bb from T = I + T A by substitution
        // from the last column down,  T[i][k] = [i == k] + sum_{m > k} T[i][m] A[m][k],
        // adding each final T[i][m] into every earlier column's partial sum.
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
                        abuf[m % 3][q] = *reinterpret_cast<const f32x4*>(&s.Ad[buf][b][m * BP_ + 4 * q]);
                };
                load_row(std::integral_constant<int, 15>{});
                load_row(std::integral_constant<int, 14>{});
                static_for<0, 16>([&](auto JJ) {
                    constexpr int m = 15 - decltype(JJ)::value;
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
                _Float16* trow = &s.Tb[buf][L::bidx(b, b)][i][0];
#pragma unroll
                for (int q = 0; q < 4; ++q)
                    *reinterpret_cast<h4*>(trow + 4 * q) =
                        to_h4(f32x4{x[4 * q], x[4 * q + 1], x[4 * q + 2], x[4 * q + 3]});
            }
        };
        // T-blocks wave: the blocks of T below the diagonal of chunk cc, by distance
        // from the diagonal:  T_bc = T_bb R,  R = sum_{c<=k<b} A_bk T_kc.
        // Lane (n, h) holds T_bc[4h + j][n] (accumulator layout), which is
        // also the B-operand layout of the next products.
        auto t_off = [&](int cc) __attribute__((always_inline)) {
            if constexpr (NT > 1) {
                const int buf = cc & 1;
                // all operands first (LDS stores below would keep later loads
                // from being hoisted): the A blocks below the diagonal, the
                // rows of each T_bb (A operand) and the columns of each T_cc
                // (B operand, lane (n, h): rows 4h..4h+3 of column n)
                h4 Ab[NT][NT], Trow[NT], Tcol[NT];
                static_for<1, NT>([&](auto BB) {
                    constexpr int b = decltype(BB)::value;
                    static_for<0, b>([&](auto KK) {
                        constexpr int k = decltype(KK)::value;
                        Ab[b][k] = *reinterpret_cast<const h4*>(&s.Ao[buf][L::oidx(b, k)][n][4 * h]);
                    });
                    Trow[b] = *reinterpret_cast<const h4*>(&s.Tb[buf][L::bidx(b, b)][n][4 * h]);
                });
                static_for<0, NT - 1>([&](auto CC) {
                    constexpr int c = decltype(CC)::value;
#pragma unroll
                    for (int j = 0; j < 4; ++j) Tcol[c][j] = s.Tb[buf][L::bidx(c, c)][4 * h + j][n];
                });
                h4 Tr[NT][NT];
                static_for<1, NT>([&](auto DD) {
                    constexpr int d = decltype(DD)::value;
                    static_for<0, NT - d>([&](auto CC) {
                        constexpr int c = decltype(CC)::value;
                        constexpr int b = c + d;
                        f32x4 R = zero4();
                        static_for<0, (d + 1) / 2>([&](auto KK) {
                            constexpr int k = c + 2 * decltype(KK)::value;
                            h4 t0;
                            if constexpr (k == c) t0 = Tcol[c];
                            else t0 = Tr[k][c];
                            h4 a1 = zero_h4(), t1 = zero_h4();
                            if constexpr (k + 1 < b) {
                                a1 = Ab[b][k + 1];
                                t1 = Tr[k + 1][c];
                            }
                            R = mfma_h(cat_h(Ab[b][k], a1), cat_h(t0, t1), R);
                        });
                        const f32x4 tbc = mfma_h(cat_h(Trow[b], zero_h4()), cat_h(to_h4(R), zero_h4()), zero4());
                        Tr[b][c] = to_h4(tbc);
                    });
                });
                static_for<1, NT>([&](auto BB) {
                    constexpr int b = decltype(BB)::value;
                    static_for<0, b>([&](auto CC) {
                        constexpr int c = decltype(CC)::value;
#pragma unroll
                        for (int j = 0; j < 4; ++j) s.Tb[buf][L::bidx(b, c)][4 * h + j][n] = Tr[b][c][j];
                    });
                });
            }
        };
        // stage-parity output: T of chunk cc as fp32 [C][C] (upper part zero)
        auto dbg_t = [&](int cc) __attribute__((always_inline)) {
            {
                {
                    const int buf = cc & 1;
                    float* dst = p.dbg_T + ((size_t)bh * nchunks + cc) * C * C;
                    for (int e = lane; e < C * C; e += 64) {
                        const int r = e / C, c = e % C;
                        const int b = r / 16, cb = c / 16;
                        dst[e] = cb <= b ? (float)s.Tb[buf][L::bidx(b, cb)][r % 16][c % 16] : 0.f;
                    }
                }
            }
        };

        auto prep_role = [&](auto W) __attribute__((always_inline)) {
            constexpr int w = decltype(W)::value;
            constexpr bool stg = R::stager(w) >= 0;
            auto step = [&](auto PAR, int i) __attribute__((always_inline)) {
                // ---- phase A ----
                if constexpr (L::VST && w == R::solve_wave) {
                    // the scan reads chunk i's values from the other buffer
                    if (i + 1 >= 0 && i + 1 < nchunks) {
                        val_store(i + 1);
                        if (i + 2 < nchunks) val_load(i + 2);
                    }
                }
                if constexpr (w == R::toff_wave) {
                    if (i >= 0) {
                        t_off(i);
                        if (p.dbg_T) {
                            wave_lds_sync();
                            dbg_t(i);
                        }
                    }
                }
                if constexpr (R::nseg(w) > 0) {
                    if (i + 1 >= 0 && i + 1 < nchunks) strips(W, i + 1);
                }
                __syncthreads();
                // ---- phase B ----
                if constexpr (w == R::vec_wave) {
                    if (i + 2 < nchunks) {
                        vectors(i + 2);
                        if (i + 3 < nchunks) gate_load(i + 3);
                    }
                }
                if constexpr (w == R::solve_wave) {
                    if (i + 1 >= 0 && i + 1 < nchunks) diag_solve(i + 1);
                }
                if constexpr (stg) {
                    if (i + 2 < nchunks) {
                        kq_store(i + 2);
                        if (i + 3 < nchunks) kq_load(i + 3);
                    }
                }
                __syncthreads();
            };
            if constexpr (w == R::vec_wave) gate_load(0);
            if constexpr (L::VST && w == R::solve_wave) val_load(0);
            if constexpr (stg) kq_load(0);
            for (int i = -2; i < nchunks; i += 2) {
                step(std::integral_constant<int, 0>{}, i);
                if (i + 1 < nchunks) step(std::integral_constant<int, 1>{}, i + 1);
            }
        };
        switch (pw) {
            case 0: prep_role(std::integral_constant<int, 0>{}); break;
            case 1: prep_role(std::integral_constant<int, 1>{}); break;
            case 2: prep_role(std::integral_constant<int, 2>{}); break;
            case 3: prep_role(std::integral_constant<int, 3>{}); break;
            case 4: if constexpr (NP > 4) prep_role(std::integral_constant<int, 4>{}); break;
            default: if constexpr (NP > 5) prep_role(std::integral_constant<int, 5>{}); break;
        }
    } else {
        // ============================== scan ===============================
        f32x4 Sacc[NK];            // Sacc[t][j] = S[col0 + n][16 t + 4 h + j]
        // value rows of a chunk, A operand of the transposing MFMA: lane
        // (n, h) holds V[16 rt + n][col0 + 8 (h & 1) .. + 7] (lanes h >= 2
        // repeat lanes h - 2; the selector gives them weight zero).  With
        // up to three scan waves they are read from the tile a prep wave
        // staged in LDS; with four (no prep wave to spare) each scan wave
        // loads its own a chunk ahead, transition tiles from an empty buffer
        // that reads zero.
        uint4 vraw[NT];
        const buf_t vbuf = buffer_over(vb, trans || L::VST ? 0u : (uint32_t)T * dv * 2);
        const uint32_t voff = 2u * (n * dv + col0 + 8 * (h & 1));
        auto v_load = [&](int cc) __attribute__((always_inline)) {
            const uint32_t t0 = (uint32_t)cc * C;
#pragma unroll
            for (int rt = 0; rt < NT; ++rt) vraw[rt] = buf_load_16B(vbuf, voff + 2u * (t0 + 16 * rt) * dv);
        };
        // selector picking value column n of the 16 (lane (n, h), k-slots 8h..8h+7)
        bf16x8 vsel;
#pragma unroll
        for (int e = 0; e < 8; ++e) vsel[e] = (__bf16)((h < 2 && 8 * h + e == n) ? 1.f : 0.f);

        // outputs: O (fp32 or bf16, row stride d_v); for a later segment with
        // bf16 O, fp32 partial outputs into seg_o; for transition tiles the
        // transformed queries into seg_q (fp32, row stride d_k)
        const void* obase;
        int ostr = dv;
        bool obf = false;
        if (trans) {
            obase = p.seg_q + tok0 * DK;
            ostr = DK;
        } else if (seg > 0 && p.seg_o) {
            obase = p.seg_o + tok0 * dv;
        } else {
            obf = p.o_bf16;
            obase = reinterpret_cast<const char*>(p.O) + tok0 * dv * (obf ? 2 : 4);
        }
        const buf_t obuf = buffer_over(obase, (uint32_t)T * ostr * (obf ? 2 : 4));
        // initial state: S0 rows (first segment), zero (later segments) or
        // identity rows (transition tiles); end state: S_final, or this
        // segment's rows of seg_state (transition rows stored transposed,
        // element (row, k) at k * d_k + row)
        const size_t sb = (size_t)bh * dv * DKG + (size_t)(col0 + n) * DKG;
        const float* s0p = (seg == 0 && p.S0) ? p.S0 + sb : nullptr;
        const size_t seg_base = ((size_t)bh * nseg + seg) * (dv + DK) * DK;
        float* sfp = !SEG  ? p.S_final + sb
                     : trans   ? p.seg_state + seg_base + (size_t)dv * DK + col0 + n
                               : p.seg_state + seg_base + (size_t)(col0 + n) * DK;
        const int sst = trans ? DK : 1;
#pragma unroll
        for (int t = 0; t < NK; ++t)
#pragma unroll
            for (int j = 0; j < 4; ++j)
                Sacc[t][j] = trans ? (col0 + n == 16 * t + 4 * h + j ? 1.f : 0.f)
                             : (s0p && 16 * t < DKG) ? s0p[16 * t + 4 * h + j] : 0.f;
        if constexpr (!L::VST) v_load(0);
        // wait here for the initial state (and the first values): at the loop
        // head the state registers must not look like pending loads, or every
        // iteration would wait for all outstanding memory operations,
        // including the previous chunk's output stores
        __builtin_amdgcn_s_waitcnt(0x0f70);   // vmcnt(0)
        // the two preparation-only iterations
        for (int i = 0; i < 4; ++i) __syncthreads();

        // token-pair operands of the k-steps over the chunk (tiles 2s, 2s+1)
        auto pair_op = [&](const f32x4* tiles, int sidx) __attribute__((always_inline)) {
            return cat_h(to_h4(tiles[2 * sidx]), 2 * sidx + 1 < NT ? to_h4(tiles[2 * sidx + 1]) : zero_h4());
        };
        // first k-step of the next chunk's key and query operands, read at
        // the end of the previous chunk (those tiles are staged two chunks
        // ahead) so that phase A starts on its products
        h8 kf0[NT], qf0[NT];
        auto kq_first = [&](int cc) __attribute__((always_inline)) {
            lds_h* kl = lds_opaque(&s.K[cc % 3][n][8 * h]);
            lds_h* ql = lds_opaque(&s.Q[cc & 1][n][8 * h]);
#pragma unroll
            for (int rt = 0; rt < NT; ++rt) {
                kf0[rt] = lds_at<h8>(kl, 16 * rt * L::KP);
                qf0[rt] = lds_at<h8>(ql, 16 * rt * L::KP);
            }
        };
        kq_first(0);
        // (up to three scan waves) a chunk's staged value rows, read at the end
        // of the previous chunk like the first key and query slices (the
        // solve wave stores them in the previous chunk's phase A)
        auto v_first = [&](int cc) __attribute__((always_inline)) {
            const uint4* vrow = &s.Vs[cc & 1][n][2 * wave + (h & 1)];
#pragma unroll
            for (int rt = 0; rt < NT; ++rt) vraw[rt] = vrow[16 * rt * L::VS];
        };
        if constexpr (L::VST) v_first(0);
        // one chunk; PAR = parity of c (the LDS buffer of Q, T and P; keys by c mod 3)
        auto chunk = [&](auto PAR, int c) __attribute__((always_inline)) {
            constexpr int buf = decltype(PAR)::value;
            const int vb3 = c % 3;
            const int t0 = c * C;
            // ---- phase A: X = K S^T, Z^T = S Q^T ----
            h8 sh[NSS];
#pragma unroll
            for (int ss = 0; ss < NSS; ++ss) sh[ss] = cat_h(to_h4(Sacc[2 * ss]), to_h4(Sacc[2 * ss + 1]));
            f32x4 X[NT], Zt[NT];
#pragma unroll
            for (int rt = 0; rt < NT; ++rt) { X[rt] = zero4(); Zt[rt] = zero4(); }
            lds_h* kl = lds_opaque(&s.K[vb3][n][8 * h]);
            lds_h* ql = lds_opaque(&s.Q[buf][n][8 * h]);
#pragma unroll
            for (int ss = 0; ss < NSS; ++ss) {
                h8 kf[NT], qf[NT];
#pragma unroll
                for (int rt = 0; rt < NT; ++rt) {
                    kf[rt] = ss == 0 ? kf0[rt] : lds_at<h8>(kl, 16 * rt * L::KP + 32 * ss);
                    qf[rt] = ss == 0 ? qf0[rt] : lds_at<h8>(ql, 16 * rt * L::KP + 32 * ss);
                }
#pragma unroll
                for (int rt = 0; rt < NT; ++rt) X[rt] = mfma_h(kf[rt], sh[ss], X[rt]);
#pragma unroll
                for (int rt = 0; rt < NT; ++rt) Zt[rt] = mfma_h(sh[ss], qf[rt], Zt[rt]);
            }
            // The right-hand side needs X and the values only: it is formed in
            // this phase, where the scan waves wait for the prep waves anyway,
            // and only its fp16 operand crosses the barrier.
            // This chunk's values in the accumulator layout (token 16 rt + 4 h + j, column n):
            f32x4 Vt[NT];
#pragma unroll
            for (int rt = 0; rt < NT; ++rt)
                Vt[rt] = mfma_bf16(__builtin_bit_cast(bf16x8, vraw[rt]), vsel, zero4());
            // (four scan waves) the next chunk's values; past the last chunk
            // every row lies outside the buffer and reads zero, and loading
            // unconditionally keeps the wait for them precise
            if constexpr (!L::VST) v_load(c + 1);
            // Y = diag(beta) (V - diag(exp g) X)  (or eta V - beta exp(g) X)
            const float* f1b = ETA ? &s.eta[vb3][0] : &s.beta[vb3][0];
            const float* f2b = ETA ? &s.bge[vb3][0] : &s.eg[vb3][0];
            f32x4 Y[NT];
#pragma unroll
            for (int rt = 0; rt < NT; ++rt) {
                const f32x4 f1 = *reinterpret_cast<const f32x4*>(f1b + 16 * rt + 4 * h);
                const f32x4 f2 = *reinterpret_cast<const f32x4*>(f2b + 16 * rt + 4 * h);
#pragma unroll
                for (int j = 0; j < 4; ++j)
                    Y[rt][j] = ETA ? f1[j] * Vt[rt][j] - f2[j] * X[rt][j] : f1[j] * (Vt[rt][j] - f2[j] * X[rt][j]);
            }
            h8 yh[NTS];
#pragma unroll
            for (int ss = 0; ss < NTS; ++ss) yh[ss] = pair_op(Y, ss);
            // factors of phase B
            f32x4 fd[NT];
            float egr[NT];
#pragma unroll
            for (int rt = 0; rt < NT; ++rt) {
                fd[rt] = *reinterpret_cast<const f32x4*>(&s.dec[vb3][16 * rt + 4 * h]);
                egr[rt] = s.eg[vb3][16 * rt + n];
            }
            const float gl = s.glast[vb3];
            __syncthreads();
            // ---- phase B ----
            // T of this chunk (its blocks below the diagonal were formed in phase A)
            h8 top[NT][NTS];
            static_for<0, NT>([&](auto BB) {
                constexpr int b = decltype(BB)::value;
                static_for<0, b / 2 + 1>([&](auto SS) {
                    constexpr int sidx = decltype(SS)::value;
                    const h4 t0_ = *reinterpret_cast<const h4*>(&s.Tb[buf][L::bidx(b, 2 * sidx)][n][4 * h]);
                    h4 t1_ = zero_h4();
                    if constexpr (2 * sidx + 1 <= b)
                        t1_ = *reinterpret_cast<const h4*>(&s.Tb[buf][L::bidx(b, 2 * sidx + 1)][n][4 * h]);
                    top[b][sidx] = cat_h(t0_, t1_);
                });
            });
            // K^T operands of the state update, by the transposing read of the
            // token-major keys: for d_k block t and token k-step ss, lane
            // (n, h) receives d_k 16 t + n at the k-slots of the update's
            // other operand (tokens 32 ss + 4 h + j, then 32 ss + 16 + 4 h + j);
            // the lane addressing them, 16 h + 4 e + m, points at token
            // 32 ss + 4 h + e (+ 16) and d_k 16 t + 4 m .. + 3, whose place in
            // the row's k-order is 32 (t / 2) + 8 m + 4 (t % 2).  The first
            // token k-step is read now, well ahead of its use, so that its
            // latency hides behind the products in between; the second is read
            // into the same registers as the first is consumed.
            h8 ktop[NK];
            lds_h* ktr = lds_opaque(&s.K[vb3][4 * h + ((lane >> 2) & 3)][8 * (lane & 3)]);
            auto kt_one = [&](int ss, int t) __attribute__((always_inline)) {
                lds_h* a = ktr + 32 * ss * L::KP + 32 * (t >> 1) + 4 * (t & 1);
                const h4 lo = lds_read_tr(a);
                const h4 hi = 32 * ss + 16 < C ? lds_read_tr(a + 16 * L::KP) : zero_h4();
                return cat_h(lo, hi);
            };
#pragma unroll
            for (int t = 0; t < NK; ++t) ktop[t] = kt_one(0, t);
            __builtin_amdgcn_sched_barrier(0);
            // V' = T Y (T lower block triangular: row block b uses k-steps s <= b / 2)
            f32x4 Vp[NT];
            static_for<0, NT>([&](auto BB) {
                constexpr int b = decltype(BB)::value;
                f32x4 acc = zero4();
                static_for<0, b / 2 + 1>([&](auto SS) {
                    constexpr int sidx = decltype(SS)::value;
                    acc = mfma_h(top[b][sidx], yh[sidx], acc);
                });
                Vp[b] = acc;
            });
            // the scores of this chunk, read now (T's registers are free) so
            // that their latency hides behind the state update
            h8 pf[NT][NTS];
            static_for<0, NT>([&](auto RR) {
                constexpr int rt = decltype(RR)::value;
                static_for<0, rt / 2 + 1>([&](auto SS) {
                    constexpr int sidx = decltype(SS)::value;
                    const h4 p0 = *reinterpret_cast<const h4*>(&s.Pb[buf][L::bidx(rt, 2 * sidx)][n][4 * h]);
                    h4 p1 = zero_h4();
                    if constexpr (2 * sidx + 1 <= rt)
                        p1 = *reinterpret_cast<const h4*>(&s.Pb[buf][L::bidx(rt, 2 * sidx + 1)][n][4 * h]);
                    pf[rt][sidx] = cat_h(p0, p1);
                });
            });
            h8 vh[NTS];
#pragma unroll
            for (int ss = 0; ss < NTS; ++ss) vh[ss] = pair_op(Vp, ss);
            // S^T <- exp(g_last) S^T + K^T diag(exp(g_last - g)) V'
            f32x4 Vd[NT];
#pragma unroll
            for (int rt = 0; rt < NT; ++rt) Vd[rt] = fd[rt] * Vp[rt];
            h8 vd[NTS];
#pragma unroll
            for (int ss = 0; ss < NTS; ++ss) vd[ss] = pair_op(Vd, ss);
#pragma unroll
            for (int t = 0; t < NK; ++t) Sacc[t] *= gl;
#pragma unroll
            for (int ss = 0; ss < NTS; ++ss)
#pragma unroll
                for (int t = 0; t < NK; ++t) {
                    Sacc[t] = mfma_h(ktop[t], vd[ss], Sacc[t]);
                    if (ss + 1 < NTS) ktop[t] = kt_one(ss + 1, t);
                }
            if (c + 1 < nchunks) {
                kq_first(c + 1);
                if constexpr (L::VST) v_first(c + 1);
            }
            // O^T = diag(exp g) Z^T + V'^T P^T  (lane: row 16 rt + n, columns 4h..4h+3):
            // all products first, then the stores under one branch on the
            // output type; output rows past the end of the sequence fall
            // outside the buffer (dropped)
            f32x4 o[NT];
            static_for<0, NT>([&](auto RR) {
                constexpr int rt = decltype(RR)::value;
                f32x4 acc = zero4();
                static_for<0, rt / 2 + 1>([&](auto SS) {
                    constexpr int sidx = decltype(SS)::value;
                    acc = mfma_h(vh[sidx], pf[rt][sidx], acc);
                });
                o[rt] = egr[rt] * Zt[rt] + acc;
            });
            const uint32_t row0 = (uint32_t)(t0 + n) * ostr + col0 + 4 * h;
            if (obf) {
#pragma unroll
                for (int rt = 0; rt < NT; ++rt)
                    buf_store(obuf, (row0 + 16u * rt * ostr) * 2, __builtin_convertvector(o[rt], bf16x4));
            } else if (p.o_wt) {
#pragma unroll
                for (int rt = 0; rt < NT; ++rt) buf_store_wt(obuf, (row0 + 16u * rt * ostr) * 4, o[rt]);
            } else {
#pragma unroll
                for (int rt = 0; rt < NT; ++rt) buf_store(obuf, (row0 + 16u * rt * ostr) * 4, o[rt]);
            }
            if (p.dbg_V) {
                // stage output: V' rows of this chunk (rows past the end of the
                // sequence fall outside the buffer and are dropped)
                const buf_t dbuf = buffer_over(p.dbg_V + (size_t)bh * T * dv, (uint32_t)T * dv * 4);
                const uint32_t lane_off = 4u * ((uint32_t)(t0 + 4 * h) * dv + col0 + n);
#pragma unroll
                for (int rt = 0; rt < NT; ++rt)
#pragma unroll
                    for (int j = 0; j < 4; ++j) {
                        // (a bit_cast of the vector component itself stored
                        // component 0 four times; copy it out first)
                        const float e = Vp[rt][j];
                        __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(e), dbuf, (int)lane_off,
                                                              (int)(4u * (16 * rt + j) * dv), 0);
                    }
            }
            __syncthreads();
        };
        for (int c = 0; c < nchunks; c += 2) {
            chunk(std::integral_constant<int, 0>{}, c);
            if (c + 1 < nchunks) chunk(std::integral_constant<int, 1>{}, c + 1);
        }
#pragma unroll
        for (int t = 0; t < NK; ++t)
#pragma unroll
            for (int j = 0; j < 4; ++j)
                if (16 * t < DKG) sfp[(16 * t + 4 * h + j) * sst] = Sacc[t][j];
    }
}

}  // namespace gdn
