// gdn_api.hip -- C ABI of the chunkwise-parallel gated delta rule (gfx950).
// Validation, launch-shape choice and dispatch over the built kernel shapes.
#include <hip/hip_runtime.h>

#include <cstdint>
#include <cstdio>
#include <string>

#include "gdn.h"
#include "gdn_kernels.h"
#include "gdn_pipe.h"
#include "gdn_recurrent.h"

namespace {

thread_local std::string g_last_error;

gdn_status fail(gdn_status st, const std::string& msg) {
    g_last_error = msg;
    return st;
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// Built shapes.  bf16: C in {32, 64}, d_k in {32, 64, 128};
// f32: C in {16, 32, 64}, d_k in {16, 32, 64}.  d_v: multiple of 16.
bool supported(const gdn_shape& s, std::string* why) {
    if (s.qkv_dtype == GDN_BF16) {
        if (s.chunk_size != 32 && s.chunk_size != 64) {
            *why = "bf16 inputs need chunk_size 32 or 64";
            return false;
        }
        if (s.d_k != 32 && s.d_k != 64 && s.d_k != 128) {
            *why = "bf16 inputs need d_k in {32, 64, 128}";
            return false;
        }
    } else {
        if (s.chunk_size != 16 && s.chunk_size != 32 && s.chunk_size != 64) {
            *why = "f32 inputs need chunk_size 16, 32 or 64";
            return false;
        }
        if (s.d_k != 16 && s.d_k != 32 && s.d_k != 64) {
            *why = "f32 inputs need d_k in {16, 32, 64}";
            return false;
        }
    }
    if (s.d_v % 16 != 0 || s.d_v < 16 || s.d_v > 1024) {
        *why = "d_v must be a multiple of 16 in [16, 1024]";
        return false;
    }
    return true;
}

gdn_status validate_shape(const gdn_shape* s) {
    if (!s) return fail(GDN_ERR_NULL_ARG, "shape is NULL");
    if (s->B < 1 || s->H < 1 || s->T < 1)
        return fail(GDN_ERR_BAD_SHAPE, "B, H and T must be >= 1");
    if (s->d_k < 1 || s->d_v < 1 || s->chunk_size < 1)
        return fail(GDN_ERR_BAD_SHAPE, "d_k, d_v and chunk_size must be >= 1");
    if ((s->qkv_dtype != GDN_BF16 && s->qkv_dtype != GDN_F32) ||
        (s->o_dtype != GDN_BF16 && s->o_dtype != GDN_F32))
        return fail(GDN_ERR_BAD_DTYPE, "dtype must be GDN_BF16 or GDN_F32");
    const long double elems = (long double)s->B * s->H * s->T * (s->d_k > s->d_v ? s->d_k : s->d_v);
    if (elems > 4.0e18L) return fail(GDN_ERR_BAD_SHAPE, "tensor too large");
    std::string why;
    if (!supported(*s, &why)) return fail(GDN_ERR_UNSUPPORTED, why);
    return GDN_OK;
}

// Waves per workgroup (16 value columns each): the largest of 4, 2, 1 that
// divides d_v / 16 and still gives at least one workgroup per compute unit.
int choose_waves(const gdn_shape& s) {
    const int cols16 = s.d_v / 16;
    const long heads = (long)s.B * s.H;
    int best = 1;
    for (int nw : {4, 2, 1}) {
        if (cols16 % nw != 0) continue;
        best = nw;
        if (heads * (cols16 / nw) >= 256) return nw;
    }
    return best;
}

template <int C, int DK, int NW, bool BF>
void launch_fwd(const gdn::FwdParams& p, long nblocks, hipStream_t st) {
    hipLaunchKernelGGL((gdn::gdn_fwd_kernel<C, DK, NW, BF>), dim3((unsigned)nblocks),
                       dim3(NW * 64), 0, st, p);
}
template <int C, int DK, int NW, bool BF>
void launch_prep(const gdn::FwdParams& p, long nblocks, hipStream_t st) {
    hipLaunchKernelGGL((gdn::gdn_prep_kernel<C, DK, NW, BF>), dim3((unsigned)nblocks),
                       dim3(NW * 64), 0, st, p);
}

using Launcher = void (*)(const gdn::FwdParams&, long, hipStream_t);

template <int C, int DK, int NS>
void launch_pipe(const gdn::FwdParams& p, long nblocks, hipStream_t st) {
    if (p.eta)
        hipLaunchKernelGGL((gdn::gdn_fwd_pipe_kernel<C, DK, NS, true>), dim3((unsigned)nblocks),
                           dim3((NS + gdn::kPrepWaves) * 64), 0, st, p);
    else
        hipLaunchKernelGGL((gdn::gdn_fwd_pipe_kernel<C, DK, NS, false>), dim3((unsigned)nblocks),
                           dim3((NS + gdn::kPrepWaves) * 64), 0, st, p);
}

// Pipelined kernel: bf16 inputs, C in {32, 64}, d_k in {64, 128}.  NS scan
// waves of 16 value columns each per workgroup: the largest of 4, 2, 1 that
// divides d_v / 16 and still gives one workgroup per compute unit (256).
// The pipelined kernel addresses one head's rows through 32-bit buffer
// offsets, so one head's largest tensor (fp32 output) must stay below 2 GiB.
bool pipe_supported(const gdn_shape& s) {
    const size_t head_bytes = (size_t)s.T * (size_t)(s.d_k > s.d_v ? s.d_k : s.d_v) * 4;
    return s.qkv_dtype == GDN_BF16 && (s.chunk_size == 32 || s.chunk_size == 64) &&
           (s.d_k == 64 || s.d_k == 128) && head_bytes < ((size_t)1 << 31);
}
int choose_scan_waves(const gdn_shape& s) {
    const long heads = (long)s.B * s.H;
    const int cols16 = s.d_v / 16;
    for (int ns : {4, 2})
        if (cols16 % ns == 0 && heads * (cols16 / ns) >= 256) return ns;
    return 1;
}
Launcher pick_pipe(const gdn_shape& s, int ns) {
    const int C = s.chunk_size, DK = s.d_k;
#define GDN_PIPE(CC, KK)                                                        \
    if (C == CC && DK == KK)                                                    \
        return ns == 4 ? launch_pipe<CC, KK, 4>                                 \
                       : ns == 2 ? launch_pipe<CC, KK, 2> : launch_pipe<CC, KK, 1>;
    GDN_PIPE(64, 128)
    GDN_PIPE(64, 64)
    GDN_PIPE(32, 128)
    GDN_PIPE(32, 64)
#undef GDN_PIPE
    return nullptr;
}

template <int C, int DK, bool BF>
Launcher pick_nw(int nw, bool prep) {
    switch (nw) {
        case 1: return prep ? launch_prep<C, DK, 1, BF> : launch_fwd<C, DK, 1, BF>;
        case 2: return prep ? launch_prep<C, DK, 2, BF> : launch_fwd<C, DK, 2, BF>;
        default: return prep ? launch_prep<C, DK, 4, BF> : launch_fwd<C, DK, 4, BF>;
    }
}

Launcher pick(const gdn_shape& s, int nw, bool prep) {
    const int C = s.chunk_size, DK = s.d_k;
    if (s.qkv_dtype == GDN_BF16) {
        if (C == 64 && DK == 128) return pick_nw<64, 128, true>(nw, prep);
        if (C == 64 && DK == 64) return pick_nw<64, 64, true>(nw, prep);
        if (C == 64 && DK == 32) return pick_nw<64, 32, true>(nw, prep);
        if (C == 32 && DK == 128) return pick_nw<32, 128, true>(nw, prep);
        if (C == 32 && DK == 64) return pick_nw<32, 64, true>(nw, prep);
        if (C == 32 && DK == 32) return pick_nw<32, 32, true>(nw, prep);
    } else {
        if (C == 64 && DK == 64) return pick_nw<64, 64, false>(nw, prep);
        if (C == 64 && DK == 32) return pick_nw<64, 32, false>(nw, prep);
        if (C == 64 && DK == 16) return pick_nw<64, 16, false>(nw, prep);
        if (C == 32 && DK == 64) return pick_nw<32, 64, false>(nw, prep);
        if (C == 32 && DK == 32) return pick_nw<32, 32, false>(nw, prep);
        if (C == 32 && DK == 16) return pick_nw<32, 16, false>(nw, prep);
        if (C == 16 && DK == 64) return pick_nw<16, 64, false>(nw, prep);
        if (C == 16 && DK == 32) return pick_nw<16, 32, false>(nw, prep);
        if (C == 16 && DK == 16) return pick_nw<16, 16, false>(nw, prep);
    }
    return nullptr;
}

using RecLauncher = void (*)(const gdn::RecParams&, long, hipStream_t);

template <int DK, bool BF>
void launch_rec(const gdn::RecParams& p, long nblocks, hipStream_t st) {
    hipLaunchKernelGGL((gdn::gdn_recurrent_kernel<DK, BF>), dim3((unsigned)nblocks),
                       dim3(gdn::kRecThreads), 0, st, p);
}

RecLauncher pick_rec(int dk, bool bf, int* rows_per_block) {
#define GDN_REC(D)                                                               \
    if (dk == D) {                                                               \
        *rows_per_block = gdn::kRecRows * (gdn::kRecThreads / 64) * (64 / gdn::rec_lanes_per_row(D)); \
        return bf ? launch_rec<D, true> : launch_rec<D, false>;                  \
    }
    GDN_REC(16)
    GDN_REC(32)
    GDN_REC(64)
    GDN_REC(96)
    GDN_REC(128)
    GDN_REC(192)
    GDN_REC(256)
#undef GDN_REC
    return nullptr;
}

gdn_status check_launch() {
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return fail(GDN_ERR_HIP, hipGetErrorString(e));
    return GDN_OK;
}

}  // namespace

extern "C" {

size_t gdn_chunk_fwd_workspace_bytes(const gdn_shape* s) {
    if (validate_shape(s) != GDN_OK) return (size_t)-1;
    return 0;
}

gdn_status gdn_chunk_fwd(const gdn_shape* s, const void* q, const void* k, const void* v,
                         const float* alpha, const float* beta, const float* S0, void* O,
                         float* S_final, void* workspace, size_t workspace_bytes, void* stream) {
    return gdn_chunk_fwd_eta(s, q, k, v, alpha, beta, nullptr, S0, O, S_final, workspace,
                             workspace_bytes, stream);
}

gdn_status gdn_chunk_fwd_eta(const gdn_shape* s, const void* q, const void* k, const void* v,
                             const float* alpha, const float* beta, const float* eta,
                             const float* S0, void* O, float* S_final, void* workspace,
                             size_t workspace_bytes, void* stream) {
    (void)workspace;
    (void)workspace_bytes;
    g_last_error.clear();
    gdn_status st = validate_shape(s);
    if (st != GDN_OK) return st;
    if (!q || !k || !v || !beta || !O || !S_final)
        return fail(GDN_ERR_NULL_ARG, "q, k, v, beta, O and S_final are required");
    if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(O) || !aligned16(S_final) ||
        (S0 && !aligned16(S0)) || !aligned16(beta) || (alpha && !aligned16(alpha)) ||
        (eta && !aligned16(eta)))
        return fail(GDN_ERR_UNSUPPORTED, "tensor pointers must be 16-byte aligned");
    const bool piped = pipe_supported(*s);
    const int nw = piped ? choose_scan_waves(*s) : choose_waves(*s);
    const Launcher launch = piped ? pick_pipe(*s, nw) : pick(*s, nw, false);
    if (!launch) return fail(GDN_ERR_UNSUPPORTED, "shape not built");
    gdn::FwdParams p{};
    p.q = q;
    p.k = k;
    p.v = v;
    p.alpha = alpha;
    p.beta = beta;
    p.eta = eta;
    p.S0 = S0;
    p.O = O;
    p.S_final = S_final;
    p.B = s->B;
    p.H = s->H;
    p.T = s->T;
    p.dv = s->d_v;
    p.n_tiles = s->d_v / (16 * nw);
    p.o_bf16 = s->o_dtype == GDN_BF16;
    p.xcd_groups = piped && ((long)s->B * s->H) % 8 == 0;
    const long nblocks = (long)s->B * s->H * p.n_tiles;
    if (nblocks > 0x7fffffffL) return fail(GDN_ERR_BAD_SHAPE, "grid too large");
    launch(p, nblocks, reinterpret_cast<hipStream_t>(stream));
    return check_launch();
}

gdn_status gdn_chunk_prep(const gdn_shape* s, const void* k, const void* v, const float* alpha,
                          const float* beta, float* T_out, float* W_out, float* U_out,
                          void* workspace, size_t workspace_bytes, void* stream) {
    (void)workspace;
    (void)workspace_bytes;
    g_last_error.clear();
    gdn_status st = validate_shape(s);
    if (st != GDN_OK) return st;
    if (!k || !v || !beta) return fail(GDN_ERR_NULL_ARG, "k, v and beta are required");
    if (!aligned16(k) || !aligned16(v) || !aligned16(beta) || (alpha && !aligned16(alpha)))
        return fail(GDN_ERR_UNSUPPORTED, "tensor pointers must be 16-byte aligned");
    if (!T_out && !W_out && !U_out) return GDN_OK;
    const int nw = choose_waves(*s);
    const Launcher launch = pick(*s, nw, true);
    if (!launch) return fail(GDN_ERR_UNSUPPORTED, "shape not built");
    gdn::FwdParams p{};
    p.k = k;
    p.v = v;
    p.alpha = alpha;
    p.beta = beta;
    p.T_out = T_out;
    p.W_out = W_out;
    p.U_out = U_out;
    p.B = s->B;
    p.H = s->H;
    p.T = s->T;
    p.dv = s->d_v;
    p.n_tiles = s->d_v / (16 * nw);
    const long nchunks = (s->T + s->chunk_size - 1) / s->chunk_size;
    const long nblocks = (long)s->B * s->H * nchunks * p.n_tiles;
    if (nblocks > 0x7fffffffL) return fail(GDN_ERR_BAD_SHAPE, "grid too large");
    launch(p, nblocks, reinterpret_cast<hipStream_t>(stream));
    return check_launch();
}

gdn_status gdn_recurrent_fwd(const gdn_shape* s, const void* q, const void* k, const void* v,
                             const float* alpha, const float* beta, const float* S0, void* O,
                             float* S_final, void* stream) {
    return gdn_recurrent_fwd_eta(s, q, k, v, alpha, beta, nullptr, S0, O, S_final, stream);
}

gdn_status gdn_recurrent_fwd_eta(const gdn_shape* s, const void* q, const void* k, const void* v,
                                 const float* alpha, const float* beta, const float* eta,
                                 const float* S0, void* O, float* S_final, void* stream) {
    g_last_error.clear();
    if (!s) return fail(GDN_ERR_NULL_ARG, "shape is NULL");
    if (s->B < 1 || s->H < 1 || s->T < 1 || s->d_k < 1 || s->d_v < 1)
        return fail(GDN_ERR_BAD_SHAPE, "B, H, T, d_k and d_v must be >= 1");
    if ((s->qkv_dtype != GDN_BF16 && s->qkv_dtype != GDN_F32) ||
        (s->o_dtype != GDN_BF16 && s->o_dtype != GDN_F32))
        return fail(GDN_ERR_BAD_DTYPE, "dtype must be GDN_BF16 or GDN_F32");
    const long double elems = (long double)s->B * s->H * s->T * (s->d_k > s->d_v ? s->d_k : s->d_v);
    if (elems > 4.0e18L) return fail(GDN_ERR_BAD_SHAPE, "tensor too large");
    if (s->d_v > 65536) return fail(GDN_ERR_UNSUPPORTED, "d_v must be <= 65536");
    int rpb = 0;
    const RecLauncher launch = pick_rec(s->d_k, s->qkv_dtype == GDN_BF16, &rpb);
    if (!launch) return fail(GDN_ERR_UNSUPPORTED, "d_k must be one of 16, 32, 64, 96, 128, 192, 256");
    if (!q || !k || !v || !beta || !O || !S_final)
        return fail(GDN_ERR_NULL_ARG, "q, k, v, beta, O and S_final are required");
    if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(O) || !aligned16(S_final) ||
        (S0 && !aligned16(S0)) || !aligned16(beta) || (alpha && !aligned16(alpha)) ||
        (eta && !aligned16(eta)))
        return fail(GDN_ERR_UNSUPPORTED, "tensor pointers must be 16-byte aligned");
    gdn::RecParams p{};
    p.q = q;
    p.k = k;
    p.v = v;
    p.alpha = alpha;
    p.beta = beta;
    p.eta = eta;
    p.S0 = S0;
    p.O = O;
    p.S_final = S_final;
    p.T = s->T;
    p.dv = s->d_v;
    p.blocks_per_head = (s->d_v + rpb - 1) / rpb;
    p.o_bf16 = s->o_dtype == GDN_BF16;
    const long nblocks = (long)s->B * s->H * p.blocks_per_head;
    if (nblocks > 0x7fffffffL) return fail(GDN_ERR_BAD_SHAPE, "grid too large");
    launch(p, nblocks, reinterpret_cast<hipStream_t>(stream));
    return check_launch();
}

const char* gdn_status_string(gdn_status st) {
    switch (st) {
        case GDN_OK: return "ok";
        case GDN_ERR_NULL_ARG: return "required pointer is NULL";
        case GDN_ERR_BAD_SHAPE: return "bad shape";
        case GDN_ERR_BAD_DTYPE: return "bad dtype";
        case GDN_ERR_UNSUPPORTED: return "unsupported configuration";
        case GDN_ERR_WORKSPACE: return "workspace too small";
        case GDN_ERR_HIP: return "HIP runtime error";
    }
    return "unknown status";
}

const char* gdn_last_error(void) { return g_last_error.c_str(); }

int32_t gdn_version(void) { return 100; }

}  // extern "C"
