// gdn_api.hip -- C ABI of the chunkwise-parallel gated delta rule (gfx950).
// Validation, launch-shape choice and dispatch over the built kernel shapes.
#include <hip/hip_runtime.h>

#include <cstdint>
#include <cstdio>
#include <string>

#include "gdn.h"
#include "gdn_launch.h"

namespace {

thread_local std::string g_last_error;

gdn_status fail(gdn_status st, const std::string& msg) {
    g_last_error = msg;
    return st;
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// Built shapes of the default (fp16-operand) path for bf16 inputs.
bool fast_pair(int C, int dk) {
    if (C != 16 && C != 32 && C != 64) return false;
    if (dk == 32 || dk == 64 || dk == 96 || dk == 128) return true;
    return dk == 256 && C <= 32;
}

// Shapes some kernel covers.  bf16: C in {16, 32, 64} with d_k in
// {32, 64, 96, 128}, d_k 256 with C <= 32 (the fast path; d_k 16 is not
// built: the bf16 and fp16 MFMAs take 32 elements per k-step, and fp32
// inputs cover d_k 16); f32: C in {16, 32, 64} with d_k in
// {16, 32, 64, 128}, d_k 256 with C <= 32 (the generic kernel; C 64 with
// d_k 256 would need more than the 160 KB of LDS).  d_v: multiple of 16 in
// [16, 1024].
bool supported(const gdn_shape& s, std::string* why) {
    if (s.chunk_size != 16 && s.chunk_size != 32 && s.chunk_size != 64) {
        *why = "chunk_size must be 16, 32 or 64";
        return false;
    }
    if (s.qkv_dtype == GDN_BF16) {
        if (!fast_pair(s.chunk_size, s.d_k)) {
            *why = "bf16 inputs need d_k in {32, 64, 96, 128}, or 256 with chunk_size <= 32";
            return false;
        }
    } else {
        const bool dk_ok = s.d_k == 16 || s.d_k == 32 || s.d_k == 64 || s.d_k == 128 ||
                           (s.d_k == 256 && s.chunk_size <= 32);
        if (!dk_ok) {
            *why = "f32 inputs need d_k in {16, 32, 64, 128}, or 256 with chunk_size <= 32";
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
    // the fused kernels address one head's rows through 32-bit buffer
    // offsets: one head's largest tensor (fp32 output) must stay below 2 GiB
    const size_t head_bytes = (size_t)s->T * (size_t)(s->d_k > s->d_v ? s->d_k : s->d_v) * 4;
    if (head_bytes >= ((size_t)1 << 31))
        return fail(GDN_ERR_UNSUPPORTED, "one head's tensors must stay below 2 GiB (T too long)");
    return GDN_OK;
}

// Waves per workgroup of the generic kernel (16 value columns each): the
// largest of 4, 2, 1 that divides d_v / 16 and still gives at least one
// workgroup per compute unit.
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

// Compute units of the current device (256 on MI355X), read once.
int device_cus() {
    static const int n = [] {
        int dev = 0, cus = 0;
        if (hipGetDevice(&dev) != hipSuccess ||
            hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
            cus <= 0)
            return 256;
        return cus;
    }();
    return n;
}

// Scan waves per workgroup of the pipelined kernels (16 value columns each,
// one workgroup per compute unit): the choice of 1, 2 or 4 (dividing
// d_v / 16) that needs the fewest rounds of workgroups over the compute
// units, a four-wave workgroup weighing 1.4 rounds (its prep waves serve
// four slices; measured at d_k 96, d_v 192: 160 us for one round of them
// against about 110 us per round of two-wave workgroups); ties go to the
// smaller workgroup.
int choose_scan_waves(const gdn_shape& s) {
    const long heads = (long)s.B * s.H;
    const int cols16 = s.d_v / 16;
    const long cus = device_cus();
    int best = 1;
    double best_cost = 1e300;
    for (int ns : {1, 2, 4}) {
        if (cols16 % ns != 0) continue;
        const long wgs = heads * (cols16 / ns);
        const double cost = (double)((wgs + cus - 1) / cus) * (ns == 4 ? 1.4 : 1.0);
        if (cost < best_cost) {
            best = ns;
            best_cost = cost;
        }
    }
    return best;
}

bool pipe_shape(const gdn_shape& s) {
    return s.qkv_dtype == GDN_BF16 && (s.chunk_size == 32 || s.chunk_size == 64) &&
           (s.d_k == 64 || s.d_k == 128);
}

gdn_status check_launch() {
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return fail(GDN_ERR_HIP, hipGetErrorString(e));
    return GDN_OK;
}

}  // namespace

namespace gdn {
FwdLauncher fast_launcher(int C, int dk, int ns, bool eta) {
#define GDN_FAST_PICK(CC, KK) \
    if (C == CC && dk == KK) return fast_launcher_c##CC##_d##KK(ns, eta);
    GDN_FAST_PICK(16, 32)
    GDN_FAST_PICK(16, 64)
    GDN_FAST_PICK(16, 96)
    GDN_FAST_PICK(16, 128)
    GDN_FAST_PICK(16, 256)
    GDN_FAST_PICK(32, 32)
    GDN_FAST_PICK(32, 64)
    GDN_FAST_PICK(32, 96)
    GDN_FAST_PICK(32, 128)
    GDN_FAST_PICK(32, 256)
    GDN_FAST_PICK(64, 32)
    GDN_FAST_PICK(64, 64)
    GDN_FAST_PICK(64, 96)
    GDN_FAST_PICK(64, 128)
#undef GDN_FAST_PICK
    return nullptr;
}
}  // namespace gdn

namespace {

enum class Path { kFast, kPrecise };

struct ChunkArgs {
    const void *q, *k, *v;
    const float *alpha, *beta, *eta, *S0;
    void* O;
    float* S_final;
    float* dbg_T;
    float* dbg_V;
};

gdn_status run_chunk(const gdn_shape* s, const ChunkArgs& a, Path path, void* stream) {
    g_last_error.clear();
    gdn_status st = validate_shape(s);
    if (st != GDN_OK) return st;
    if (!a.q || !a.k || !a.v || !a.beta || !a.O || !a.S_final)
        return fail(GDN_ERR_NULL_ARG, "q, k, v, beta, O and S_final are required");
    if (!aligned16(a.q) || !aligned16(a.k) || !aligned16(a.v) || !aligned16(a.O) ||
        !aligned16(a.S_final) || (a.S0 && !aligned16(a.S0)) || !aligned16(a.beta) ||
        (a.alpha && !aligned16(a.alpha)) || (a.eta && !aligned16(a.eta)) ||
        (a.dbg_T && !aligned16(a.dbg_T)) || (a.dbg_V && !aligned16(a.dbg_V)))
        return fail(GDN_ERR_UNSUPPORTED, "tensor pointers must be 16-byte aligned");
    const bool bf = s->qkv_dtype == GDN_BF16;
    gdn::FwdLauncher launch = nullptr;
    int nw = 1;
    bool pipelined = false;
    if (bf && path == Path::kFast && fast_pair(s->chunk_size, s->d_k)) {
        nw = choose_scan_waves(*s);
        launch = gdn::fast_launcher(s->chunk_size, s->d_k, nw, a.eta != nullptr);
        pipelined = true;
    } else if (bf && pipe_shape(*s)) {
        nw = choose_scan_waves(*s);
        launch = gdn::pipe_launcher(s->chunk_size, s->d_k, nw, a.eta != nullptr);
        pipelined = true;
    } else {
        nw = choose_waves(*s);
        launch = gdn::generic_launcher(s->chunk_size, s->d_k, nw, bf, false);
    }
    if (!launch) return fail(GDN_ERR_UNSUPPORTED, "shape not built for this path");
    if ((a.dbg_T || a.dbg_V) && !(bf && path == Path::kFast && fast_pair(s->chunk_size, s->d_k)))
        return fail(GDN_ERR_UNSUPPORTED, "stage outputs exist for the fast bf16 path only");
    gdn::FwdParams p{};
    p.q = a.q;
    p.k = a.k;
    p.v = a.v;
    p.alpha = a.alpha;
    p.beta = a.beta;
    p.eta = a.eta;
    p.S0 = a.S0;
    p.O = a.O;
    p.S_final = a.S_final;
    p.dbg_T = a.dbg_T;
    p.dbg_V = a.dbg_V;
    p.B = s->B;
    p.H = s->H;
    p.T = s->T;
    p.dv = s->d_v;
    p.n_tiles = s->d_v / (16 * nw);
    p.o_bf16 = s->o_dtype == GDN_BF16;
    // The workgroups of one head are placed on one XCD (ids congruent mod 8,
    // sharing that XCD's L2 copy of the head's keys and queries); with B * H
    // not a multiple of 8 the grid is padded and the extra workgroups exit.
    const long heads = (long)s->B * s->H;
    p.xcd_groups = pipelined;
    const long grid_heads = pipelined ? (heads + 7) / 8 * 8 : heads;
    // fp32 output written through at system scope keeps the written bytes at
    // the output size; at d_v >= 256 plain non-temporal stores measured 6 %
    // faster (the write-back of partly written lines costs bytes, not time)
    p.o_wt = s->d_v < 256;
    const long nblocks = grid_heads * p.n_tiles;
    if (nblocks > 0x7fffffffL) return fail(GDN_ERR_BAD_SHAPE, "grid too large");
    launch(p, nblocks, reinterpret_cast<hipStream_t>(stream));
    return check_launch();
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
    return run_chunk(s, ChunkArgs{q, k, v, alpha, beta, eta, S0, O, S_final, nullptr, nullptr},
                     Path::kFast, stream);
}

gdn_status gdn_chunk_fwd_precise(const gdn_shape* s, const void* q, const void* k, const void* v,
                                 const float* alpha, const float* beta, const float* eta,
                                 const float* S0, void* O, float* S_final, void* stream) {
    return run_chunk(s, ChunkArgs{q, k, v, alpha, beta, eta, S0, O, S_final, nullptr, nullptr},
                     Path::kPrecise, stream);
}

gdn_status gdn_chunk_fwd_stages(const gdn_shape* s, const void* q, const void* k, const void* v,
                                const float* alpha, const float* beta, const float* eta,
                                const float* S0, void* O, float* S_final, float* T_out,
                                float* Vp_out, void* stream) {
    if (s && s->qkv_dtype != GDN_BF16) {
        g_last_error = "stage outputs exist for bf16 inputs only";
        return GDN_ERR_UNSUPPORTED;
    }
    return run_chunk(s, ChunkArgs{q, k, v, alpha, beta, eta, S0, O, S_final, T_out, Vp_out},
                     Path::kFast, stream);
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
    const gdn::FwdLauncher launch =
        gdn::generic_launcher(s->chunk_size, s->d_k, nw, s->qkv_dtype == GDN_BF16, true);
    if (!launch) return fail(GDN_ERR_UNSUPPORTED, "shape not built for the stage kernel");
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
    const gdn::RecLauncher launch = gdn::rec_launcher(s->d_k, s->qkv_dtype == GDN_BF16, &rpb);
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

int32_t gdn_version(void) { return 200; }

}  // extern "C"
