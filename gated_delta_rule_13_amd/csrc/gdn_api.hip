// gdn_api.hip -- C ABI of the chunkwise-parallel gated delta rule (gfx950).
// Validation, launch-shape choice and dispatch over the built kernel shapes.
#include <hip/hip_runtime.h>

#include <cstdint>
#include <cstdio>
#include <mutex>
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
    if (dk == 16 || dk == 32 || dk == 64 || dk == 96 || dk == 128) return true;
    return dk == 256 && C <= 32;
}

// The shape the kernels run: at d_k 256 a 64-token chunk is computed as two
// 32-token chunks (64-token tiles of d_k 256 would need more than the
// 160 KB of LDS).  The chunk length only groups the same recurrence, so the
// result is the same function of the inputs, up to rounding.
gdn_shape compute_shape(const gdn_shape& s) {
    gdn_shape c = s;
    if (s.d_k == 256 && s.chunk_size == 64) c.chunk_size = 32;
    return c;
}

// Shapes some kernel covers (checked on the compute shape).  bf16: C in
// {16, 32, 64} with d_k in {16, 32, 64, 96, 128, 256} (the fast path; d_k
// 16 runs zero-padded on the d_k 32 kernel); f32: C in {16, 32, 64} with
// d_k in {16, 32, 64, 128, 256} (the generic kernel).  d_v: multiple of 16
// in [16, 1024].
bool supported(const gdn_shape& s0, std::string* why) {
    if (s0.chunk_size != 16 && s0.chunk_size != 32 && s0.chunk_size != 64) {
        *why = "chunk_size must be 16, 32 or 64";
        return false;
    }
    const gdn_shape s = compute_shape(s0);
    if (s.qkv_dtype == GDN_BF16) {
        if (!fast_pair(s.chunk_size, s.d_k)) {
            *why = "bf16 inputs need d_k in {16, 32, 64, 96, 128, 256}";
            return false;
        }
    } else {
        const bool dk_ok = s.d_k == 16 || s.d_k == 32 || s.d_k == 64 || s.d_k == 128 ||
                           (s.d_k == 256 && s.chunk_size <= 32);
        if (!dk_ok) {
            *why = "f32 inputs need d_k in {16, 32, 64, 128, 256}";
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
// one workgroup per compute unit): the choice among 1, 2, 4 and, for the
// fused kernel, 3 (dividing d_v / 16) that needs the fewest rounds of
// workgroups over the compute units, a four-wave workgroup weighing 1.4
// rounds (its four prep waves serve four slices; measured at d_k 96,
// d_v 192: 160 us for one round of them against about 110 us per round of
// two-wave workgroups) and a three-wave one 1.2 (five prep waves; 141 us
// for one round at that shape); ties go to the smaller workgroup.
int choose_scan_waves(const gdn_shape& s, bool three = false) {
    const long heads = (long)s.B * s.H;
    const int cols16 = s.d_v / 16;
    const long cus = device_cus();
    int best = 1;
    double best_cost = 1e300;
    for (int ns : {1, 2, 3, 4}) {
        if (cols16 % ns != 0 || (ns == 3 && !three)) continue;
        const long wgs = heads * (cols16 / ns);
        const double cost = (double)((wgs + cus - 1) / cus) * (ns == 4 ? 1.4 : ns == 3 ? 1.2 : 1.0);
        if (cost < best_cost) {
            best = ns;
            best_cost = cost;
        }
    }
    return best;
}

// ---------------------------------------------------------------------------
// Sequence-parallel form of the default path.  When the heads and value
// tiles of a call leave compute units idle, each sequence is cut into
// segments of whole chunks that run at once (the later ones from a zero
// state, with d_k extra transition rows), then one more launch combines the
// segments and corrects the later segments' outputs (gdn_seq.h).
// Cost model in microseconds, fitted to measurements on MI355X (one fused
// kernel iteration: 1.4 us at d_k <= 64, 1.6 us above, times 1.25 for two
// scan waves, 1.5 for three and 1.75 for four):
//   plain  rounds(B H d_v / (16 ns)) (n_chunks + 2) it
//   seq    rounds(B H (n_v + (n_seg - 1) (n_v + n_k))) (L + 2) it
//          + 6.5 (the second launch and its first memory round trip)
//          + (n_seg - 1) step   (the combine's dependent steps: 1 us at
//                                d_k <= 64, 2.5 us at 96 / 128, 4 us at 256)
//          + the correction's bytes at 1.5 TB/s
// with rounds(x) = ceil(x / CUs), n_v and n_k the value and transition
// tiles per segment and L the chunks per segment.  The sequence-parallel
// form is taken when it is estimated at least 10 % faster.
struct Plan {
    int ns = 1;           // scan waves per workgroup
    int nseg = 1;         // segments per sequence
    int seg_len = 0;      // tokens per segment
    size_t off_q = 0, off_o = 0, bytes = 0;   // workspace layout
};

double iter_us(int dk, int ns) {
    return (dk <= 64 ? 1.4 : 1.6) * (ns == 1 ? 1.0 : ns == 2 ? 1.25 : ns == 3 ? 1.5 : 1.75);
}
long rounds_over_cus(long wgs) {
    const long cus = device_cus();
    return (wgs + cus - 1) / cus;
}

double plain_cost(const gdn_shape& s, int ns) {
    const long nchunks = (s.T + s.chunk_size - 1) / s.chunk_size;
    const long wgs = (long)s.B * s.H * (s.d_v / (16 * ns));
    return (double)rounds_over_cus(wgs) * (double)(nchunks + 2) * iter_us(s.d_k, ns);
}

double seq_cost(const gdn_shape& s, int ns, int seg_chunks) {
    const long nchunks = (s.T + s.chunk_size - 1) / s.chunk_size;
    const long nseg = (nchunks + seg_chunks - 1) / seg_chunks;
    const long nv = s.d_v / (16 * ns), nk = s.d_k / (16 * ns);
    const long bh = (long)s.B * s.H;
    const long wgs = bh * (nv + (nseg - 1) * (nv + nk));
    const double fused = (double)rounds_over_cus(wgs) * (double)(seg_chunks + 2) * iter_us(s.d_k, ns);
    const double step = s.d_k <= 64 ? 1.0 : s.d_k <= 128 ? 2.5 : 4.0;
    const double corr_tokens = (double)bh * (double)(s.T - (long)seg_chunks * s.chunk_size);
    const double corr_bytes = corr_tokens * 4.0 * (s.d_k + 2.0 * s.d_v);
    return fused + 6.5 + step * (double)(nseg - 1) + corr_bytes / 1.5e6;
}

void plan_workspace(const gdn_shape& s, Plan* pl) {
    pl->off_q = pl->off_o = pl->bytes = 0;
    if (pl->nseg <= 1) return;
    auto up = [](size_t x) { return (x + 255) & ~(size_t)255; };
    const size_t bh = (size_t)s.B * s.H;
    pl->off_q = up(bh * pl->nseg * (size_t)(s.d_v + s.d_k) * s.d_k * 4);
    pl->off_o = up(pl->off_q + bh * (size_t)s.T * s.d_k * 4);
    pl->bytes = pl->off_o + (s.o_dtype == GDN_BF16 ? bh * (size_t)s.T * s.d_v * 4 : 0);
}

// Plan of a default-path call with bf16 inputs on the fused kernel:
// seg_chunks 0 picks by the cost model, seg_chunks > 0 fixes the chunks per
// segment (one segment: the plain form).  The segmented form runs one scan
// wave per workgroup (the most workgroups, the shortest iteration); the
// model is only trusted where its fused pass is one round of workgroups
// over the compute units and there are at most 8 segments, so the default
// plan stays inside that range.
Plan make_plan(const gdn_shape& s, int seg_chunks) {
    Plan pl;
    pl.ns = choose_scan_waves(s, true);
    pl.seg_len = s.T;
    const long nchunks = (s.T + s.chunk_size - 1) / s.chunk_size;
    int best_L = 0;
    if (s.d_k < 32) {
        // (no segments at d_k 16: its kernel runs zero-padded)
    } else if (seg_chunks > 0) {
        if (seg_chunks < nchunks) best_L = seg_chunks;
    } else {
        const long bh = (long)s.B * s.H;
        const long nv = s.d_v / 16, nk = s.d_k / 16;
        double best = 0.9 * plain_cost(s, pl.ns);
        for (long L = 1; L < nchunks; ++L) {
            const long nseg = (nchunks + L - 1) / L;
            // only the smallest L of each segment count
            if (L > 1 && nseg == (nchunks + L - 2) / (L - 1)) continue;
            if (nseg > 8 || rounds_over_cus(bh * (nv + (nseg - 1) * (nv + nk))) > 1) continue;
            const double c = seq_cost(s, 1, (int)L);
            if (c < best) {
                best = c;
                best_L = (int)L;
            }
        }
    }
    if (best_L > 0) {
        pl.ns = 1;
        pl.seg_len = best_L * s.chunk_size;
        pl.nseg = (int)((nchunks + best_L - 1) / best_L);
    }
    plan_workspace(s, &pl);
    return pl;
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
FwdLauncher fast_launcher(int C, int dk, int ns, bool eta, bool seg) {
#define GDN_FAST_PICK(CC, KK) \
    if (C == CC && dk == KK) return fast_launcher_c##CC##_d##KK(ns, eta, seg);
    GDN_FAST_PICK(16, 16)
    GDN_FAST_PICK(32, 16)
    GDN_FAST_PICK(64, 16)
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

// seg_chunks: < 0 the plain form only; 0 the default plan; > 0 that many
// chunks per segment (default path, fused kernel).
gdn_status run_chunk(const gdn_shape* s_in, const ChunkArgs& a, Path path, void* stream,
                     int seg_chunks = -1, void* workspace = nullptr, size_t workspace_bytes = 0) {
    g_last_error.clear();
    gdn_status st = validate_shape(s_in);
    if (st != GDN_OK) return st;
    const gdn_shape cs = compute_shape(*s_in);
    const gdn_shape* s = &cs;
    // (segment lengths count the caller's chunks)
    if (seg_chunks > 0) seg_chunks *= s_in->chunk_size / cs.chunk_size;
    if (!a.q || !a.k || !a.v || !a.beta || !a.O || !a.S_final)
        return fail(GDN_ERR_NULL_ARG, "q, k, v, beta, O and S_final are required");
    if (!aligned16(a.q) || !aligned16(a.k) || !aligned16(a.v) || !aligned16(a.O) ||
        !aligned16(a.S_final) || (a.S0 && !aligned16(a.S0)) || !aligned16(a.beta) ||
        (a.alpha && !aligned16(a.alpha)) || (a.eta && !aligned16(a.eta)) ||
        (a.dbg_T && !aligned16(a.dbg_T)) || (a.dbg_V && !aligned16(a.dbg_V)))
        return fail(GDN_ERR_UNSUPPORTED, "tensor pointers must be 16-byte aligned");
    const bool bf = s->qkv_dtype == GDN_BF16;
    const bool fused = bf && path == Path::kFast && fast_pair(s->chunk_size, s->d_k);
    Plan plan;
    plan.ns = choose_scan_waves(*s, true);
    if (fused && seg_chunks >= 0) plan = make_plan(*s, seg_chunks);
    if (seg_chunks > 0 && !fused &&
        (long)seg_chunks * s->chunk_size < (long)s->T)
        return fail(GDN_ERR_UNSUPPORTED, "segments exist on the default path with bf16 inputs only");
    if (seg_chunks > 0 && s->d_k < 32 && (long)seg_chunks * s->chunk_size < (long)s->T)
        return fail(GDN_ERR_UNSUPPORTED, "segments need d_k >= 32");
    if (plan.nseg > 1) {
        if (!workspace || workspace_bytes < plan.bytes)
            return fail(GDN_ERR_WORKSPACE, "workspace smaller than gdn_chunk_fwd_workspace_bytes");
        if ((reinterpret_cast<uintptr_t>(workspace) & 255u) != 0)
            return fail(GDN_ERR_UNSUPPORTED, "workspace must be 256-byte aligned");
    }
    gdn::FwdLauncher launch = nullptr;
    int nw = 1;
    bool pipelined = false;
    if (fused) {
        nw = plan.ns;
        launch = gdn::fast_launcher(s->chunk_size, s->d_k, nw, a.eta != nullptr, plan.nseg > 1);
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
    p.n_tiles_v = s->d_v / (16 * nw);
    p.n_tiles = p.n_tiles_v;
    p.o_bf16 = s->o_dtype == GDN_BF16;
    p.nseg = 1;
    p.seg_len = s->T;
    gdn::SeqLauncher finish = nullptr;
    if (plan.nseg > 1) {
        finish = gdn::seq_launcher(s->d_k);
        if (!finish) return fail(GDN_ERR_UNSUPPORTED, "segments not built for this d_k");
        char* ws = static_cast<char*>(workspace);
        p.nseg = plan.nseg;
        p.seg_len = plan.seg_len;
        p.n_tiles = p.n_tiles_v + s->d_k / (16 * nw);
        p.seg_state = reinterpret_cast<float*>(ws);
        p.seg_q = reinterpret_cast<float*>(ws + plan.off_q);
        p.seg_o = p.o_bf16 ? reinterpret_cast<float*>(ws + plan.off_o) : nullptr;
    }
    // The workgroups of one unit (head and segment) are placed on one XCD
    // (ids congruent mod 8, sharing that XCD's L2 copy of the unit's keys and
    // queries); with units not a multiple of 8 the grid is padded and the
    // extra workgroups exit.
    const long units = (long)s->B * s->H * p.nseg;
    p.xcd_groups = pipelined;
    const long grid_units = pipelined ? (units + 7) / 8 * 8 : units;
    // fp32 output written through at system scope keeps the written bytes at
    // the output size.  Where the scan waves load their own values (the
    // split-bf16 kernel; the fused kernel with four scan waves and four prep
    // waves) their waits for those loads also wait for their earlier stores,
    // and at d_v >= 256 plain non-temporal stores measured 6 % faster there
    // (the write-back of partly written lines costs bytes, not time).
    const bool staged = fused && gdn::fast_prep_waves(nw, s->chunk_size, s->d_k < 32 ? 32 : s->d_k) != 4;
    p.o_wt = s->d_v < 256 || staged;
    const long nblocks = grid_units * p.n_tiles;
    if (nblocks > 0x7fffffffL) return fail(GDN_ERR_BAD_SHAPE, "grid too large");
    if (finish) {
        // the finishing kernel: (head, later segment, token group) units padded
        // to a multiple of 8, d_v / 16 row blocks each
        const long units = (long)s->B * s->H * (p.nseg - 1) *
                           ((p.seg_len + gdn::seq_group_tokens(s->d_k) - 1) /
                            gdn::seq_group_tokens(s->d_k));
        if ((units + 7) / 8 * 8 * (s->d_v / 16) > 0x7fffffffL)
            return fail(GDN_ERR_BAD_SHAPE, "grid too large");
    }
    const hipStream_t hs = reinterpret_cast<hipStream_t>(stream);
    launch(p, nblocks, hs);
    if (finish) {
        gdn::SeqParams q{};
        q.BH = s->B * s->H;
        q.nseg = p.nseg;
        q.seg_len = p.seg_len;
        q.T = s->T;
        q.dv = s->d_v;
        q.seg_state = p.seg_state;
        q.seg_q = p.seg_q;
        q.seg_o = p.seg_o;
        q.O = a.O;
        q.o_bf16 = p.o_bf16;
        q.S_final = a.S_final;
        finish(q, hs);
    }
    return check_launch();
}

}  // namespace

namespace {

// Scratch of gdn_chunk_fwd_seq_noalloc (for callers that cannot allocate):
// a file-scope device array, one copy per GPU, held until the process ends.
// Host code never uses the array's name as an address: its device address
// is looked up once per device with hipGetSymbolAddress (with that device
// current) and kept in scratch_addr.
constexpr size_t kScratchBytes = (size_t)64 << 20;
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_addr[kMaxDevices] = {};

// Device address of the current device's scratch array, or null (error
// recorded) when it cannot be found.
void* scratch_addr() {
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) {
        g_last_error = "no current HIP device (or device index beyond 63)";
        return nullptr;
    }
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_addr[dev]) {
        void* ptr = nullptr;
        const hipError_t e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
        if (e != hipSuccess || !ptr) {
            g_last_error = std::string("hipGetSymbolAddress(scratch): ") + hipGetErrorString(e);
            return nullptr;
        }
        g_scratch_addr[dev] = ptr;
    }
    return g_scratch_addr[dev];
}

}  // namespace

extern "C" {

size_t gdn_chunk_fwd_workspace_bytes(const gdn_shape* s) {
    return gdn_chunk_fwd_seq_workspace_bytes(s, 0);
}

size_t gdn_chunk_fwd_seq_workspace_bytes(const gdn_shape* s, int seg_chunks) {
    if (validate_shape(s) != GDN_OK) return (size_t)-1;
    if (seg_chunks < 0) {
        g_last_error = "seg_chunks must be >= 0";
        return (size_t)-1;
    }
    if (s->qkv_dtype != GDN_BF16) return 0;
    const gdn_shape cs = compute_shape(*s);
    return make_plan(cs, seg_chunks * (s->chunk_size / cs.chunk_size)).bytes;
}

gdn_status gdn_chunk_fwd_seq(const gdn_shape* s, int seg_chunks, const void* q, const void* k,
                             const void* v, const float* alpha, const float* beta,
                             const float* eta, const float* S0, void* O, float* S_final,
                             void* workspace, size_t workspace_bytes, void* stream) {
    if (seg_chunks < 0) {
        g_last_error = "seg_chunks must be >= 0";
        return GDN_ERR_BAD_SHAPE;
    }
    return run_chunk(s, ChunkArgs{q, k, v, alpha, beta, eta, S0, O, S_final, nullptr, nullptr},
                     Path::kFast, stream, seg_chunks, workspace, workspace_bytes);
}

gdn_status gdn_chunk_fwd_seq_noalloc(const gdn_shape* s, int seg_chunks, const void* q,
                                     const void* k, const void* v, const float* alpha,
                                     const float* beta, const float* eta, const float* S0,
                                     void* O, float* S_final, void* stream) {
    g_last_error.clear();
    if (seg_chunks < 0) {
        g_last_error = "seg_chunks must be >= 0";
        return GDN_ERR_BAD_SHAPE;
    }
    const size_t need = gdn_chunk_fwd_seq_workspace_bytes(s, seg_chunks);
    if (need == (size_t)-1) {
        const gdn_status st = validate_shape(s);
        return st != GDN_OK ? st : GDN_ERR_BAD_SHAPE;
    }
    if (need > kScratchBytes)
        return fail(GDN_ERR_WORKSPACE,
                    "this plan needs " + std::to_string(need) +
                        " bytes of scratch, more than the library's 64 MiB (67108864 bytes); "
                        "use gdn_chunk_fwd_seq with a workspace");
    void* ws = nullptr;
    if (need > 0) {
        ws = scratch_addr();
        if (!ws) return GDN_ERR_HIP;
    }
    return run_chunk(s, ChunkArgs{q, k, v, alpha, beta, eta, S0, O, S_final, nullptr, nullptr},
                     Path::kFast, stream, seg_chunks, ws, need > 0 ? kScratchBytes : 0);
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
    return run_chunk(s, ChunkArgs{q, k, v, alpha, beta, eta, S0, O, S_final, nullptr, nullptr},
                     Path::kFast, stream, 0, workspace, workspace_bytes);
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
    if (s && s->d_k == 256 && s->chunk_size == 64) {
        // (T per chunk is laid out by the caller's chunk length)
        g_last_error = "stage outputs at d_k 256 need chunk_size <= 32";
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
