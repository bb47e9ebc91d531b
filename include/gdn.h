/*
 * gdn.h -- C ABI of the MI355X (gfx950) chunkwise-parallel gated delta rule.
 *
 * The operation (all pages agree once the orientation is fixed; S is
 * d_v x d_k and o = S q):
 *
 *     S_t = alpha_t S_{t-1} (I - beta_t k_t k_t^T) + beta_t v_t k_t^T
 *     o_t = S_t q_t                     (the output sees token t's write)
 *
 * Sources: "从零开始的 GDN 推导", the recurrent form under the notation
 * section (gate alpha_t multiplying the erased state) and the section on O
 * (o_t = q_t S_{t+1}, i.e. inclusive); "RNN的复兴03:现代RNN的并行计算",
 * section 1, equation (2) (S in R^{d_v x d_k}); the circuit-complexity page,
 * "类 RNN 模型训练" (o_t = S_t q_t).  The library evaluates it with the
 * chunkwise-parallel method of "从零开始的 GDN 推导" (UT transform, W and U,
 * per-chunk state and output, chunks chained), which reaches the same result
 * up to rounding order.
 *
 * Conventions for every entry point:
 *  - Tensor pointers are DEVICE pointers to row-major, contiguous memory on
 *    the current HIP device; the caller owns all of them.  The library never
 *    allocates, frees or keeps a pointer after the call returns.
 *  - Calls are stream-ordered and asynchronous: `stream` is a hipStream_t
 *    (NULL = the default stream).  The return value reports argument
 *    validation and launch errors; a fault inside a kernel surfaces at the
 *    caller's next synchronisation.
 *  - No global mutable state: the functions are thread-safe and re-entrant.
 *  - Values are not checked: NaN or Inf in the inputs propagate to the
 *    outputs of the affected (b, h) sequence only.
 *  - Nothing is written when validation fails.
 */
#ifndef GDN_H
#define GDN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    GDN_OK = 0,
    GDN_ERR_NULL_ARG = 1,     /* a required pointer is NULL                   */
    GDN_ERR_BAD_SHAPE = 2,    /* B, H, T < 1, or a dimension out of range     */
    GDN_ERR_BAD_DTYPE = 3,    /* dtype code not one of gdn_dtype              */
    GDN_ERR_UNSUPPORTED = 4,  /* valid but not built: e.g. chunk/d_k/dtype mix */
    GDN_ERR_WORKSPACE = 5,    /* workspace smaller than the query returned    */
    GDN_ERR_HIP = 6           /* the HIP runtime reported an error            */
} gdn_status;

typedef enum { GDN_BF16 = 0, GDN_F32 = 1 } gdn_dtype;

typedef struct {
    int32_t B, H, T;          /* batch, heads, sequence length (T >= 1)        */
    int32_t d_k, d_v;         /* key/query and value head dimensions           */
    int32_t chunk_size;       /* C: tokens per chunk                           */
    int32_t qkv_dtype;        /* gdn_dtype of q, k and v (one dtype for all)   */
    int32_t o_dtype;          /* gdn_dtype of O (GDN_F32 recommended)          */
} gdn_shape;

/*
 * Supported combinations (anything else that is well-formed returns
 * GDN_ERR_UNSUPPORTED):
 *   chunk_size in {16, 32, 64};
 *   qkv_dtype GDN_BF16: d_k in {16, 32, 64, 96, 128, 256} (d_k 16 runs on
 *                       the d_k 32 kernel with the keys and queries padded
 *                       with zeros as they are staged: the MFMAs take 32
 *                       elements per k-step; no sequence-parallel segments);
 *   qkv_dtype GDN_F32:  d_k in {16, 32, 64, 128, 256};
 *   at d_k 256 a chunk of 64 tokens is computed as two chunks of 32 (its
 *   64-token tiles would need more than the 160 KB of LDS of one compute
 *   unit): the same recurrence grouped differently, so the same result up
 *   to rounding (gdn_chunk_fwd_stages, whose T is laid out per chunk, and
 *   gdn_chunk_prep reject that case);
 *   d_v a multiple of 16 in [16, 1024]; one head's largest tensor (T x
 *   max(d_k, d_v) x 4 bytes) below 2 GiB.
 * T may be any value >= 1; a last chunk shorter than chunk_size is handled
 * exactly (padding tokens are identity transitions).
 *
 * Arithmetic.  bf16 inputs run one fused kernel whose matrix products take
 * fp16 operands (11 significant bits; bf16 inputs convert exactly) with fp32
 * accumulation and an fp32 state: against the exact result the normwise
 * error is near 6e-4 on gated workloads.  Operands must stay inside the fp16
 * range (|x| < 65504; the state and the values are the ones that grow).
 * Without decay and with beta near 2 (reflections) the state keeps every
 * rounding, so the error grows with the number of chunks; gdn_chunk_fwd_precise
 * then keeps it near 1e-5.  f32 inputs use fp32 matrix products throughout.
 */

/*
 * Bytes of device workspace gdn_chunk_fwd (and gdn_chunk_fwd_eta) needs for
 * this shape on the current device: 0 unless the call takes the
 * sequence-parallel form (see gdn_chunk_fwd_seq), which it does for bf16
 * inputs when the heads and value tiles would leave compute units idle (few
 * heads, long sequences).  Returns (size_t)-1 if the shape is invalid or
 * unsupported.
 */
size_t gdn_chunk_fwd_workspace_bytes(const gdn_shape* s);

/*
 * Chunkwise-parallel forward pass.  Layouts:
 *   q, k     [B, H, T, d_k]   qkv_dtype   (k rows are usually L2-normalised
 *                                          by the caller; not required)
 *   v        [B, H, T, d_v]   qkv_dtype
 *   alpha    [B, H, T] float, gate in (0, 1]; NULL means alpha = 1 (no gate).
 *            alpha <= 0 is outside the method (its logarithm is used).
 *   beta     [B, H, T] float, any finite value (the pages use (0, 2)).
 *   S0       [B, H, d_v, d_k] float initial state; NULL means zero.
 *   O        [B, H, T, d_v]   o_dtype, written.
 *   S_final  [B, H, d_v, d_k] float, written; may be the same pointer as S0
 *            (the state is updated in place).
 * workspace / workspace_bytes: at least gdn_chunk_fwd_workspace_bytes(s)
 * bytes of device memory (may be NULL when that is 0).
 */
gdn_status gdn_chunk_fwd(const gdn_shape* s,
                         const void* q, const void* k, const void* v,
                         const float* alpha, const float* beta, const float* S0,
                         void* O, float* S_final,
                         void* workspace, size_t workspace_bytes,
                         void* stream);

/*
 * The same pass with a separate write strength eta ("RNN的复兴03", section 1:
 * erase strength beta, write strength eta):
 *     S_t = alpha_t S_{t-1} (I - beta_t k_t k_t^T) + eta_t v_t k_t^T.
 * eta [B, H, T] float, any finite value; NULL means eta = beta, which is
 * exactly gdn_chunk_fwd.  beta = 0, eta = 1 gives gated linear attention
 * ("从电路复杂性理论的角度分析大模型的可并行性和表达能力", GLA).
 * Everything else as gdn_chunk_fwd.
 */
gdn_status gdn_chunk_fwd_eta(const gdn_shape* s,
                             const void* q, const void* k, const void* v,
                             const float* alpha, const float* beta, const float* eta,
                             const float* S0, void* O, float* S_final,
                             void* workspace, size_t workspace_bytes,
                             void* stream);

/*
 * gdn_chunk_fwd_eta with the sequence-parallel form chosen by the caller.
 * The state recurrence is linear in the state, so it is associative and can
 * be evaluated by a parallel scan ("Параллельность RNN?", section
 * "Уровень 2"); the chunk form already passes each chunk's end state to the
 * next ("从零开始的 GDN 推导", 总结).  Each sequence is cut into segments of
 * seg_chunks chunks (the last one shorter).  All segments run at once: the
 * first from S0; every later one from a zero state, together with the d_k
 * rows of its transition M = A_first ... A_last (A_t = alpha_t (I - beta_t
 * k_t k_t^T)) started from the identity, whose outputs are the queries
 * carried through the segment, qm_t = A_first ... A_t q_t.  A combine over
 * segments (X_{j+1} = X_j M_j + E_j, E_j the end state from zero) and a
 * correction o_t += X_j qm_t finish the pass.  Results equal those of the
 * plain form up to rounding (the combine and the correction multiply
 * split-bf16 operands, about 16 significant bits, with fp32 accumulation).
 *   seg_chunks  0: the form and segment length gdn_chunk_fwd would choose;
 *               >= 1: segments of that many chunks (one segment, i.e.
 *               seg_chunks >= ceil(T / chunk_size), is the plain form);
 *               < 0: GDN_ERR_BAD_SHAPE.  More than one segment needs bf16
 *               inputs (else GDN_ERR_UNSUPPORTED).
 * workspace: at least gdn_chunk_fwd_seq_workspace_bytes(s, seg_chunks)
 * bytes of device memory, 256-byte aligned (GDN_ERR_WORKSPACE if smaller or
 * NULL when needed).  After the call it holds, from offset 0,
 *   [B*H][n_seg][d_v + d_k][d_k] float: rows 0..d_v-1 of segment j: its end
 *     state from a zero state (segment 0: from S0); rows d_v.. : M_j
 *     transposed, row c holding M_j[0..d_k-1][c] (segments >= 1);
 *   then, at the next multiple of 256 bytes, [B*H*T][d_k] float: qm_t for
 *     the tokens of segments >= 1;
 *   then (bf16 O only) [B*H*T][d_v] float: outputs from a zero state.
 * Everything else as gdn_chunk_fwd_eta.
 */
size_t gdn_chunk_fwd_seq_workspace_bytes(const gdn_shape* s, int seg_chunks);
gdn_status gdn_chunk_fwd_seq(const gdn_shape* s, int seg_chunks,
                             const void* q, const void* k, const void* v,
                             const float* alpha, const float* beta, const float* eta,
                             const float* S0, void* O, float* S_final,
                             void* workspace, size_t workspace_bytes,
                             void* stream);

/*
 * gdn_chunk_fwd_seq without a workspace argument, for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving
 * loops, harnesses that forbid allocation): the workspace is a 64 MiB
 * (67108864-byte) device array inside the library, one copy per GPU,
 * looked up on the first call on each device and held until the process
 * ends.  The call allocates nothing.  Plans whose workspace
 * (gdn_chunk_fwd_seq_workspace_bytes) exceeds 64 MiB return
 * GDN_ERR_WORKSPACE and write nothing.  Nothing in the array needs to start
 * at zero (every byte a call reads was written earlier in the same call),
 * and it keeps the last call's contents.  Calls that overlap on one GPU
 * (two streams, two threads) share that array and race: serialize them.
 * Runs on the current device.  Everything else as gdn_chunk_fwd_seq.
 */
gdn_status gdn_chunk_fwd_seq_noalloc(const gdn_shape* s, int seg_chunks,
                                     const void* q, const void* k, const void* v,
                                     const float* alpha, const float* beta, const float* eta,
                                     const float* S0, void* O, float* S_final,
                                     void* stream);

/*
 * The same pass with bf16 inputs through the split-bf16 kernels: every
 * derived matrix-product operand is a pair of bf16 numbers (hi + lo, about
 * 16 significant bits), which keeps the normwise error near 1e-5 whatever
 * the gates, at roughly twice the run time of gdn_chunk_fwd.  Shapes: bf16
 * with chunk_size in {32, 64} and d_k in {64, 128} take the pipelined
 * split kernel, bf16 d_k 32 and all f32 shapes the generic one (the other
 * bf16 shapes, chunk_size 16 or d_k 16 / 96 / 256, return GDN_ERR_UNSUPPORTED).
 * eta may
 * be NULL (eta = beta).  Arguments and conventions as gdn_chunk_fwd_eta,
 * without a workspace.
 */
gdn_status gdn_chunk_fwd_precise(const gdn_shape* s,
                                 const void* q, const void* k, const void* v,
                                 const float* alpha, const float* beta, const float* eta,
                                 const float* S0, void* O, float* S_final,
                                 void* stream);

/*
 * gdn_chunk_fwd_eta (bf16 inputs only) with two intermediates of the kernel
 * written out, for stage-by-stage checks of the pass itself:
 *   T_out  [B, H, NT, C, C] float: T = (I - A)^{-1} of every chunk as the
 *          kernel holds it (fp16 values, NT = ceil(T / C); zero above the
 *          diagonal and, in a ragged last chunk, identity past its end);
 *          A strictly lower with A_ri = -beta_r exp(g_r - g_i) k_r.k_i
 *          ("从零开始的 GDN 推导", UT transform, with L = -A);
 *   Vp_out [B, H, T, d_v] float: the pseudo-values V' = U - W S^T of every
 *          chunk ("从零开始的 GDN 推导", S update), before their rounding to
 *          the fp16 operands of the output and state products.
 * Either may be NULL.  O and S_final are written as by gdn_chunk_fwd_eta.
 * Shapes: bf16 as for gdn_chunk_fwd; f32 inputs return GDN_ERR_UNSUPPORTED.
 */
gdn_status gdn_chunk_fwd_stages(const gdn_shape* s,
                                const void* q, const void* k, const void* v,
                                const float* alpha, const float* beta, const float* eta,
                                const float* S0, void* O, float* S_final,
                                float* T_out, float* Vp_out,
                                void* stream);

/*
 * Chunk-local quantities of the same method, for inspection and testing of
 * the intermediate stages.  For every chunk c (NT = ceil(T / C) chunks, the
 * last one zero-padded to C tokens):
 *   T_out  [B, H, NT, C, C] float: T = (I - A)^{-1}, A strictly lower with
 *          A_ri = -beta_r exp(g_r - g_i) k_r.k_i (i < r), g the chunk-local
 *          inclusive cumulative sum of log alpha ("从零开始的 GDN 推导",
 *          UT transform, with L = -A);
 *   W_out  [B, H, T, d_k] float: W = T diag(beta) diag(exp(g)) K;
 *   U_out  [B, H, T, d_v] float: U = T diag(beta) V ("S 的推导").
 * Any of the three output pointers may be NULL (that output is skipped).
 * Computed by the generic stage kernel (fp32 solve, split-bf16 products):
 * bf16 with chunk_size in {32, 64} and d_k in {32, 64, 128}, f32 as for
 * gdn_chunk_fwd; other shapes return GDN_ERR_UNSUPPORTED.
 */
gdn_status gdn_chunk_prep(const gdn_shape* s,
                          const void* k, const void* v,
                          const float* alpha, const float* beta,
                          float* T_out, float* W_out, float* U_out,
                          void* workspace, size_t workspace_bytes,
                          void* stream);

/*
 * Recurrent (token-by-token) forward pass: the same recurrence applied one
 * token at a time ("从零开始的 GDN 推导", recurrent form; "RNN的复兴03",
 * section 1), for short sequences such as a decode step appended to a
 * chunked prefill.  The state is read once, kept on chip for all T tokens
 * and written once, so for T = 1 the cost is one pass of the state through
 * HBM.  Same tensors, layouts and conventions as gdn_chunk_fwd:
 *   q, k [B, H, T, d_k], v [B, H, T, d_v] (qkv_dtype), alpha (NULL = 1) and
 *   beta [B, H, T] float, S0 [B, H, d_v, d_k] float (NULL = zero),
 *   O [B, H, T, d_v] (o_dtype), S_final [B, H, d_v, d_k] float; S_final may
 *   be the same pointer as S0 (in-place update), other overlaps are not
 *   allowed.  chunk_size is ignored.
 * Supported: qkv_dtype GDN_BF16 or GDN_F32; d_k in {16, 32, 64, 96, 128,
 * 192, 256}; 1 <= d_v <= 65536; any T >= 1 (the work is serial in T, so long
 * sequences belong to gdn_chunk_fwd).  Pointers 16-byte aligned.  Errors are
 * returned before any launch, as for gdn_chunk_fwd.
 */
gdn_status gdn_recurrent_fwd(const gdn_shape* s,
                             const void* q, const void* k, const void* v,
                             const float* alpha, const float* beta, const float* S0,
                             void* O, float* S_final,
                             void* stream);

/* gdn_recurrent_fwd with a separate write strength eta (NULL means
 * eta = beta), as for gdn_chunk_fwd_eta. */
gdn_status gdn_recurrent_fwd_eta(const gdn_shape* s,
                                 const void* q, const void* k, const void* v,
                                 const float* alpha, const float* beta, const float* eta,
                                 const float* S0, void* O, float* S_final,
                                 void* stream);

/* Static text for a status code. */
const char* gdn_status_string(gdn_status st);

/* Text of the last error on the calling thread (HIP error string or the
 * reason a shape was rejected); "" if none.  Valid until the next call. */
const char* gdn_last_error(void);

/* Library version: major * 10000 + minor * 100 + patch. */
int32_t gdn_version(void);

#ifdef __cplusplus
}
#endif

#endif /* GDN_H */
