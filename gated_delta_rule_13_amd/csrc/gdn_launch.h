// gdn_launch.h -- host-side launchers of the kernel instantiations.  Each
// kernel family is instantiated in a translation unit of its own
// (gdn_inst_*.hip) so that the library builds in parallel; the C ABI in
// gdn_api.hip only validates, picks a launcher and calls it.
#pragma once
#include <hip/hip_runtime.h>

#include "gdn_kernels.h"
#include "gdn_recurrent.h"
#include "gdn_seq.h"

namespace gdn {

using FwdLauncher = void (*)(const FwdParams&, long nblocks, hipStream_t);
using RecLauncher = void (*)(const RecParams&, long nblocks, hipStream_t);
using SeqLauncher = void (*)(const SeqParams&, hipStream_t);

// fp16-operand fused kernel (bf16 inputs): C in {16, 32, 64}, d_k in
// {16, 32, 64, 96, 128} (and 256 with C <= 32), ns scan waves in {1, 2, 3, 4};
// seg: the sequence-parallel launch (ns = 1 only).  Null when the shape is
// not built.  One definition per (C, d_k), in the object built from
// gdn_inst_fast.hip with that pair.
FwdLauncher fast_launcher(int C, int dk, int ns, bool eta, bool seg);
#define GDN_FAST_DECL(CC, KK) FwdLauncher fast_launcher_c##CC##_d##KK(int ns, bool eta, bool seg);
GDN_FAST_DECL(16, 16)
GDN_FAST_DECL(32, 16)
GDN_FAST_DECL(64, 16)
GDN_FAST_DECL(16, 32)
GDN_FAST_DECL(16, 64)
GDN_FAST_DECL(16, 96)
GDN_FAST_DECL(16, 128)
GDN_FAST_DECL(16, 256)
GDN_FAST_DECL(32, 32)
GDN_FAST_DECL(32, 64)
GDN_FAST_DECL(32, 96)
GDN_FAST_DECL(32, 128)
GDN_FAST_DECL(32, 256)
GDN_FAST_DECL(64, 32)
GDN_FAST_DECL(64, 64)
GDN_FAST_DECL(64, 96)
GDN_FAST_DECL(64, 128)
#undef GDN_FAST_DECL

// split-bf16 pipelined kernel (bf16 inputs, errors near 1e-5): C in {32, 64},
// d_k in {64, 128}.
FwdLauncher pipe_launcher(int C, int dk, int ns, bool eta);

// generic fused kernel (fp32 inputs, and bf16 shapes the others do not
// cover) and its stage kernel (T, W, U).
FwdLauncher generic_launcher_bf16(int C, int dk, int nw, bool prep);
FwdLauncher generic_launcher_f32(int C, int dk, int nw, bool prep);
inline FwdLauncher generic_launcher(int C, int dk, int nw, bool bf16, bool prep) {
    return bf16 ? generic_launcher_bf16(C, dk, nw, prep) : generic_launcher_f32(C, dk, nw, prep);
}

// finishing kernel of a sequence-parallel run of the fused kernel (the
// combine over segments and the correction of the later segments'
// outputs): d_k in {32, 64, 96, 128, 256}.
SeqLauncher seq_launcher(int dk);

// token-by-token kernel; *rows_per_block receives the state rows one
// workgroup covers.
RecLauncher rec_launcher(int dk, bool bf16, int* rows_per_block);

}  // namespace gdn
