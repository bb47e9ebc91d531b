// gdn_inst_generic.hip -- instantiations of the generic fused kernel and of
// its stage kernel (T, W, U per chunk), for bf16 inputs when built with
// GDN_GEN_BF16=1 and for fp32 inputs when built with GDN_GEN_BF16=0.
#include "gdn_kernels.h"
#include "gdn_launch.h"

namespace gdn {
namespace {
template <int C, int DK, int NW, bool BF>
void launch_fwd(const FwdParams& p, long nblocks, hipStream_t st) {
    hipLaunchKernelGGL((gdn_fwd_kernel<C, DK, NW, BF>), dim3((unsigned)nblocks), dim3(NW * 64), 0, st, p);
}
template <int C, int DK, int NW, bool BF>
void launch_prep(const FwdParams& p, long nblocks, hipStream_t st) {
    hipLaunchKernelGGL((gdn_prep_kernel<C, DK, NW, BF>), dim3((unsigned)nblocks), dim3(NW * 64), 0, st, p);
}
template <int C, int DK, bool BF>
FwdLauncher pick_nw(int nw, bool prep) {
    switch (nw) {
        case 1: return prep ? launch_prep<C, DK, 1, BF> : launch_fwd<C, DK, 1, BF>;
        case 2: return prep ? launch_prep<C, DK, 2, BF> : launch_fwd<C, DK, 2, BF>;
        default: return prep ? launch_prep<C, DK, 4, BF> : launch_fwd<C, DK, 4, BF>;
    }
}
}  // namespace

#if !defined(GDN_GEN_BF16)
#error "build with -DGDN_GEN_BF16=1 (bf16 inputs) or -DGDN_GEN_BF16=0 (fp32 inputs)"
#endif
#if GDN_GEN_BF16
FwdLauncher generic_launcher_bf16(int C, int DK, int nw, bool prep) {
    if (C == 64 && DK == 128) return pick_nw<64, 128, true>(nw, prep);
    if (C == 64 && DK == 64) return pick_nw<64, 64, true>(nw, prep);
    if (C == 64 && DK == 32) return pick_nw<64, 32, true>(nw, prep);
    if (C == 32 && DK == 128) return pick_nw<32, 128, true>(nw, prep);
    if (C == 32 && DK == 64) return pick_nw<32, 64, true>(nw, prep);
    if (C == 32 && DK == 32) return pick_nw<32, 32, true>(nw, prep);
    return nullptr;
}
#else
FwdLauncher generic_launcher_f32(int C, int DK, int nw, bool prep) {
    if (C == 64 && DK == 128) return pick_nw<64, 128, false>(nw, prep);
    if (C == 64 && DK == 64) return pick_nw<64, 64, false>(nw, prep);
    if (C == 64 && DK == 32) return pick_nw<64, 32, false>(nw, prep);
    if (C == 64 && DK == 16) return pick_nw<64, 16, false>(nw, prep);
    if (C == 32 && DK == 256) return pick_nw<32, 256, false>(nw, prep);
    if (C == 32 && DK == 128) return pick_nw<32, 128, false>(nw, prep);
    if (C == 32 && DK == 64) return pick_nw<32, 64, false>(nw, prep);
    if (C == 32 && DK == 32) return pick_nw<32, 32, false>(nw, prep);
    if (C == 32 && DK == 16) return pick_nw<32, 16, false>(nw, prep);
    if (C == 16 && DK == 256) return pick_nw<16, 256, false>(nw, prep);
    if (C == 16 && DK == 128) return pick_nw<16, 128, false>(nw, prep);
    if (C == 16 && DK == 64) return pick_nw<16, 64, false>(nw, prep);
    if (C == 16 && DK == 32) return pick_nw<16, 32, false>(nw, prep);
    if (C == 16 && DK == 16) return pick_nw<16, 16, false>(nw, prep);
    return nullptr;
}
#endif
}  // namespace gdn
