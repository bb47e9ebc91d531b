// gdn_inst_fast.hip -- instantiations of the fp16-operand fused kernel for
// one (chunk, d_k) pair, given on the command line as GDN_C and GDN_DK.
#include "gdn_fast.h"
#include "gdn_launch.h"

#if !defined(GDN_C) || !defined(GDN_DK)
#error "build with -DGDN_C=<chunk> -DGDN_DK=<d_k>"
#endif
// d_k 16 runs on the d_k 32 kernel with the keys and queries zero-padded
#if GDN_DK == 16
#define GDN_DKK 32
#else
#define GDN_DKK GDN_DK
#endif

#define GDN_NAME2(CC, KK) fast_launcher_c##CC##_d##KK
#define GDN_NAME(CC, KK) GDN_NAME2(CC, KK)

namespace gdn {
namespace {
template <int NS, bool ETA, bool SEG>
void launch(const FwdParams& p, long nblocks, hipStream_t st) {
    hipLaunchKernelGGL((gdn_fwd_fast_kernel<GDN_C, GDN_DKK, NS, ETA, SEG, GDN_DK>), dim3((unsigned)nblocks),
                       dim3((NS + fast_prep_waves(NS, GDN_C, GDN_DKK)) * 64), 0, st, p);
}
}  // namespace

// (the sequence-parallel form runs one scan wave per workgroup only)
FwdLauncher GDN_NAME(GDN_C, GDN_DK)(int ns, bool eta, bool seg) {
#if GDN_DK == 16
    if (seg) return nullptr;   // (segments need d_k >= 32)
#else
    if (seg) return ns == 1 ? (eta ? launch<1, true, true> : launch<1, false, true>) : nullptr;
#endif
    switch (ns) {
        case 1: return eta ? launch<1, true, false> : launch<1, false, false>;
        case 2: return eta ? launch<2, true, false> : launch<2, false, false>;
        case 3: return eta ? launch<3, true, false> : launch<3, false, false>;
        case 4: return eta ? launch<4, true, false> : launch<4, false, false>;
    }
    return nullptr;
}
}  // namespace gdn
