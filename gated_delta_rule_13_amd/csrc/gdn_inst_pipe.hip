// gdn_inst_pipe.hip -- instantiations of the split-bf16 pipelined kernel.
#include "gdn_launch.h"
#include "gdn_pipe.h"

namespace gdn {
namespace {
template <int C, int DK, int NS>
void launch(const FwdParams& p, long nblocks, hipStream_t st) {
    if (p.eta)
        hipLaunchKernelGGL((gdn_fwd_pipe_kernel<C, DK, NS, true>), dim3((unsigned)nblocks),
                           dim3((NS + kPrepWaves) * 64), 0, st, p);
    else
        hipLaunchKernelGGL((gdn_fwd_pipe_kernel<C, DK, NS, false>), dim3((unsigned)nblocks),
                           dim3((NS + kPrepWaves) * 64), 0, st, p);
}
}  // namespace

FwdLauncher pipe_launcher(int C, int dk, int ns, bool eta) {
    (void)eta;   // the launcher picks the instantiation from p.eta
#define GDN_PIPE(CC, KK)                                                            \
    if (C == CC && dk == KK)                                                        \
        return ns == 4 ? launch<CC, KK, 4> : ns == 2 ? launch<CC, KK, 2> : launch<CC, KK, 1>;
    GDN_PIPE(64, 128)
    GDN_PIPE(64, 64)
    GDN_PIPE(32, 128)
    GDN_PIPE(32, 64)
#undef GDN_PIPE
    return nullptr;
}
}  // namespace gdn
