// gdn_inst_rec.hip -- instantiations of the token-by-token kernel.
#include "gdn_launch.h"
#include "gdn_recurrent.h"

namespace gdn {
namespace {
template <int DK, bool BF>
void launch(const RecParams& p, long nblocks, hipStream_t st) {
    hipLaunchKernelGGL((gdn_recurrent_kernel<DK, BF>), dim3((unsigned)nblocks), dim3(kRecThreads), 0, st, p);
}
}  // namespace

RecLauncher rec_launcher(int dk, bool bf, int* rows_per_block) {
#define GDN_REC(D)                                                                   \
    if (dk == D) {                                                                   \
        *rows_per_block = kRecRows * (kRecThreads / 64) * (64 / rec_lanes_per_row(D)); \
        return bf ? launch<D, true> : launch<D, false>;                              \
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
}  // namespace gdn
