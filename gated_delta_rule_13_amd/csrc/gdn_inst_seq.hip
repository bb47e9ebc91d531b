// gdn_inst_seq.hip -- instantiations of the finishing kernel of a
// sequence-parallel run.
#include "gdn_launch.h"
#include "gdn_seq.h"

namespace gdn {
namespace {
template <int DK>
void launch(const SeqParams& p, hipStream_t st) {
    // units (head, segment >= 1, token group) padded to a multiple of 8,
    // d_v / 16 row blocks each
    const long ngps = (p.seg_len + FinishShape<DK>::G - 1) / FinishShape<DK>::G;
    const long units = (long)p.BH * (p.nseg - 1) * ngps;
    const long nblocks = (units + 7) / 8 * 8 * (p.dv / 16);
    hipLaunchKernelGGL((gdn_seq_finish_kernel<DK>), dim3((unsigned)nblocks), dim3(256), 0, st, p);
}
}  // namespace

SeqLauncher seq_launcher(int dk) {
    switch (dk) {
        case 32: return launch<32>;
        case 64: return launch<64>;
        case 96: return launch<96>;
        case 128: return launch<128>;
        case 256: return launch<256>;
    }
    return nullptr;
}
}  // namespace gdn
