// bf16 instantiations of the input-window implicit-GEMM conv kernel.
#include "conv_igemm_win.h"

namespace igc {
hipError_t launch_conv_win_bf16(const ConvParams &p, int tile, bool big, hipStream_t stream)
{
    return launch_conv_win_dt<DT_BF16>(p, tile, big, stream);
}
}  // namespace igc
