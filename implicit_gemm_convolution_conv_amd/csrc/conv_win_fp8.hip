// fp8 instantiations of the input-window implicit-GEMM conv kernel.
#include "conv_igemm_win.h"

namespace igc {
hipError_t launch_conv_win_fp8(const ConvParams &p, int tile, bool big, hipStream_t stream)
{
    return launch_conv_win_dt<DT_FP8>(p, tile, big, stream);
}
}  // namespace igc
