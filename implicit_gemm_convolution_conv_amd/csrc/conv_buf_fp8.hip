// fp8-e4m3 instantiations of the buffer-addressed direct-to-LDS implicit-GEMM conv kernels.
#include "conv_igemm_ppw.h"

namespace igc {
hipError_t launch_conv_buf_fp8(const ConvParams &p, int tile, Mode mode, hipStream_t stream)
{
    if (tile == 33)
        return launch_conv_pp<DT_FP8>(p, mode, stream);
    if (tile == 34)
        return launch_conv_ppw<DT_FP8>(p, stream);
    return launch_conv_buf_dt<DT_FP8>(p, tile, mode, stream);
}
}  // namespace igc
