// bf16 instantiations of the buffer-addressed direct-to-LDS implicit-GEMM conv kernels.
#include "conv_igemm_ppw.h"

namespace igc {
hipError_t launch_conv_buf_bf16(const ConvParams &p, int tile, Mode mode, hipStream_t stream)
{
    if (tile == 33)
        return launch_conv_pp<DT_BF16>(p, mode, stream);
    if (tile == 34)
        return launch_conv_ppw<DT_BF16>(p, stream);
    return launch_conv_buf_dt<DT_BF16>(p, tile, mode, stream);
}
}  // namespace igc
