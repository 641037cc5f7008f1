// bf16 instantiations of the buffer-addressed direct-to-LDS implicit-GEMM conv kernels.
#include "conv_igemm_pp.h"

namespace igc {
hipError_t launch_conv_buf_bf16(const ConvParams &p, int tile, Mode mode, hipStream_t stream)
{
    if (tile == TILE_BUF_PINGPONG)
        return launch_conv_pp<DT_BF16>(p, mode, stream);
    return launch_conv_buf_dt<DT_BF16>(p, tile, mode, stream);
}
}  // namespace igc
