// bf16 instantiations of the buffer-addressed direct-to-LDS implicit-GEMM conv kernel.
#include "conv_igemm_buf.h"

namespace igc {
hipError_t launch_conv_buf_bf16(const ConvParams &p, int tile, Mode mode, hipStream_t stream)
{
    return launch_conv_buf_dt<DT_BF16>(p, tile, mode, stream);
}
}  // namespace igc
