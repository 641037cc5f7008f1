// fp8 instantiations of the direct-to-LDS implicit-GEMM conv kernel.
#include "conv_igemm_dma.h"

namespace igc {
hipError_t launch_conv_dma_fp8(const ConvParams &p, int tile, Mode mode, bool big, bool cblock, hipStream_t stream)
{
    return launch_conv_dma_dt<DT_FP8>(p, tile, mode, big, cblock, stream);
}
}  // namespace igc
