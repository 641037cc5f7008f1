// fp8 (E4M3FN) instantiations of the implicit-GEMM conv kernel.
#include "conv_igemm.h"

namespace igc {
hipError_t launch_conv_fp8(const ConvParams &p, int tile, Mode mode, bool big, bool cblock, hipStream_t stream)
{
    return launch_conv_dt<DT_FP8>(p, tile, mode, big, cblock, stream);
}
}  // namespace igc
