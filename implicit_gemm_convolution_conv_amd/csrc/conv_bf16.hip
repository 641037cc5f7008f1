// bf16 instantiations of the implicit-GEMM conv kernel.
#include "conv_igemm.h"

namespace igc {
hipError_t launch_conv_bf16(const ConvParams &p, int tile, Mode mode, bool big, bool cblock, hipStream_t stream)
{
    return launch_conv_dt<DT_BF16>(p, tile, mode, big, cblock, stream);
}
}  // namespace igc
