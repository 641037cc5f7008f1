// Direct-to-LDS conv kernel instantiations: fp8, 128-byte steps: 256x256 and 4-stage 128x128 tiles.
#include "conv_igemm_dma.h"

namespace igc {
IGC_DMA_INSTANTIATE(DT_FP8, 21);
IGC_DMA_INSTANTIATE(DT_FP8, 22);
IGC_DMA_INSTANTIATE(DT_FP8, 23);
}  // namespace igc
