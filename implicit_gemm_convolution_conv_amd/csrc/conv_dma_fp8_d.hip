// Direct-to-LDS conv kernel instantiations: fp8, 128-byte steps: 128x128, 256x128 and 64x64 tiles.
#include "conv_igemm_dma.h"

namespace igc {
IGC_DMA_INSTANTIATE(DT_FP8, 24);
IGC_DMA_INSTANTIATE(DT_FP8, 25);
IGC_DMA_INSTANTIATE(DT_FP8, 26);
}  // namespace igc
