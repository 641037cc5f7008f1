// Direct-to-LDS conv kernel instantiations: fp8, 64-byte steps (32x32 MFMA blocks): 256x256 and 128x128 tiles.
#include "conv_igemm_dma.h"

namespace igc {
IGC_DMA_INSTANTIATE(DT_FP8, 7);
IGC_DMA_INSTANTIATE(DT_FP8, 9);
IGC_DMA_INSTANTIATE(DT_FP8, 12);
}  // namespace igc
