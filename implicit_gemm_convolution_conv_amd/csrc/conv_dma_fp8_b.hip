// Direct-to-LDS conv kernel instantiations: fp8, 64-byte steps (32x32 MFMA blocks): 64x64, 4-wave 256x256 and 256x128 tiles.
#include "conv_igemm_dma.h"

namespace igc {
IGC_DMA_INSTANTIATE(DT_FP8, 13);
IGC_DMA_INSTANTIATE(DT_FP8, 15);
IGC_DMA_INSTANTIATE(DT_FP8, 19);
}  // namespace igc
