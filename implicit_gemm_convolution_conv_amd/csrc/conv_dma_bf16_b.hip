// Direct-to-LDS conv kernel instantiations: bf16, 64-byte steps: 8-stage, 64x64, 256x128 and 128x256 tiles.
#include "conv_igemm_dma.h"

namespace igc {
IGC_DMA_INSTANTIATE(DT_BF16, 10);
IGC_DMA_INSTANTIATE(DT_BF16, 11);
IGC_DMA_INSTANTIATE(DT_BF16, 18);
IGC_DMA_INSTANTIATE(DT_BF16, 19);
IGC_DMA_INSTANTIATE(DT_BF16, 20);
}  // namespace igc
