// Direct-to-LDS conv kernel instantiations: bf16, 64-byte steps: 256x256 and 128x128 tiles.
#include "conv_igemm_dma.h"

namespace igc {
IGC_DMA_INSTANTIATE(DT_BF16, 6);
IGC_DMA_INSTANTIATE(DT_BF16, 7);
IGC_DMA_INSTANTIATE(DT_BF16, 8);
IGC_DMA_INSTANTIATE(DT_BF16, 9);
}  // namespace igc
