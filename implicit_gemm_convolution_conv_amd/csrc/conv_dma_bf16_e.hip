// Direct-to-LDS conv kernel instantiations: bf16, 128-byte steps: 128x128, 256x128 and 64x64 tiles.
#include "conv_igemm_dma.h"

namespace igc {
IGC_DMA_INSTANTIATE(DT_BF16, 24);
IGC_DMA_INSTANTIATE(DT_BF16, 25);
IGC_DMA_INSTANTIATE(DT_BF16, 26);
IGC_DMA_INSTANTIATE(DT_BF16, 40);
}  // namespace igc
