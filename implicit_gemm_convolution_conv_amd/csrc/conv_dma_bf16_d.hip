// Direct-to-LDS conv kernel instantiations: bf16, 128-byte steps: 256x256 and 4-stage 128x128 tiles.
#include "conv_igemm_dma.h"

namespace igc {
IGC_DMA_INSTANTIATE(DT_BF16, 21);
IGC_DMA_INSTANTIATE(DT_BF16, 22);
IGC_DMA_INSTANTIATE(DT_BF16, 23);
}  // namespace igc
