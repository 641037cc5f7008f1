// Direct-to-LDS conv kernel instantiations: bf16, 64-byte steps: 4-wave 256x256 tiles.
#include "conv_igemm_dma.h"

namespace igc {
IGC_DMA_INSTANTIATE(DT_BF16, 14);
IGC_DMA_INSTANTIATE(DT_BF16, 15);
}  // namespace igc
