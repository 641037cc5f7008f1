// Global-address direct-to-LDS conv kernel instantiations, bf16: 256x256 and 256x192 tiles.
#include "conv_igemm_dma.h"

namespace igc {
IGC_DMA_INSTANTIATE(DT_BF16, TILE_DMA_256);
IGC_DMA_INSTANTIATE(DT_BF16, TILE_DMA_256x192);
}  // namespace igc
