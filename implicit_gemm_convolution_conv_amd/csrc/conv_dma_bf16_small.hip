// Global-address direct-to-LDS conv kernel instantiations, bf16: 128x128 and 64x64 tiles.
#include "conv_igemm_dma.h"

namespace igc {
IGC_DMA_INSTANTIATE(DT_BF16, TILE_DMA_128);
IGC_DMA_INSTANTIATE(DT_BF16, TILE_DMA_64);
}  // namespace igc
