// Global-address direct-to-LDS conv kernel instantiations, fp8-e4m3: 128x128 and 64x64 tiles.
#include "conv_igemm_dma.h"

namespace igc {
IGC_DMA_INSTANTIATE(DT_FP8, TILE_DMA_128);
IGC_DMA_INSTANTIATE(DT_FP8, TILE_DMA_64);
}  // namespace igc
