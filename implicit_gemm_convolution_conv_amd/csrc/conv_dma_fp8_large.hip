// Global-address direct-to-LDS conv kernel instantiations, fp8-e4m3: 256x256 tile.
#include "conv_igemm_dma.h"

namespace igc {
IGC_DMA_INSTANTIATE(DT_FP8, TILE_DMA_256);
}  // namespace igc
