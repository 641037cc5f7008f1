// Dispatch of the direct-to-LDS conv kernel on the tile index. The tiles are
// instantiated in the conv_dma_{bf16,fp8}_*.hip units, a few per unit, so the
// units compile in parallel; the declarations below keep this unit from
// instantiating them again.
#include "conv_igemm_dma.h"

namespace igc {

IGC_DMA_EXTERN(DT_BF16, TILE_DMA_256);
IGC_DMA_EXTERN(DT_BF16, TILE_DMA_128);
IGC_DMA_EXTERN(DT_BF16, TILE_DMA_64);
IGC_DMA_EXTERN(DT_BF16, TILE_DMA_256x192);
IGC_DMA_EXTERN(DT_FP8, TILE_DMA_256);
IGC_DMA_EXTERN(DT_FP8, TILE_DMA_128);
IGC_DMA_EXTERN(DT_FP8, TILE_DMA_64);

hipError_t launch_conv_dma_bf16(const ConvParams &p, int tile, Mode mode, bool big, bool cblock, hipStream_t stream)
{
    switch (tile) {
    case TILE_DMA_256: return launch_conv_dma_tile<DT_BF16, TILE_DMA_256>(p, mode, big, cblock, stream);
    case TILE_DMA_128: return launch_conv_dma_tile<DT_BF16, TILE_DMA_128>(p, mode, big, cblock, stream);
    case TILE_DMA_64: return launch_conv_dma_tile<DT_BF16, TILE_DMA_64>(p, mode, big, cblock, stream);
    case TILE_DMA_256x192: return launch_conv_dma_tile<DT_BF16, TILE_DMA_256x192>(p, mode, big, cblock, stream);
    default: return hipErrorInvalidValue;
    }
}

hipError_t launch_conv_dma_fp8(const ConvParams &p, int tile, Mode mode, bool big, bool cblock, hipStream_t stream)
{
    switch (tile) {
    case TILE_DMA_256: return launch_conv_dma_tile<DT_FP8, TILE_DMA_256>(p, mode, big, cblock, stream);
    case TILE_DMA_128: return launch_conv_dma_tile<DT_FP8, TILE_DMA_128>(p, mode, big, cblock, stream);
    case TILE_DMA_64: return launch_conv_dma_tile<DT_FP8, TILE_DMA_64>(p, mode, big, cblock, stream);
    default: return hipErrorInvalidValue;
    }
}

}  // namespace igc
