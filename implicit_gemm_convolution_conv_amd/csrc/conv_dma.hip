// Dispatch of the direct-to-LDS conv kernel on the tile index. The tiles are
// instantiated in the conv_dma_{bf16,fp8}_*.hip units, a few per unit, so the
// units compile in parallel; the declarations below keep this unit from
// instantiating them again.
#include "conv_igemm_dma.h"

namespace igc {

IGC_DMA_EXTERN(DT_BF16, 6);
IGC_DMA_EXTERN(DT_BF16, 7);
IGC_DMA_EXTERN(DT_BF16, 8);
IGC_DMA_EXTERN(DT_BF16, 9);
IGC_DMA_EXTERN(DT_BF16, 10);
IGC_DMA_EXTERN(DT_BF16, 11);
IGC_DMA_EXTERN(DT_BF16, 18);
IGC_DMA_EXTERN(DT_BF16, 19);
IGC_DMA_EXTERN(DT_BF16, 20);
IGC_DMA_EXTERN(DT_BF16, 14);
IGC_DMA_EXTERN(DT_BF16, 15);
IGC_DMA_EXTERN(DT_BF16, 21);
IGC_DMA_EXTERN(DT_BF16, 22);
IGC_DMA_EXTERN(DT_BF16, 23);
IGC_DMA_EXTERN(DT_BF16, 24);
IGC_DMA_EXTERN(DT_BF16, 25);
IGC_DMA_EXTERN(DT_BF16, 26);
IGC_DMA_EXTERN(DT_BF16, 40);
IGC_DMA_EXTERN(DT_FP8, 7);
IGC_DMA_EXTERN(DT_FP8, 9);
IGC_DMA_EXTERN(DT_FP8, 12);
IGC_DMA_EXTERN(DT_FP8, 13);
IGC_DMA_EXTERN(DT_FP8, 15);
IGC_DMA_EXTERN(DT_FP8, 19);
IGC_DMA_EXTERN(DT_FP8, 21);
IGC_DMA_EXTERN(DT_FP8, 22);
IGC_DMA_EXTERN(DT_FP8, 23);
IGC_DMA_EXTERN(DT_FP8, 24);
IGC_DMA_EXTERN(DT_FP8, 25);
IGC_DMA_EXTERN(DT_FP8, 26);

hipError_t launch_conv_dma_bf16(const ConvParams &p, int tile, Mode mode, bool big, bool cblock, hipStream_t stream)
{
    switch (tile) {
    case 6: return launch_conv_dma_tile<DT_BF16, 6>(p, mode, big, cblock, stream);
    case 7: return launch_conv_dma_tile<DT_BF16, 7>(p, mode, big, cblock, stream);
    case 8: return launch_conv_dma_tile<DT_BF16, 8>(p, mode, big, cblock, stream);
    case 9: return launch_conv_dma_tile<DT_BF16, 9>(p, mode, big, cblock, stream);
    case 10: return launch_conv_dma_tile<DT_BF16, 10>(p, mode, big, cblock, stream);
    case 11: return launch_conv_dma_tile<DT_BF16, 11>(p, mode, big, cblock, stream);
    case 18: return launch_conv_dma_tile<DT_BF16, 18>(p, mode, big, cblock, stream);
    case 19: return launch_conv_dma_tile<DT_BF16, 19>(p, mode, big, cblock, stream);
    case 20: return launch_conv_dma_tile<DT_BF16, 20>(p, mode, big, cblock, stream);
    case 14: return launch_conv_dma_tile<DT_BF16, 14>(p, mode, big, cblock, stream);
    case 15: return launch_conv_dma_tile<DT_BF16, 15>(p, mode, big, cblock, stream);
    case 21: return launch_conv_dma_tile<DT_BF16, 21>(p, mode, big, cblock, stream);
    case 22: return launch_conv_dma_tile<DT_BF16, 22>(p, mode, big, cblock, stream);
    case 23: return launch_conv_dma_tile<DT_BF16, 23>(p, mode, big, cblock, stream);
    case 24: return launch_conv_dma_tile<DT_BF16, 24>(p, mode, big, cblock, stream);
    case 25: return launch_conv_dma_tile<DT_BF16, 25>(p, mode, big, cblock, stream);
    case 26: return launch_conv_dma_tile<DT_BF16, 26>(p, mode, big, cblock, stream);
    case 40: return launch_conv_dma_tile<DT_BF16, 40>(p, mode, big, cblock, stream);
    default: return hipErrorInvalidValue;
    }
}

hipError_t launch_conv_dma_fp8(const ConvParams &p, int tile, Mode mode, bool big, bool cblock, hipStream_t stream)
{
    switch (tile) {
    case 7: return launch_conv_dma_tile<DT_FP8, 7>(p, mode, big, cblock, stream);
    case 9: return launch_conv_dma_tile<DT_FP8, 9>(p, mode, big, cblock, stream);
    case 12: return launch_conv_dma_tile<DT_FP8, 12>(p, mode, big, cblock, stream);
    case 13: return launch_conv_dma_tile<DT_FP8, 13>(p, mode, big, cblock, stream);
    case 15: return launch_conv_dma_tile<DT_FP8, 15>(p, mode, big, cblock, stream);
    case 19: return launch_conv_dma_tile<DT_FP8, 19>(p, mode, big, cblock, stream);
    case 21: return launch_conv_dma_tile<DT_FP8, 21>(p, mode, big, cblock, stream);
    case 22: return launch_conv_dma_tile<DT_FP8, 22>(p, mode, big, cblock, stream);
    case 23: return launch_conv_dma_tile<DT_FP8, 23>(p, mode, big, cblock, stream);
    case 24: return launch_conv_dma_tile<DT_FP8, 24>(p, mode, big, cblock, stream);
    case 25: return launch_conv_dma_tile<DT_FP8, 25>(p, mode, big, cblock, stream);
    case 26: return launch_conv_dma_tile<DT_FP8, 26>(p, mode, big, cblock, stream);
    default: return hipErrorInvalidValue;
    }
}

}  // namespace igc
