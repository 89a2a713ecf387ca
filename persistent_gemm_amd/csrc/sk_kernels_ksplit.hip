// Stream-K GEMM kernels whose waves split each k-step (WK groups of waves,
// sk_kernel.h: Cfg), for skinny problems: a 16 x 32 output tile has too few
// MFMA blocks to occupy more than one or two waves, so these give each tile
// four waves anyway, each multiplying its own k-slice, and every k-step reads
// WK * KB contiguous bytes of each row.  At 16 x 8192 x 8192 the 256 tiles of
// 16 x 32 are one per compute unit, so the whole of B streams once with no
// split tiles.  They read MX scales straight from the caller's arrays only.
// Their indices follow those of sk_kernels_mx.hip.

#include "sk_kernel.h"

namespace sk {

static const Variant kSplitVariants[] = {
    SK_VARIANT_WK(DT_MXFP4, 16, 32, 128, 16, 1, 1, 4, 4, 1),
    SK_VARIANT_WK(DT_MXFP4, 16, 32, 128, 16, 1, 1, 3, 4, 1),
    SK_VARIANT_WK(DT_MXFP4, 16, 32, 64, 16, 1, 1, 6, 4, 1),
};

const Variant* split_variants(int* count) {
  *count = (int)(sizeof(kSplitVariants) / sizeof(kSplitVariants[0]));
  return kSplitVariants;
}

}  // namespace sk
