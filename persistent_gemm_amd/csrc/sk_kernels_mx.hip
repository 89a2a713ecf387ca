// Stream-K GEMM kernels for the MX formats with 6-bit elements (MXFP6: E2M3 or
// E3M2, each operand with its own E8M0 block scales) and for one MXFP4 and one
// MXFP8 operand.  They use the kernel template's WIDE LDS image (32 bytes per
// 32-element block), in which the 6-bit and E2M1 blocks are padded to the E4M3
// block size, and the scaled MFMA takes each operand in its own format
// (sk_kernel.h: gchunk, read_chunk, mfma_operand).  Their indices follow those
// of sk_kernels.hip.

#include "sk_kernel.h"

namespace sk {

static const Variant kWideVariants[] = {
    // MXFP6 E2M3 x E2M3 (the first variant of a tile shape is the automatic choice for it)
    SK_VARIANT(DT_MXFP6_E2M3, 256, 256, 128, 32, 2, 4, 2, 2),
    SK_VARIANT(DT_MXFP6_E2M3, 256, 256, 64, 32, 2, 4, 4, 2),
    SK_VARIANT(DT_MXFP6_E2M3, 128, 128, 128, 32, 2, 2, 4, 1),
    SK_VARIANT(DT_MXFP6_E2M3, 64, 64, 64, 32, 2, 2, 4, 2),
    SK_VARIANT(DT_MXFP6_E2M3, 16, 256, 128, 16, 1, 4, 3, 1),
    SK_VARIANT(DT_MXFP6_E2M3, 16, 128, 128, 16, 1, 4, 4, 1),
    // MXFP6 E3M2 x E3M2
    SK_VARIANT(DT_MXFP6_E3M2, 256, 256, 128, 32, 2, 4, 2, 2),
    SK_VARIANT(DT_MXFP6_E3M2, 256, 256, 64, 32, 2, 4, 4, 2),
    SK_VARIANT(DT_MXFP6_E3M2, 128, 128, 128, 32, 2, 2, 4, 1),
    SK_VARIANT(DT_MXFP6_E3M2, 64, 64, 64, 32, 2, 2, 4, 2),
    SK_VARIANT(DT_MXFP6_E3M2, 16, 256, 128, 16, 1, 4, 3, 1),
    SK_VARIANT(DT_MXFP6_E3M2, 16, 128, 128, 16, 1, 4, 4, 1),
    // A MXFP4 (E2M1) x B MXFP8 (E4M3)
    SK_VARIANT(DT_MXFP4_MXFP8, 256, 256, 64, 32, 2, 4, 4, 2),
    SK_VARIANT(DT_MXFP4_MXFP8, 128, 128, 128, 32, 2, 2, 4, 1),
    SK_VARIANT(DT_MXFP4_MXFP8, 64, 64, 64, 32, 2, 2, 4, 2),
    SK_VARIANT(DT_MXFP4_MXFP8, 16, 256, 128, 16, 1, 4, 3, 1),
    // A MXFP8 (E4M3) x B MXFP4 (E2M1)
    SK_VARIANT(DT_MXFP8_MXFP4, 256, 256, 64, 32, 2, 4, 4, 2),
    SK_VARIANT(DT_MXFP8_MXFP4, 128, 128, 128, 32, 2, 2, 4, 1),
    SK_VARIANT(DT_MXFP8_MXFP4, 64, 64, 64, 32, 2, 2, 4, 2),
    SK_VARIANT(DT_MXFP8_MXFP4, 16, 256, 128, 16, 1, 4, 3, 1),
};

const Variant* wide_variants(int* count) {
  *count = (int)(sizeof(kWideVariants) / sizeof(kWideVariants[0]));
  return kWideVariants;
}

}  // namespace sk
