// Stream-K GEMM kernels for gfx950 (MI355X): the MX scale re-layout pass and
// the table of compiled kernel variants (the kernel template is sk_kernel.h;
// the MXFP6 and mixed-format kernels are instantiated in sk_kernels_mx.hip).

#include "sk_kernel.h"

namespace sk {

// ---------------------------------------------------------------- MX scale re-layout

// The scale pre-pass: src[r][c] (E8M0, [rows][s_pitch]) into the copy the
// kernel reads, k-step major and in the MFMA lane order of a tile:
//
//   dst[ks][t][q] for q < TR * SPR, q = (((v * MF + l) * NG + g) * NB + i) * NU + u
//                = src[t * TR + v * (NB * MF) + i * MF + l][ks * SPR + g * NU + u]
//
// t is the tile (TR rows: BM for A, BN for B), v the wave row (of NB * MF rows),
// l the row inside an MFMA block, g the lane group, i the block and u the
// sub-step; so a lane's NB * NU bytes for a k-step are contiguous.  127 (a
// scale of 1) stands for rows past `rows` and bytes past s_pitch (a ragged last
// k-step).  All the factors are powers of two, given as shifts.  One
// workgroup moves a tile's rows for RB / SPR k-steps (RB bytes of each row)
// through LDS: rows are read 16 bytes at a time when aligned, each k-step's
// block is written 16 bytes at a time.  The LDS rows are RB + 4 bytes apart
// (an odd number of banks), since the lanes of a wave gather bytes from rows
// a few apart.  RB = 16 gives four small workgroups per CU at 8192^3, whose
// loads and stores overlap; a pass of few large workgroups waits out one
// memory round trip after another.
struct RelayoutOp {
  const uint8_t* src;
  uint8_t* dst;
  int rows, dst_rows, vec16, blocks;   // dst_rows: rows rounded up to whole tiles; blocks: tiles
  int tr, mf_s, ng_s, nb_s, nu_s;      // TR, and log2 of MF, NG, NB, NU
};

template <int SPR, int RB>
__global__ __launch_bounds__(256) void sk_scale_relayout(RelayoutOp a, RelayoutOp b, int s_pitch, int ksteps) {
  constexpr int KT = RB / SPR;                 // k-steps per workgroup
  constexpr int PITCH = RB + 4;                // LDS bytes per tile row
  constexpr int PR = RB / 16;                  // 16-byte pieces per row
  __shared__ __attribute__((aligned(16))) uint8_t t8[256 * PITCH];   // [tile row][RB bytes + 4]
  const bool is_a = (int)blockIdx.x < a.blocks;
  const RelayoutOp o = is_a ? a : b;
  const int tb = is_a ? (int)blockIdx.x : (int)blockIdx.x - a.blocks;
  const int r0 = tb * o.tr, k0 = blockIdx.y * KT;
  const int tid = threadIdx.x;
  const uint8_t* __restrict__ src = o.src;
  if (o.vec16) {
    // s_pitch % 16 == 0: a 16-byte piece is wholly inside the row or past its end
    for (int pc = tid; pc < o.tr * PR; pc += 256) {
      const int r = pc / PR, q = pc % PR, row = r0 + r, col = k0 * SPR + q * 16;
      v4u v = v4u{0x7f7f7f7fu, 0x7f7f7f7fu, 0x7f7f7f7fu, 0x7f7f7f7fu};
      if (row < o.rows && col < s_pitch) v = *(const v4u*)(src + (int64_t)row * s_pitch + col);
      uint32_t* d = (uint32_t*)(t8 + r * PITCH + q * 16);
      d[0] = v[0];
      d[1] = v[1];
      d[2] = v[2];
      d[3] = v[3];
    }
  } else {
    for (int bi = tid; bi < o.tr * RB; bi += 256) {
      const int r = bi / RB, c = bi % RB, row = r0 + r, col = k0 * SPR + c;
      t8[r * PITCH + c] = (row < o.rows && col < s_pitch) ? src[(int64_t)row * s_pitch + col] : (uint8_t)127;
    }
  }
  __syncthreads();
  const int qb = o.tr * SPR / 16;              // 16-byte pieces of one k-step's tile block
  const int mf_m = (1 << o.mf_s) - 1, ng_m = (1 << o.ng_s) - 1, nb_m = (1 << o.nb_s) - 1, nu_m = (1 << o.nu_s) - 1;
  for (int pc = tid; pc < KT * qb; pc += 256) {
    const int k = pc / qb, q0 = (pc - k * qb) * 16, ks = k0 + k;
    if (ks >= ksteps) continue;
    uint32_t w[4] = {0u, 0u, 0u, 0u};
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      int q = q0 + e;
      const int u = q & nu_m;
      q >>= o.nu_s;
      const int i = q & nb_m;
      q >>= o.nb_s;
      const int g = q & ng_m;
      q >>= o.ng_s;
      const int l = q & mf_m, v = q >> o.mf_s;
      const int r = (((v << o.nb_s) + i) << o.mf_s) + l, j = (g << o.nu_s) + u;
      w[e >> 2] |= (uint32_t)t8[r * PITCH + k * SPR + j] << (8 * (e & 3));
    }
    *(v4u*)(o.dst + ((int64_t)ks * o.dst_rows + r0) * SPR + q0) = v4u{w[0], w[1], w[2], w[3]};
  }
}

namespace {
int log2i(int x) {
  int s = 0;
  while ((1 << s) < x) ++s;
  return s;
}
}  // namespace

hipError_t launch_scale_relayout(const uint8_t* src_a, uint8_t* dst_a, const ScaleLayout& la, const uint8_t* src_b,
                                 uint8_t* dst_b, const ScaleLayout& lb, int s_pitch, int ksteps, int spr,
                                 hipStream_t s) {
  if (spr != 2 && spr != 4 && spr != 8) return hipErrorInvalidValue;
  if (((uintptr_t)dst_a | (uintptr_t)dst_b) & 15) return hipErrorInvalidValue;
  auto op = [&](const uint8_t* src, uint8_t* dst, const ScaleLayout& l) {
    RelayoutOp o;
    o.src = src;
    o.dst = dst;
    o.rows = l.rows;
    o.tr = l.tile_rows;
    o.dst_rows = (l.rows + l.tile_rows - 1) / l.tile_rows * l.tile_rows;
    o.blocks = o.dst_rows / l.tile_rows;
    o.vec16 = (s_pitch % 16 == 0 && ((uintptr_t)src & 15) == 0) ? 1 : 0;
    o.mf_s = log2i(l.mf);
    o.ng_s = log2i(l.ng);
    o.nb_s = log2i(l.nblk);
    o.nu_s = log2i(l.nu);
    return o;
  };
  for (const ScaleLayout* l : {&la, &lb}) {
    const bool pow2 = !(l->mf & (l->mf - 1)) && !(l->ng & (l->ng - 1)) && !(l->nblk & (l->nblk - 1)) &&
                      !(l->nu & (l->nu - 1));
    if (!pow2 || l->ng * l->nu != spr || l->tile_rows % (l->nblk * l->mf) || l->tile_rows > 256 || l->tile_rows < 16)
      return hipErrorInvalidValue;
  }
  const RelayoutOp a = op(src_a, dst_a, la), b = op(src_b, dst_b, lb);
  constexpr int RB = 16;
  const dim3 grid((unsigned)(a.blocks + b.blocks), (unsigned)((ksteps + RB / spr - 1) / (RB / spr)));
  if (spr == 2) hipLaunchKernelGGL((sk_scale_relayout<2, RB>), grid, dim3(256), 0, s, a, b, s_pitch, ksteps);
  else if (spr == 4) hipLaunchKernelGGL((sk_scale_relayout<4, RB>), grid, dim3(256), 0, s, a, b, s_pitch, ksteps);
  else hipLaunchKernelGGL((sk_scale_relayout<8, RB>), grid, dim3(256), 0, s, a, b, s_pitch, ksteps);
  return hipGetLastError();
}

static const Variant kVariants[] = {
    // MXFP4 (the first variant of a tile shape is the automatic choice for it)
    SK_VARIANT(DT_MXFP4, 256, 256, 64, 32, 2, 2, 4, 1),
    SK_VARIANT(DT_MXFP4, 256, 256, 64, 32, 2, 4, 4, 2),
    SK_VARIANT(DT_MXFP4, 128, 128, 128, 32, 2, 2, 4, 1),
    SK_VARIANT(DT_MXFP4, 64, 64, 64, 32, 2, 2, 4, 2),
    SK_VARIANT(DT_MXFP4, 16, 256, 64, 16, 1, 4, 4, 1),
    SK_VARIANT(DT_MXFP4, 16, 256, 64, 16, 1, 4, 8, 1),
    SK_VARIANT(DT_MXFP4, 16, 128, 64, 16, 1, 4, 4, 1),
    // bf16
    SK_VARIANT(DT_BF16, 256, 256, 64, 32, 2, 4, 4, 2),
    SK_VARIANT(DT_BF16, 256, 256, 64, 32, 2, 2, 4, 1),
    SK_VARIANT(DT_BF16, 128, 128, 128, 32, 2, 2, 4, 1),
    SK_VARIANT(DT_BF16, 128, 192, 128, 32, 2, 2, 3, 1),
    SK_VARIANT(DT_BF16, 64, 64, 64, 32, 2, 2, 4, 2),
    // fp8
    SK_VARIANT(DT_FP8, 256, 256, 64, 32, 2, 4, 4, 2),
    SK_VARIANT(DT_FP8, 256, 256, 64, 32, 2, 2, 4, 1),
    SK_VARIANT(DT_FP8, 128, 128, 128, 32, 2, 2, 4, 1),
    SK_VARIANT(DT_FP8, 64, 64, 64, 32, 2, 2, 4, 2),
    SK_VARIANT(DT_FP8, 16, 256, 128, 16, 1, 4, 3, 1),
    // MXFP8 (E4M3 elements, E8M0 scale per 32 K)
    SK_VARIANT(DT_MXFP8, 256, 256, 64, 32, 2, 4, 4, 2),
    SK_VARIANT(DT_MXFP8, 256, 256, 64, 32, 2, 2, 4, 1),
    SK_VARIANT(DT_MXFP8, 128, 128, 128, 32, 2, 2, 4, 1),
    SK_VARIANT(DT_MXFP8, 64, 64, 64, 32, 2, 2, 4, 2),
    SK_VARIANT(DT_MXFP8, 16, 256, 128, 16, 1, 4, 3, 1),
    // 256x256 tiles with 128-byte k-steps in two stages (half the barriers per K)
    SK_VARIANT(DT_MXFP4, 256, 256, 128, 32, 2, 2, 2, 1),
    SK_VARIANT(DT_MXFP4, 256, 256, 128, 32, 2, 4, 2, 2),
    SK_VARIANT(DT_BF16, 256, 256, 128, 32, 2, 2, 2, 1),
    SK_VARIANT(DT_BF16, 256, 256, 128, 32, 2, 4, 2, 2),
    SK_VARIANT(DT_FP8, 256, 256, 128, 32, 2, 2, 2, 1),
    SK_VARIANT(DT_FP8, 256, 256, 128, 32, 2, 4, 2, 2),
    // 16-row MXFP4 tiles with 128-byte k-steps: every row read of a k-step is a
    // whole 128-byte line, so each line in flight carries twice the bytes
    SK_VARIANT(DT_MXFP4, 16, 128, 128, 16, 1, 4, 4, 1),
    SK_VARIANT(DT_MXFP4, 16, 128, 128, 16, 1, 4, 8, 1),
    SK_VARIANT(DT_MXFP4, 16, 64, 128, 16, 1, 2, 8, 1),
    SK_VARIANT(DT_MXFP4, 16, 32, 128, 16, 1, 1, 8, 1),
};

// sk_kernels_mx.hip: the MXFP6 and mixed-format kernels, numbered after these;
// sk_kernels_ksplit.hip: the k-split kernels, numbered after those.
const Variant* wide_variants(int* count);
const Variant* split_variants(int* count);

namespace {
constexpr int kBase = (int)(sizeof(kVariants) / sizeof(kVariants[0]));
}

int num_variants() {
  int nw = 0, ns = 0;
  wide_variants(&nw);
  split_variants(&ns);
  return kBase + nw + ns;
}
const Variant* variant(int index) {
  if (index >= 0 && index < kBase) return &kVariants[index];
  int nw = 0, ns = 0;
  const Variant* w = wide_variants(&nw);
  if (index >= kBase && index < kBase + nw) return &w[index - kBase];
  const Variant* x = split_variants(&ns);
  return (index >= kBase + nw && index < kBase + nw + ns) ? &x[index - kBase - nw] : nullptr;
}

}  // namespace sk
