// Widening of a packed MXFP4 operand to MXFP8 elements, so that a product of
// one MXFP4 and one MXFP8 operand runs on the MXFP8 kernels: every E2M1 value
// (0, 0.5, 1, 1.5, 2, 3, 4, 6 and their negatives) is exactly an E4M3FN value,
// and the E8M0 block scales stay as they are.  Bound by HBM.

#include <hip/hip_runtime.h>

#include <cstdint>

#include "sk_common.h"

namespace sk {

namespace {

typedef uint32_t v4w __attribute__((ext_vector_type(4)));

// The E4M3 bytes of the eight E2M1 magnitudes as a byte table for v_perm_b32,
// whose selector bytes 0..3 pick bytes of its second operand and 4..7 bytes of
// its first: bytes 0x00 0x30 0x38 0x3C | 0x40 0x44 0x48 0x4C.
constexpr uint32_t kMagLo = 0x3C383000u, kMagHi = 0x4C484440u;

// Eight E2M1 codes (one source dword, even K in each byte's low nibble) to
// eight E4M3 bytes in K order, as two dwords.
__device__ __forceinline__ void widen_word(uint32_t x, uint32_t& lo, uint32_t& hi) {
  const uint32_t ev = __builtin_amdgcn_perm(kMagHi, kMagLo, x & 0x07070707u) | ((x & 0x08080808u) << 4);
  const uint32_t od = __builtin_amdgcn_perm(kMagHi, kMagLo, (x >> 4) & 0x07070707u) | (x & 0x80808080u);
  // interleave: K order is ev.b0 od.b0 ev.b1 od.b1 | ev.b2 od.b2 ev.b3 od.b3
  lo = __builtin_amdgcn_perm(od, ev, 0x05010400u);
  hi = __builtin_amdgcn_perm(od, ev, 0x07030602u);
}

// dst[r][k] = E4M3 byte of the E2M1 code at src[r][k / 2] (even k in the low
// nibble).  Each thread widens 16 source bytes (32 codes) into 32 bytes.
__global__ __launch_bounds__(256) void sk_widen_e2m1(const uint8_t* __restrict__ src, uint8_t* __restrict__ dst,
                                                      int64_t pieces) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= pieces) return;
  const v4w x = *(const v4w*)(src + i * 16);
  uint32_t w[8];
#pragma unroll
  for (int k = 0; k < 4; ++k) widen_word(x[k], w[2 * k], w[2 * k + 1]);
  const v4w y0 = v4w{w[0], w[1], w[2], w[3]}, y1 = v4w{w[4], w[5], w[6], w[7]};
  v4w* q = (v4w*)(dst + i * 32);
  q[0] = y0;
  q[1] = y1;
}

}  // namespace

hipError_t launch_widen_e2m1(const uint8_t* src, uint8_t* dst, int64_t bytes, hipStream_t s) {
  if (bytes % 16 || ((uintptr_t)src & 15) || ((uintptr_t)dst & 15)) return hipErrorInvalidValue;
  const int64_t pieces = bytes / 16;
  if (pieces == 0) return hipSuccess;
  hipLaunchKernelGGL(sk_widen_e2m1, dim3((unsigned)((pieces + 255) / 256)), dim3(256), 0, s, src, dst, pieces);
  return hipGetLastError();
}

}  // namespace sk
