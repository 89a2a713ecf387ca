// Device-ceiling probes for the GEMM's roofline (built as libskprobe.so, run by
// bench.py --ceiling; no part of the GEMM path).  They measure, on the whole
// device, what the dense peaks of the data sheet do not say:
//
//   * MFMA-only throughput: every wave issues back-to-back MFMAs into 8
//     independent accumulators, operands in registers, 2 waves per SIMD;
//     operand data fixed per lane, rotating through 8 random operand pairs
//     (each MFMA sees other bits than the one before, as in a GEMM), or zero.
//     Under full load the shader clock is limited by power, and the power
//     drawn depends on the bits the MFMAs toggle.
//   * The same rotating-operand MFMA stream with direct-to-LDS loads of
//     random bytes interleaved (L loads of 1 KiB per wave per 8 MFMAs), from a
//     span per workgroup small enough to stay in L2 or large enough to stream
//     from memory.
//   * The cold read of 32 MiB spread over the device, the skinny GEMM's B:
//     direct-to-LDS loads of 32 rows x 4 KiB per workgroup, 128 bytes of each
//     row per load as the GEMM's k-steps take them, or plain 16-byte vector
//     loads of a contiguous slice per workgroup; each launch reads a region
//     the launches before it did not touch, so none of it is in the MALL.
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v16f __attribute__((ext_vector_type(16)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef __bf16 v8bf __attribute__((ext_vector_type(8)));
typedef unsigned v4u __attribute__((ext_vector_type(4)));

constexpr int kGrid = 256, kThreads = 512;

__device__ __forceinline__ uint32_t mix32(uint32_t x) {
  x ^= x >> 16;
  x *= 0x7feb352du;
  x ^= x >> 15;
  x *= 0x846ca68bu;
  x ^= x >> 16;
  return x;
}

// Operand words of pair i for this lane: MODE 0 the same for every i, 1 a
// different random pair per i, 2 zero.  KIND 2 (bf16): exponent fields kept
// in a narrow range so that no value is an infinity or NaN.
template <int KIND, int MODE>
__device__ __forceinline__ void operands(v8i (&a)[8], v8i (&b)[8]) {
  const uint32_t lane = blockIdx.x * kThreads + threadIdx.x;
#pragma unroll
  for (int i = 0; i < 8; ++i)
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int p = MODE == 1 ? i : 0;
      uint32_t x = mix32(lane * 131u + p * 8 + j), y = mix32(lane * 977u + p * 8 + j + 12345u);
      if (KIND == 2) {
        x = (x & 0x807f807fu) | 0x3f003f00u;   // bf16 pairs in [1, 2) with random signs and mantissas
        y = (y & 0x807f807fu) | 0x3f003f00u;
      } else if (KIND == 1) {
        x &= 0xf7f7f7f7u;                      // E4M3 without the all-ones exponent (no NaN)
        y &= 0xf7f7f7f7u;
      }
      if (MODE == 2) x = y = 0;
      a[i][j] = (int)x;
      b[i][j] = (int)y;
    }
}

// KIND 0: scaled FP4 (E2M1) 32x32x64; 1: scaled E4M3 32x32x64; 2: bf16 32x32x16;
// 3: scaled FP4 16x16x128; 4: bf16 16x16x32 (the 16x16 forms accumulate into 4 floats);
// 5: scaled FP6 (E2M3) 32x32x64 (every 6-bit code is a finite value).
template <int KIND>
__device__ __forceinline__ v4f mfma16(const v8i& a, const v8i& b, v4f c, int sa, int sb) {
  if constexpr (KIND == 3) return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, c, 4, 4, 0, sa, 0, sb);
  else {
    const v8bf x = __builtin_bit_cast(v8bf, int4{a[0], a[1], a[2], a[3]});
    const v8bf y = __builtin_bit_cast(v8bf, int4{b[0], b[1], b[2], b[3]});
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(x, y, c, 0, 0, 0);
  }
}

template <int KIND>
__device__ __forceinline__ v16f mfma(const v8i& a, const v8i& b, v16f c, int sa, int sb) {
  if constexpr (KIND == 0) return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 4, 4, 0, sa, 0, sb);
  else if constexpr (KIND == 1) return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 0, 0, sa, 0, sb);
  else if constexpr (KIND == 5) return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 2, 2, 0, sa, 0, sb);
  else {
    const v8bf x = __builtin_bit_cast(v8bf, int4{a[0], a[1], a[2], a[3]});
    const v8bf y = __builtin_bit_cast(v8bf, int4{b[0], b[1], b[2], b[3]});
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(x, y, c, 0, 0, 0);
  }
}

template <int KIND, int MODE>
__global__ __launch_bounds__(kThreads) void mfma_rate16(int iters, float* out) {
  v4f acc[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) acc[i] = v4f{};
  v8i a[8], b[8];
  operands<KIND == 4 ? 2 : 0, MODE>(a, b);
  const uint32_t lane = blockIdx.x * kThreads + threadIdx.x;
  const int sa = MODE == 1 ? 125 + (int)(mix32(lane) % 5) : 127;
  const int sb = MODE == 1 ? 125 + (int)(mix32(lane + 99u) % 5) : 127;
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int i = 0; i < 8; ++i) acc[i] = mfma16<KIND>(a[i], b[(i + 3) & 7], acc[i], sa, sb);
  }
  float s = 0;
#pragma unroll
  for (int i = 0; i < 8; ++i) s += acc[i][0] + acc[i][3];
  out[blockIdx.x * kThreads + threadIdx.x] = s;
}

template <int KIND, int MODE>
__global__ __launch_bounds__(kThreads) void mfma_rate(int iters, float* out) {
  v16f acc[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) acc[i] = v16f{};
  v8i a[8], b[8];
  operands<KIND, MODE>(a, b);
  const uint32_t lane = blockIdx.x * kThreads + threadIdx.x;
  const int sa = MODE == 1 ? 125 + (int)(mix32(lane) % 5) : 127;
  const int sb = MODE == 1 ? 125 + (int)(mix32(lane + 99u) % 5) : 127;
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int i = 0; i < 8; ++i) acc[i] = mfma<KIND>(a[i], b[(i + 3) & 7], acc[i], sa, sb);
  }
  float s = 0;
#pragma unroll
  for (int i = 0; i < 8; ++i) s += acc[i][0] + acc[i][15];
  out[blockIdx.x * kThreads + threadIdx.x] = s;
}

// Rotating-operand FP4 MFMAs with L direct-to-LDS loads per 8 MFMAs per wave,
// each 1 KiB (64 lanes x 16 bytes) of the workgroup's span of `span` bytes,
// cycled through; at most 12 loads per wave in flight.
template <int L>
__global__ __launch_bounds__(kThreads) void mfma_dma(const uint8_t* src, uint32_t span, int iters, float* out) {
  __shared__ __attribute__((aligned(16))) uint8_t ring[kThreads / 64][16][1024];
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
  const uint64_t base = (uint64_t)(uintptr_t)(src + (uint64_t)blockIdx.x * span);
  v4u rs = v4u{(uint32_t)base, (uint32_t)(base >> 32) & 0xffffu, span, 0x00020000u};
#pragma unroll
  for (int i = 0; i < 4; ++i) rs[i] = __builtin_amdgcn_readfirstlane(rs[i]);
  v16f acc[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) acc[i] = v16f{};
  v8i a[8], b[8];
  operands<0, 1>(a, b);
  const uint32_t chunks = span / 1024;
  uint32_t c = (uint32_t)wave;
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      acc[i] = mfma<0>(a[i], b[(i + 3) & 7], acc[i], 127, 127);
      if constexpr (L > 0) {
        if (i % (8 / L) == 0) {
          const uint32_t lds = (uint32_t)(uintptr_t)&ring[wave][(it * 8 + i) & 15][0];
          const uint32_t voff = (c % chunks) * 1024u + (uint32_t)lane * 16u;
          c += kThreads / 64;
          asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tbuffer_load_dwordx4 %0, %2, 0 offen lds"
                       :: "v"(voff), "s"(__builtin_amdgcn_readfirstlane(lds)), "s"(rs) : "memory", "m0");
        }
      }
    }
    asm volatile("s_waitcnt vmcnt(12)" ::: "memory");
  }
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  float s = 0;
#pragma unroll
  for (int i = 0; i < 8; ++i) s += acc[i][0] + acc[i][15];
  out[blockIdx.x * kThreads + threadIdx.x] = s;
}

// Direct-to-LDS row streaming: workgroup w reads rows [32 w, +32) of a
// [8192][4096]-byte matrix, 128 bytes of every row per step (one load of 64
// lanes x 16 bytes covers 8 rows), 12 loads in flight per wave; the bytes land
// in a 64 KiB LDS ring and are not used.
__global__ __launch_bounds__(256) void stream_rows(const uint8_t* src) {
  __shared__ __attribute__((aligned(16))) uint8_t ring[4][16][1024];
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
  const uint64_t tb = (uint64_t)(uintptr_t)(src + (uint64_t)blockIdx.x * 32 * 4096);
  v4u rs = v4u{(uint32_t)tb, (uint32_t)(tb >> 32) & 0xffffu, 32u * 4096u, 0x00020000u};
#pragma unroll
  for (int i = 0; i < 4; ++i) rs[i] = __builtin_amdgcn_readfirstlane(rs[i]);
  int n = 0;
  for (int k = 0; k < 4096 / 128; ++k) {
    const int row = wave * 8 + lane / 8;   // 4 waves x 8 rows: the 32 rows
    const uint32_t voff = (uint32_t)row * 4096u + (uint32_t)k * 128u + (uint32_t)(lane % 8) * 16u;
    const uint32_t lds = (uint32_t)(uintptr_t)&ring[wave][n & 15][0];
    ++n;
    asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tbuffer_load_dwordx4 %0, %2, 0 offen lds\n\ts_waitcnt vmcnt(12)"
                 :: "v"(voff), "s"(__builtin_amdgcn_readfirstlane(lds)), "s"(rs) : "memory", "m0");
  }
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
}

// Plain 16-byte vector loads: workgroup w reads the w-th of gridDim.x equal
// contiguous slices of the n16 16-byte words, 8 loads in flight per thread.
__global__ __launch_bounds__(256) void stream_plain(const v4u* src, uint64_t n16, uint32_t* out) {
  const uint64_t per = n16 / gridDim.x;
  const v4u* p = src + (uint64_t)blockIdx.x * per;
  v4u acc = {0, 0, 0, 0};
  for (uint64_t i = threadIdx.x; i < per; i += 256 * 8) {
    v4u x[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) x[u] = i + u * 256 < per ? __builtin_nontemporal_load(p + i + u * 256) : v4u{0, 0, 0, 0};
#pragma unroll
    for (int u = 0; u < 8; ++u) acc ^= x[u];
  }
  if ((acc[0] ^ acc[1] ^ acc[2] ^ acc[3]) == 0x12345678u) out[threadIdx.x] = 1;   // keeps the loads
}

typedef void (*RateKernel)(int, float*);

template <int KIND>
RateKernel rate_kernel(int mode) {
  if constexpr (KIND == 3 || KIND == 4) return mode == 0 ? mfma_rate16<KIND, 0> : mode == 1 ? mfma_rate16<KIND, 1> : mfma_rate16<KIND, 2>;
  else return mode == 0 ? mfma_rate<KIND, 0> : mode == 1 ? mfma_rate<KIND, 1> : mfma_rate<KIND, 2>;
}

// Milliseconds of one launch of `launch` (after one launch of warm-up work).
template <class F>
int time_launch(F&& launch, float* ms) {
  hipEvent_t e0, e1;
  if (hipEventCreate(&e0) != hipSuccess || hipEventCreate(&e1) != hipSuccess) return 1;
  int rc = 0;
  launch(true);
  if (hipDeviceSynchronize() != hipSuccess) rc = 1;
  if (!rc && hipEventRecord(e0) != hipSuccess) rc = 1;
  if (!rc) launch(false);
  if (!rc && (hipEventRecord(e1) != hipSuccess || hipEventSynchronize(e1) != hipSuccess)) rc = 1;
  if (!rc && hipEventElapsedTime(ms, e0, e1) != hipSuccess) rc = 1;
  if (!rc && hipGetLastError() != hipSuccess) rc = 1;
  (void)hipEventDestroy(e0);
  (void)hipEventDestroy(e1);
  return rc;
}

}  // namespace

extern "C" {

// Whole-device MFMA-only rate: kind 0 scaled FP4 32x32x64, 1 scaled E4M3
// 32x32x64, 2 bf16 32x32x16, 3 scaled FP4 16x16x128, 4 bf16 16x16x32, 5 scaled
// FP6 (E2M3) 32x32x64; mode 0
// fixed operands, 1 rotating random operands, 2 zero operands.  256 workgroups of 8 waves, `iters` x 8 MFMAs per
// wave.  Writes the launch's milliseconds and FLOP; returns 0, or 1 on error.
int skp_mfma_rate(int kind, int mode, int iters, float* ms, double* flop) {
  if (kind < 0 || kind > 5 || mode < 0 || mode > 2 || iters < 1 || !ms || !flop) return 1;
  float* out = nullptr;
  if (hipMalloc(&out, (size_t)kGrid * kThreads * sizeof(float)) != hipSuccess) return 1;
  RateKernel k = kind == 0 ? rate_kernel<0>(mode) : kind == 1 ? rate_kernel<1>(mode) : kind == 2 ? rate_kernel<2>(mode)
               : kind == 3 ? rate_kernel<3>(mode) : kind == 4 ? rate_kernel<4>(mode) : rate_kernel<5>(mode);
  const int rc = time_launch(
      [&](bool warm) { hipLaunchKernelGGL(k, dim3(kGrid), dim3(kThreads), 0, 0, warm ? iters / 4 + 1 : iters, out); },
      ms);
  (void)hipFree(out);
  const double per = kind == 2 ? 2.0 * 32 * 32 * 16 : kind == 3 ? 2.0 * 16 * 16 * 128 : kind == 4 ? 2.0 * 16 * 16 * 32
                                                                                     : 2.0 * 32 * 32 * 64;
  *flop = per * 8.0 * iters * (kThreads / 64) * kGrid;
  return rc;
}

// Rotating-operand FP4 MFMAs with `loads` (0, 1, 2 or 4) direct-to-LDS loads of
// 1 KiB per wave per 8 MFMAs, from src (device memory of 256 * span bytes,
// span a multiple of 1 KiB below 2^31).  Writes milliseconds, FLOP and bytes
// loaded; returns 0, or 1 on error.
int skp_mfma_dma(int loads, const void* src, uint32_t span, int iters, float* ms, double* flop, double* bytes) {
  if (!(loads == 0 || loads == 1 || loads == 2 || loads == 4) || !src || span < 1024 || span % 1024 || iters < 1 ||
      !ms || !flop || !bytes)
    return 1;
  float* out = nullptr;
  if (hipMalloc(&out, (size_t)kGrid * kThreads * sizeof(float)) != hipSuccess) return 1;
  void (*k)(const uint8_t*, uint32_t, int, float*) =
      loads == 0 ? mfma_dma<0> : loads == 1 ? mfma_dma<1> : loads == 2 ? mfma_dma<2> : mfma_dma<4>;
  const int rc = time_launch(
      [&](bool warm) {
        hipLaunchKernelGGL(k, dim3(kGrid), dim3(kThreads), 0, 0, (const uint8_t*)src, span,
                           warm ? iters / 4 + 1 : iters, out);
      },
      ms);
  (void)hipFree(out);
  *flop = 2.0 * 32 * 32 * 64 * 8.0 * iters * (kThreads / 64) * kGrid;
  *bytes = 1024.0 * loads * iters * (kThreads / 64) * kGrid;
  return rc;
}

// The cold read of 32 MiB: pattern 0 direct-to-LDS rows (256 workgroups of
// 4 waves), 1 plain vector loads (1024 workgroups of 4 waves).  src: device
// memory of at least `regions` x 64 MiB; launch i reads the 32 MiB at i x
// 64 MiB, so a region is read once.  Writes each launch's milliseconds (HIP
// events around the launch, which include its dispatch) to ms[0 .. regions);
// returns 0, or 1 on error.
int skp_stream(int pattern, const void* src, int regions, float* ms) {
  if ((pattern != 0 && pattern != 1) || !src || regions < 1 || regions > 64 || !ms) return 1;
  uint32_t* out = nullptr;
  if (hipMalloc(&out, 1024) != hipSuccess) return 1;
  int rc = 0;
  for (int r = 0; r < regions && !rc; ++r) {
    const uint8_t* base = (const uint8_t*)src + (uint64_t)r * (64ull << 20);
    rc = time_launch(
        [&](bool warm) {
          if (warm) {
            hipLaunchKernelGGL(stream_plain, dim3(64), dim3(256), 0, 0, (const v4u*)out, (uint64_t)64, out);
          } else if (pattern == 0) {
            hipLaunchKernelGGL(stream_rows, dim3(256), dim3(256), 0, 0, base);
          } else {
            hipLaunchKernelGGL(stream_plain, dim3(1024), dim3(256), 0, 0, (const v4u*)base, (uint64_t)(32ull << 20) / 16, out);
          }
        },
        &ms[r]);
  }
  (void)hipFree(out);
  return rc;
}

}  // extern "C"
