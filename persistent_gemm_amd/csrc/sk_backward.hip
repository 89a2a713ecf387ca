// Helper kernels of the bf16 backward pass (gradients of C = A * B^T + bias):
// a tiled bf16 transpose, which turns the stored operands into the K-contiguous
// layouts the Stream-K GEMM reads, and the bias gradient, a column sum of dC
// taken in a fixed order and rounded once.  All of them are bound by HBM.

#include <hip/hip_runtime.h>

#include <cstdint>

#include "sk_common.h"

namespace sk {

namespace {

constexpr int TT = 64;   // transpose tile: TT x TT elements

// dst[c][r] = src[r][c] for r < rows, c < cols (bf16 bit patterns).  One
// workgroup moves one 64 x 64 tile through LDS: each thread loads 16
// consecutive elements of a source row and stores 16 consecutive elements of a
// destination row (two 16-byte accesses each way when the tile is whole and
// rows are whole 16-byte pieces; element by element at ragged edges).  The LDS
// pitch of 66 elements spreads the column reads over the banks.
typedef uint32_t v4w __attribute__((ext_vector_type(4)));

__global__ __launch_bounds__(256) void sk_transpose_bf16(const uint16_t* __restrict__ src, uint16_t* __restrict__ dst,
                                                          int rows, int cols) {
  __shared__ uint16_t tile[TT][TT + 2];
  const int r0 = blockIdx.y * TT, c0 = blockIdx.x * TT;
  const int t = threadIdx.x, tr = t / 4, tc = (t % 4) * 16;
  const bool whole = r0 + TT <= rows && c0 + TT <= cols && (rows % 8) == 0 && (cols % 8) == 0;
  if (whole) {
    const v4w* p = (const v4w*)(src + (int64_t)(r0 + tr) * cols + c0 + tc);
    const v4w x0 = p[0], x1 = p[1];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      tile[tr][tc + 2 * j] = (uint16_t)x0[j];
      tile[tr][tc + 2 * j + 1] = (uint16_t)(x0[j] >> 16);
      tile[tr][tc + 8 + 2 * j] = (uint16_t)x1[j];
      tile[tr][tc + 8 + 2 * j + 1] = (uint16_t)(x1[j] >> 16);
    }
  } else {
    const int r = r0 + tr;
#pragma unroll
    for (int j = 0; j < 16; ++j) {
      const int c = c0 + tc + j;
      tile[tr][tc + j] = (r < rows && c < cols) ? src[(int64_t)r * cols + c] : (uint16_t)0;
    }
  }
  __syncthreads();
  const int c = c0 + tr;   // destination row
  if (whole) {
    v4w y0, y1;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      y0[j] = (uint32_t)tile[tc + 2 * j][tr] | ((uint32_t)tile[tc + 2 * j + 1][tr] << 16);
      y1[j] = (uint32_t)tile[tc + 8 + 2 * j][tr] | ((uint32_t)tile[tc + 8 + 2 * j + 1][tr] << 16);
    }
    v4w* q = (v4w*)(dst + (int64_t)c * rows + r0 + tc);
    q[0] = y0;
    q[1] = y1;
  } else if (c < cols) {
#pragma unroll
    for (int j = 0; j < 16; ++j) {
      const int r = r0 + tc + j;
      if (r < rows) dst[(int64_t)c * rows + r] = tile[tc + j][tr];
    }
  }
}

constexpr int CS_ROWS = 32;    // rows of dC summed by one workgroup of the first pass
constexpr int CS_COLS = 2048;  // columns of one workgroup: 8 per thread

// First pass of dbias: part[chunk][n] = sum of dC[m][n] over the chunk's rows,
// in increasing m, in fp32.  Each thread sums 8 adjacent columns, reading 16
// bytes of a row at a time (N is a multiple of 8, rows are 16-byte aligned);
// a workgroup covers 2048 columns of 32 rows.
__global__ __launch_bounds__(256) void sk_colsum_partial(const uint16_t* __restrict__ dc, float* __restrict__ part,
                                                          int M, int N) {
  const int n0 = blockIdx.x * CS_COLS + threadIdx.x * 8;
  const int chunk = blockIdx.y, m0 = chunk * CS_ROWS, m1 = min(M, m0 + CS_ROWS);
  if (n0 >= N) return;
  float s[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
#pragma unroll 8
  for (int m = m0; m < m1; ++m) {
    const v4w x = *(const v4w*)(dc + (int64_t)m * N + n0);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      s[2 * j] += __uint_as_float(x[j] << 16);
      s[2 * j + 1] += __uint_as_float(x[j] & 0xffff0000u);
    }
  }
  float* out = part + (int64_t)chunk * N + n0;
#pragma unroll
  for (int j = 0; j < 8; ++j) out[j] = s[j];
}

// Second pass: dbias[n] = bf16 of the sum of the chunk partials, rounded once
// to nearest-even (NaN kept quiet).  A workgroup handles 32 columns with 8
// threads each: thread t of a column sums the t-th contiguous run of chunks in
// increasing order, then the column's first thread adds the 8 run sums in
// increasing t.  The association is fixed, so the bits repeat.
__global__ __launch_bounds__(256) void sk_colsum_final(const float* __restrict__ part, uint16_t* __restrict__ dbias,
                                                        int chunks, int N) {
  __shared__ float run_sum[8][32];
  const int col = threadIdx.x & 31, t = threadIdx.x >> 5;
  const int n = blockIdx.x * 32 + col;
  const int per = (chunks + 7) / 8, c0 = t * per, c1 = min(chunks, c0 + per);
  float s = 0.0f;
  if (n < N) {
#pragma unroll 8
    for (int c = c0; c < c1; ++c) s += part[(int64_t)c * N + n];
  }
  run_sum[t][col] = s;
  __syncthreads();
  if (t != 0 || n >= N) return;
  float r = 0.0f;
#pragma unroll
  for (int k = 0; k < 8; ++k) r += run_sum[k][col];
  const uint32_t u = __float_as_uint(r);
  uint16_t h;
  if ((u & 0x7fffffffu) > 0x7f800000u) h = (uint16_t)((u >> 16) | 0x40u);
  else h = (uint16_t)((u + 0x7fffu + ((u >> 16) & 1u)) >> 16);
  dbias[n] = h;
}

}  // namespace

hipError_t launch_transpose_bf16(const uint16_t* src, uint16_t* dst, int rows, int cols, hipStream_t s) {
  const dim3 grid((unsigned)((cols + TT - 1) / TT), (unsigned)((rows + TT - 1) / TT));
  hipLaunchKernelGGL(sk_transpose_bf16, grid, dim3(256), 0, s, src, dst, rows, cols);
  return hipGetLastError();
}

int64_t colsum_scratch_bytes(int M, int N) { return (int64_t)((M + CS_ROWS - 1) / CS_ROWS) * N * (int64_t)sizeof(float); }

hipError_t launch_colsum_bf16(const uint16_t* dc, float* part, uint16_t* dbias, int M, int N, hipStream_t s) {
  const int chunks = (M + CS_ROWS - 1) / CS_ROWS;
  if (N % 8 || ((uintptr_t)dc & 15)) return hipErrorInvalidValue;
  hipLaunchKernelGGL(sk_colsum_partial, dim3((unsigned)((N + CS_COLS - 1) / CS_COLS), (unsigned)chunks), dim3(256), 0,
                     s, dc, part, M, N);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(sk_colsum_final, dim3((unsigned)((N + 31) / 32)), dim3(256), 0, s, part, dbias, chunks, N);
  return hipGetLastError();
}

}  // namespace sk
