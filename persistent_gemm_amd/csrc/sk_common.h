// Shared between the host side (planner, launch) and the device side (kernel).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace sk {

// Input types.  DT_MXFP4_MXFP8 / DT_MXFP8_MXFP4: A in one MX format and B in
// the other (E2M1 x E4M3 or E4M3 x E2M1, each with its own E8M0 scales).
enum : int {
  DT_MXFP4 = 0, DT_BF16 = 1, DT_FP8 = 2, DT_MXFP8 = 3, DT_MXFP6_E2M3 = 4, DT_MXFP6_E3M2 = 5,
  DT_MXFP4_MXFP8 = 6, DT_MXFP8_MXFP4 = 7
};
constexpr int kNumDtypes = 8;

// Lock flags per scratch area; the grid never exceeds this many workgroups.
constexpr int kMaxGrid = 1024;
// Index of the device error word inside the flag array.
constexpr int kErrIndex = kMaxGrid;
constexpr int kFlagWords = kMaxGrid + 64;

// Size limits that keep every in-kernel index and byte offset in 32 bits:
// a 256-row slab of C (256 * N * 2 bytes), of A or B (256 * row bytes) and
// the Stream-K iteration count (tiles * iterations per tile) stay below 2^31.
constexpr int64_t kMaxM = (int64_t)1 << 31;
constexpr int64_t kMaxN = (int64_t)1 << 22;
constexpr int64_t kMaxK = (int64_t)1 << 21;
constexpr int64_t kMaxIters = ((int64_t)1 << 31) - 1;

// Everything one launch needs.  Pointers are device pointers.
struct KArgs {
  const uint8_t* A;
  const uint8_t* B;
  const uint8_t* SA;        // MX block scales of A, k-step-major: [k-step][M][SPR] (direct kernels: [M][s_pitch])
  const uint8_t* SB;        // MX block scales of B, k-step-major: [k-step][N][SPR] (direct kernels: [N][s_pitch])
  const float* fsa;         // fp8 per-tensor scale of A (NULL = 1)
  const float* fsb;         // fp8 per-tensor scale of B (NULL = 1)
  const uint16_t* bias;     // bf16[N] or NULL
  uint16_t* C;              // bf16[M][N]
  float* P;                 // fp32 partial tiles, one BM*BN slot per workgroup
  uint32_t* locks;          // one flag per workgroup; flag == epoch means "partial published"
  uint32_t* err;            // set to 1 when a wait gives up
  uint64_t spin_limit;      // ticks of the 100 MHz realtime counter
  int32_t M, N, K;
  int32_t row_bytes;        // bytes of K data per row of A (its pitch)
  int32_t row_bytes_b;      // the same for B (differs from A's when the formats differ)
  uint32_t sa_kstride;      // bytes per k-step block of SA and of SB (padded rows * SPR)
  uint32_t sb_kstride;
  int32_t tiles;            // T
  int32_t sk_tiles;         // tiles [0, sk_tiles) are split by MAC iteration
  int32_t q, r;             // Stream-K iterations S = q*G + r
  int32_t tiles_m, tiles_n;
  int32_t iters;            // I, MAC iterations (k-steps) per tile
  int32_t G;                // persistent workgroups
  uint32_t epoch;           // this launch's flag value
  int32_t drop_wg;          // test hook: this workgroup never publishes (-1: none)
  uint32_t delay_seed;      // test hook: nonzero = seeded sleeps before publishing
  int32_t s_pitch;          // row pitch (bytes) of SA and SB when they are the caller's [rows][K/32] scales
  uint64_t* trace;          // NULL, or kTraceWords 100 MHz timestamps per workgroup (see sk_gemm_args.trace)
};

// Phase trace of a launch (sk_gemm_args.trace): kTraceWords words per workgroup.
constexpr int kTraceWords = 32;
constexpr int kTraceItems = 6;   // items recorded per workgroup (words 1 .. 4 * kTraceItems)

// Stream-K partition of S = q*G + r MAC iterations: workgroup w owns
// [begin(w), begin(w+1)), the first r workgroups getting one extra iteration.
__host__ __device__ inline int32_t sk_begin(int32_t w, int32_t q, int32_t r) {
  return w * q + (w < r ? w : r);
}

// The workgroup whose range holds iteration x (x < S).
__host__ __device__ inline int32_t sk_owner_of(int32_t x, int32_t q, int32_t r) {
  const int32_t big = r * (q + 1);
  if (x < big) return x / (q + 1);
  return r + (x - big) / q;  // q > 0 here, because x < S
}

// One unit of work of a workgroup: MAC iterations [k0, k1) of one tile.
enum : int { WORK_WHOLE = 0, WORK_CONTRIB = 1, WORK_OWNER = 2 };
struct WorkItem {
  int32_t tile;
  int32_t k0, k1;
  int32_t mode;       // WORK_WHOLE: finish the tile; WORK_CONTRIB: publish a partial;
                      // WORK_OWNER: add the partials of workgroups [first, w) then finish
  int32_t first;      // WORK_OWNER only: lowest contributing workgroup
};

// The work of workgroup w, in the order it is done:
//   1. the contributor segment, when w's Stream-K range ends inside a tile;
//   2. the whole tiles inside the range;
//   3. the owned split tile, when the range starts inside a tile and reaches its end;
//   4. the data-parallel tiles sk_tiles + w + j*G.
// Contributions come first and owners wait only on lower workgroups, so no
// workgroup ever waits on one that could be waiting on it.
struct WorkIter {
  int32_t s, e, I, tf, tl, whole, whole_end, dp, tiles, q, r, G, phase;
  bool contrib, owner;

  __host__ __device__ WorkIter(int32_t w, int32_t sk_tiles, int32_t tiles_, int32_t iters, int32_t q_, int32_t r_,
                               int32_t G_) {
    I = iters;
    q = q_;
    r = r_;
    G = G_;
    tiles = tiles_;
    s = e = 0;
    if (sk_tiles > 0) {
      s = sk_begin(w, q, r);
      e = sk_begin(w + 1, q, r);
    }
    const bool any = s < e;
    tf = any ? s / I : 0;
    tl = any ? (e - 1) / I : 0;
    contrib = any && (e % I) != 0;
    owner = any && (s % I) != 0 && (tf < tl || (e % I) == 0);
    whole = any ? ((s % I) ? tf + 1 : tf) : 0;
    whole_end = any ? ((e % I) ? tl : tl + 1) : 0;
    dp = sk_tiles + w;
    phase = 0;
  }

  __host__ __device__ bool next(WorkItem& it) {
    it.k0 = 0;
    it.k1 = I;
    it.first = -1;
    if (phase == 0) {
      phase = 1;
      if (contrib) {
        it.tile = tl;
        it.k0 = (s > tl * I ? s : tl * I) - tl * I;
        it.k1 = e - tl * I;
        it.mode = WORK_CONTRIB;
        return true;
      }
    }
    if (phase == 1) {
      if (whole < whole_end) {
        it.tile = whole++;
        it.mode = WORK_WHOLE;
        return true;
      }
      phase = 2;
    }
    if (phase == 2) {
      phase = 3;
      if (owner) {
        it.tile = tf;
        it.k0 = s - tf * I;
        it.mode = WORK_OWNER;
        it.first = sk_owner_of(tf * I, q, r);
        return true;
      }
    }
    if (dp >= tiles) return false;
    it.tile = dp;
    dp += G;
    it.mode = WORK_WHOLE;
    return true;
  }
};

// One compiled kernel shape.
struct Variant {
  int dtype;
  int bm, bn;       // output tile
  int kb;           // LDS bytes of each operand row per MAC iteration (k-step)
  int bk;           // K elements per MAC iteration
  int mfma;         // 32 (32x32 MFMA) or 16 (16x16 MFMA)
  int threads;
  int lds;
  int wm, wn;       // waves along M and N
  int ng, nu;       // MFMA lane groups, MFMAs per block per k-slice
  int wk;           // k-slices per k-step, each multiplied by its own group of waves
  // The kernel reading MX scales from the re-laid copy (and the non-MX
  // kernels), or nullptr for a kernel that only reads the caller's scales.
  hipError_t (*launch)(int grid, const KArgs& a, hipStream_t s);
  // The same kernel reading MX scales straight from the caller's row-major
  // [rows][K/32] arrays (no re-layout pass), or nullptr where not compiled.
  hipError_t (*launch_direct)(int grid, const KArgs& a, hipStream_t s);
};

int num_variants();
const Variant* variant(int index);

// How one operand's MX scales are laid out for the kernel: tiles of
// tile_rows rows, each k-step's block in the MFMA lane order given by the
// block rows (mf), lane groups (ng), blocks per wave (nblk) and MFMAs per
// block per k-step (nu); ng * nu is the scale bytes per row per k-step.
struct ScaleLayout {
  int rows, tile_rows, mf, ng, nblk, nu;
};

// Copies the MX scales of A and of B ([rows][s_pitch] each) into the
// k-step-major, lane-ordered copies the kernel reads, in one launch; each
// copy holds whole tiles (rows rounded up to tile_rows).  spr is 2, 4 or 8;
// dst must be 16-byte aligned.
hipError_t launch_scale_relayout(const uint8_t* src_a, uint8_t* dst_a, const ScaleLayout& la, const uint8_t* src_b,
                                 uint8_t* dst_b, const ScaleLayout& lb, int s_pitch, int ksteps, int spr,
                                 hipStream_t s);

// bf16 backward helpers (sk_backward.hip).  dst[c][r] = src[r][c] for a
// rows x cols bf16 matrix.
hipError_t launch_transpose_bf16(const uint16_t* src, uint16_t* dst, int rows, int cols, hipStream_t s);
// dbias[n] = bf16(sum over m of dC[m][n]), fp32 sums in a fixed order; `part`
// holds colsum_scratch_bytes(M, N) bytes of device scratch.
int64_t colsum_scratch_bytes(int M, int N);
hipError_t launch_colsum_bf16(const uint16_t* dc, float* part, uint16_t* dbias, int M, int N, hipStream_t s);

}  // namespace sk
