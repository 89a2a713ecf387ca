// Stream-K GEMM kernel template for gfx950 (MI355X), included by the sources that
// instantiate its variants (sk_kernels.hip, sk_kernels_mx.hip).
//
// One persistent kernel template serves MXFP4, bf16 and fp8.  Each of the G
// workgroups (4 or 8 wave64) walks its work list (WorkIter):
//   1. its Stream-K contributor segment, if its iteration range ends inside a
//      tile: the fp32 partial goes to its scratch slot P[w], then flag w is
//      released with this launch's epoch;
//   2. the whole tiles inside its range;
//   3. its owned split tile, if its range starts inside a tile: it computes its
//      own (last) K part of that tile, then adds the partials of the lower
//      workgroups that hold the earlier K parts, in descending workgroup order,
//      waiting on each flag; then the epilogue;
//   4. its data-parallel tiles sk_tiles + w + j*G.
// A tile is finished by the workgroup holding its last MAC iteration; it only
// ever waits on lower-numbered workgroups, which were dispatched before it and
// publish their partial first thing, so the wait graph has no cycle even when
// the grid is larger than what fits on the device at once.
//
// Main loop.  Per MAC iteration (k-step) each operand row contributes KB bytes
// (64 or 128: 128 or 256 FP4 values, 64 or 128 fp8, 32 or 64 bf16).  The A and
// B k-slices are copied straight from HBM into LDS with 16-byte direct-to-LDS
// buffer loads (one wave instruction fills one 1 KiB row group; rows and K
// chunks past the matrix read as zero) into a ring of STAGES buffers, issued
// STAGES-1 k-steps ahead of use.  MXFP4 scale bytes go the same way (dword
// loads) from a k-step-major copy of the scales that a small pass before the
// GEMM writes (sk_scale_relayout below), so that one k-step's scales of a
// tile are one contiguous block.  Operands are consumed by MFMA:
//   MXFP4: v_mfma_scale_f32_{32x32x64,16x16x128}_f8f6f4 with E2M1 operands and
//          the E8M0 block scales as the per-lane scale operands;
//   fp8:   the same instruction with E4M3 operands and unit block scales; the
//          per-tensor scales are applied in the epilogue;
//   bf16:  v_mfma_f32_{32x32x16,16x16x32}_bf16.
// Lane layout (checked on the device): lane l holds operand row l % MF and the
// (l / MF)-th K group of the instruction; each lane's 32 FP4 values are one
// scale block, whose E8M0 byte is picked by op_sel from the lane's scale word.
// Every lane takes LB = KB / (64 / MF) contiguous bytes of a row per k-step,
// so the K order inside a k-step is permuted identically for A and B (the sum
// is unchanged) and each lane's scale bytes are contiguous in memory.  Each
// MFMA block is computed transposed (B block as the first operand), so a lane
// ends with runs of four consecutive output columns of one row.
//
// The whole work list of a workgroup is one stream of k-steps through the
// stage ring: loads for the next work item are issued while the current one
// is being finished, so HBM traffic does not stop at tile boundaries.  A tile
// is finished from registers: partials are stored and summed in register
// order (each wave store is one contiguous 1 KiB run), and the output is
// rounded and written as 8-byte runs of four bf16.

#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>
#include <utility>

#include "sk_common.h"

namespace sk {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v16f __attribute__((ext_vector_type(16)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef __bf16 v8bf __attribute__((ext_vector_type(8)));
typedef unsigned v4u __attribute__((ext_vector_type(4)));
typedef unsigned v2u __attribute__((ext_vector_type(2)));
typedef __attribute__((address_space(3))) uint8_t lds_u8;
typedef __attribute__((address_space(3))) void lds_void;

// Buffer resource word 3 for gfx9-family raw (untyped) buffers.
constexpr int kRsrcWord3 = 0x00020000;
// Any offset at or past 2^31 lies beyond every resource built here: reads 0,
// writes are dropped.
constexpr uint32_t kOob = 0x80000000u;

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, kRsrcWord3);
}

// A raw buffer resource as four words (for the inline-asm loads below):
// base address, no stride, `bytes` records, raw-buffer flags.
__device__ __forceinline__ v4u rsrc_words(const void* base, uint32_t bytes) {
  const uint64_t b = (uint64_t)(uintptr_t)base;
  return v4u{(uint32_t)b, (uint32_t)(b >> 32) & 0xffffu, bytes, (uint32_t)kRsrcWord3};
}

__device__ __forceinline__ __amdgpu_buffer_rsrc_t rsrc_of(const v4u& r) {
  const uint64_t b = ((uint64_t)r[1] << 32) | r[0];
  return make_rsrc((const void*)(uintptr_t)b, r[2]);
}

// Direct-to-LDS buffer loads (the lane's bytes land at LDS address m0 +
// lane * size), written as inline asm on purpose: the compiler, seeing an LDS
// write it cannot tell apart from the stage being read, would otherwise put
// an s_waitcnt vmcnt(0) before every later LDS read, draining the loads issued
// for the stages ahead.  The kernel waits for each stage with explicit vmcnt
// counts instead.  One wait state separates the m0 write from its use.
__device__ __forceinline__ void dma_load16(const v4u& rsrc, uint32_t voff, uint32_t soff, uint32_t lds) {
  asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tbuffer_load_dwordx4 %0, %2, %3 offen lds"
               :: "v"(voff), "s"(lds), "s"(rsrc), "s"(soff) : "memory", "m0");
}
__device__ __forceinline__ void dma_load4(const v4u& rsrc, uint32_t voff, uint32_t soff, uint32_t lds) {
  asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tbuffer_load_dword %0, %2, %3 offen lds"
               :: "v"(voff), "s"(lds), "s"(rsrc), "s"(soff) : "memory", "m0");
}
// The same with the LDS address given as a base plus a constant, added
// straight into m0 (one scalar instruction instead of an add and a move).
template <uint32_t IMM>
__device__ __forceinline__ void dma_load16_at(const v4u& rsrc, uint32_t voff, uint32_t soff, uint32_t lds) {
  asm volatile("s_add_u32 m0, %1, %4\n\ts_nop 0\n\tbuffer_load_dwordx4 %0, %2, %3 offen lds"
               :: "v"(voff), "s"(lds), "s"(rsrc), "s"(soff), "n"(IMM) : "memory", "m0", "scc");
}
template <uint32_t IMM>
__device__ __forceinline__ void dma_load4_at(const v4u& rsrc, uint32_t voff, uint32_t soff, uint32_t lds) {
  asm volatile("s_add_u32 m0, %1, %4\n\ts_nop 0\n\tbuffer_load_dword %0, %2, %3 offen lds"
               :: "v"(voff), "s"(lds), "s"(rsrc), "s"(soff), "n"(IMM) : "memory", "m0", "scc");
}

template <int N, class F>
__device__ __forceinline__ void static_for(F&& f) {
  if constexpr (N > 0) {
    static_for<N - 1>(f);
    f(std::integral_constant<int, N - 1>{});
  }
}

constexpr int cdiv(int a, int b) { return (a + b - 1) / b; }

// Element formats of the scaled MFMA operands (the instruction's format codes).
enum : int { FMT_E4M3 = 0, FMT_E2M3 = 2, FMT_E3M2 = 3, FMT_E2M1 = 4, FMT_BF16 = -1 };
constexpr int fmt_of_a(int dt) {
  return dt == DT_MXFP4 || dt == DT_MXFP4_MXFP8 ? FMT_E2M1
       : dt == DT_BF16                          ? FMT_BF16
       : dt == DT_MXFP6_E2M3                    ? FMT_E2M3
       : dt == DT_MXFP6_E3M2                    ? FMT_E3M2
                                                : FMT_E4M3;
}
constexpr int fmt_of_b(int dt) {
  return dt == DT_MXFP4_MXFP8 ? FMT_E4M3 : dt == DT_MXFP8_MXFP4 ? FMT_E2M1 : fmt_of_a(dt);
}
constexpr int fmt_bits(int f) { return f == FMT_E4M3 ? 8 : f == FMT_E2M1 ? 4 : f == FMT_BF16 ? 16 : 6; }

// WK > 1 splits each k-step among WK groups of waves: a k-step then covers WK
// consecutive k-slices of KB bytes per row, slice s held in sub-stage s of the
// stage (each laid out as a whole stage of a WK = 1 kernel), and the waves of
// group s multiply slice s into accumulators of their own.  Their sums are
// added once per tile.  A tile too small to give every wave its own output
// block (16 x 32) still gets several waves' loads in flight, and each k-step
// reads WK * KB contiguous bytes of every row.
template <int DT_, int BM_, int BN_, int KB_, int MF_, int WM_, int WN_, int STAGES_, int WK_ = 1>
struct Cfg {
  static constexpr int DT = DT_, BM = BM_, BN = BN_, KB = KB_, MF = MF_, WM = WM_, WN = WN_;
  static constexpr int STAGES = STAGES_;
  static constexpr int WK = WK_;
  static constexpr int OW = WM * WN;                   // waves over the output tile (group 0: waves 0 .. OW-1)
  static constexpr int NW = OW * WK;
  static constexpr int NT = 64 * NW;
  static constexpr int WTM = BM / WM, WTN = BN / WN;   // per-wave tile
  static constexpr int FM = WTM / MF, FN = WTN / MF;   // MFMA blocks per wave
  static constexpr int NG = 64 / MF;                   // K groups across the lanes
  static constexpr int LB = KB / NG;                   // bytes per lane per row per k-step
  // MX: block-scaled operands (E8M0 per 32 K).  WIDE: the LDS image holds 32
  // bytes per 32-element block, one byte per element (E4M3 elements as they
  // are; a 6-bit block's 24 bytes and an E2M1 block's 16 are padded into the
  // 32), so operands of different formats share one layout; only packed E2M1
  // on its own (16 bytes per block) and bf16 are not WIDE.
  static constexpr bool MX = DT != DT_BF16 && DT != DT_FP8;
  static constexpr bool WIDE = DT != DT_MXFP4 && DT != DT_BF16;
  static constexpr int FA = fmt_of_a(DT), FB = fmt_of_b(DT);  // element formats of A and B
  static constexpr int U = WIDE ? 32 : 16;             // LDS bytes per lane per MFMA
  static constexpr int NU = LB / U;                    // MFMAs per block per k-step
  static constexpr int NCH = U / 16;                   // 16-byte chunks per lane per MFMA
  static constexpr int SPR = DT == DT_MXFP4 ? KB / 16 : (MX ? KB / 32 : 0);  // scale bytes per row per k-slice
  static constexpr int BKS = DT == DT_MXFP4 ? 2 * KB : (DT == DT_BF16 ? KB / 2 : KB);   // K per k-slice
  static constexpr int BK = WK * BKS;                  // K per k-step
  // bytes of one row's k-slice in memory (the LDS image of a WIDE block may be padded)
  static constexpr int KBG_A = WIDE ? BKS * fmt_bits(FA) / 8 : KB;
  static constexpr int KBG_B = WIDE ? BKS * fmt_bits(FB) / 8 : KB;
  static constexpr int KSA = WK * KBG_A, KSB = WK * KBG_B;   // ... and of its k-step
  static constexpr int ACC = MF == 32 ? 16 : 4;        // fp32 accumulators per block per lane
  // MX scale bytes a lane reads per k-step: its lane group's NU bytes of each
  // of its FM (FN) blocks, stored contiguously by the scale pre-pass
  static constexpr int NSA = MX ? FM * NU : 1, NSB = MX ? FN * NU : 1;
  static constexpr int SWA = (NSA + 3) / 4, SWB = (NSB + 3) / 4;   // 32-bit words holding them

  // LDS image of one operand k-slice: rows of KB bytes, one after another.  The
  // 16-byte chunks of row r are stored permuted: slot p holds chunk p ^ swz(r),
  // with swz taking bits of r mod 16 (see swz()).  A direct-to-LDS load of one
  // wave fills RG = 1024/KB whole rows, eight (or four) consecutive lanes
  // reading one contiguous row segment from memory; and 16 lanes that read the
  // same chunk of 16 consecutive rows hit 16 different 16-byte bank groups.
  static constexpr int RG = 1024 / KB;
  static constexpr int CPR = KB / 16;                  // chunks per row
  static constexpr int A_GRP = BM / RG, B_GRP = BN / RG;             // row groups per sub-stage
  static constexpr int A_GROUPS = WK * A_GRP, B_GROUPS = WK * B_GRP;  // ... per stage
  // Scale bytes of a k-slice, [row][SPR], filled by dword loads of 64 lanes
  // (256 bytes per instruction), so each area is a whole number of 256 B; a
  // sub-stage is then A rows, B rows, A's scales, B's scales.  SW (k-split
  // kernels): the scale bytes of all WK k-slices of every row, [row][WK *
  // SPR], once per stage after the sub-stages, filled by 16-byte loads (a
  // whole number of 1 KiB per area): a quarter of the load requests, each
  // row's bytes of a k-step being contiguous in the caller's array.
  static constexpr bool SW = WK > 1;
  static constexpr int SROW = SW ? WK * SPR : SPR;     // bytes per row of a scale area
  static constexpr int SUNIT = SW ? 1024 : 256;        // bytes per scale load instruction
  static constexpr int SA_I = MX ? cdiv(BM * SROW, SUNIT) : 0;
  static constexpr int SB_I = MX ? cdiv(BN * SROW, SUNIT) : 0;
  static constexpr int SA_INST = SW ? SA_I : WK * SA_I, SB_INST = SW ? SB_I : WK * SB_I;
  static constexpr int A_OFF = 0;
  static constexpr int B_OFF = BM * KB;
  static constexpr int SUB = (BM + BN) * KB + (SW ? 0 : (SA_I + SB_I) * SUNIT);
  static constexpr int SA_OFF = SW ? WK * SUB : (BM + BN) * KB;   // SW: in the stage; else in each sub-stage
  static constexpr int SB_OFF = SA_OFF + SA_I * SUNIT;
  // SW: A's and B's scale loads share one count per wave; a wave past the
  // last of them issues one with every lane out of range (it writes zeros)
  // into a spare kilobyte of the stage, so every wave issues the same count.
  static constexpr int SPT = SW ? cdiv(SA_INST + SB_INST, NW) : 0;
  static constexpr int JUNK_OFF = SB_OFF + SB_I * SUNIT;
  static constexpr int STAGE = SW ? JUNK_OFF + (SPT * NW > SA_INST + SB_INST ? 1024 : 0) : WK * SUB;
  static constexpr int LDS = STAGES * STAGE;
  // Direct loads per wave per k-step; a wave with nothing left repeats a
  // group (same bytes to the same place), so every wave issues the same count.
  static constexpr int A_PT = cdiv(A_GROUPS, NW), B_PT = cdiv(B_GROUPS, NW);
  static constexpr int SA_PT = SW ? SPT : cdiv(SA_INST, NW), SB_PT = SW ? 0 : cdiv(SB_INST, NW);
  static constexpr int LOADS_PER_STAGE_S = A_PT + B_PT + SA_PT + SB_PT;
  // Loads whose LDS target is a constant plus 1 KiB (scales: 256 B) per wave:
  // every wave has a group of its own in each load (no wrap-around) and a
  // load's NW groups lie in one sub-stage.
  static constexpr bool LIN_A = A_GROUPS % NW == 0 && A_GRP % NW == 0;
  static constexpr bool LIN_B = B_GROUPS % NW == 0 && B_GRP % NW == 0;
  static constexpr bool LIN_S = !SW && MX && SA_INST % NW == 0 && SA_I % NW == 0 && SB_INST % NW == 0 && SB_I % NW == 0;
  // ... and whose loads all give the lane the same chunk of its row (the NW
  // row groups between two of a wave's loads are a whole number of 16-row
  // swizzle periods), so they share one in-row limit
  static constexpr bool LIM1_A = LIN_A && WK == 1 && (NW * RG) % 16 == 0;
  static constexpr bool LIM1_B = LIN_B && WK == 1 && (NW * RG) % 16 == 0;
  // Eight-wave kernels whose operand fragments take 8 VGPRs (E4M3 and the
  // six-bit types, NCH == 2) refill A's fragments in place and double-buffer
  // only B's: two full sets of operands would not fit beside the
  // accumulators in the 128 VGPRs such a wave has.
  static constexpr bool INPLACE = NW >= 8 && NCH == 2;
  static constexpr int P_SLOT = BM * BN;                // floats per scratch slot
  static constexpr int P_WAVE = FM * FN * ACC * 64;     // floats per wave in a slot
  static constexpr int NQ = ACC / 4;                    // 4-column runs per block per lane
  // Output staging (epilogue): per wave, MF rows x SC columns of bf16 in the
  // stage freed by a tile's last k-step, read back as 16-byte row chunks.
  // (wave tiles narrower than 32 columns are stored from registers instead)
  static constexpr bool STAGED = WTN % 32 == 0;
  static constexpr int SC = WTN % 64 == 0 ? 64 : 32;
  static constexpr int SCH = SC / 8;                    // 16-byte chunks per staged row
  static constexpr int SRP = 64 / SCH;                  // staged rows per wave store
  static constexpr int STG_WAVE = MF * SC * 2;
  // WK > 1: waves' accumulators passed between them in the same freed stage,
  // after the output staging: [wave][P_WAVE floats] for finish_split (every
  // wave), [wave - OW][P_WAVE floats] for reduce_k (waves OW .. NW-1)
  static constexpr int RED_OFF = OW * STG_WAVE;
  static constexpr int RED_BYTES = WK > 1 ? WK * OW * P_WAVE * 4 : 0;
  static constexpr int BIAS_OFF = STAGES * STAGE;       // bf16 bias of the current tile
  static constexpr int LDS_TOTAL = BIAS_OFF + BN * 2;

  static_assert(MF == 32 || MF == 16, "MFMA shape");
  static_assert(WTM % MF == 0 && WTN % MF == 0, "wave tile must be whole MFMA blocks");
  static_assert(LB % U == 0 && NU >= 1, "k-step must give each lane whole MFMA operands");
  static_assert(KB == 64 || KB == 128, "k-step bytes per row");
  static_assert(BM % RG == 0 && BN % RG == 0, "row groups tile the operands");
  static_assert(MF % 16 == 0, "MFMA blocks cover whole 16-row swizzle periods");
  static_assert(!MX || SPR == 2 || SPR == 4 || SPR == 8, "scale bytes per row per k-step");
  static_assert(NSA <= 16 && NSB <= 16 && (NSA & (NSA - 1)) == 0 && (NSB & (NSB - 1)) == 0, "packed scale reads");
  static_assert(STAGES >= 2 && STAGES <= 8, "pipeline depth");
  static_assert((STAGES - 2) * LOADS_PER_STAGE_S <= 63, "vmcnt range");
  static_assert(LDS_TOTAL <= 160 * 1024, "LDS");
  static_assert(BN <= NT, "one bias element per thread");
  static_assert(RED_OFF + RED_BYTES <= STAGE, "output staging and the k-split sums fit in one stage");
  static_assert(WK == 1 || WK == 2 || WK == 4, "k-split");
  static_assert(!SW || !MX || SROW % 16 == 0, "16-byte scale loads cover whole row segments");
  static_assert(!STAGED || (WTN % SC == 0 && SC % MF == 0 && MF % SRP == 0), "output staging windows");
};

template <class C>
struct Acc {
  typedef typename std::conditional<C::MF == 32, v16f, v4f>::type T;
  T v[C::FM][C::FN];
  __device__ __forceinline__ void zero() {
#pragma unroll
    for (int i = 0; i < C::FM; ++i)
#pragma unroll
      for (int j = 0; j < C::FN; ++j) v[i][j] = T{};
  }
};

// ---------------------------------------------------------------- MFMA wrappers

// A lane's eight operand registers of one MFMA for element format FMT, from its
// LDS reads: E4M3 takes both 16-byte chunks; a 6-bit block (24 bytes) the first
// chunk and the 8 bytes read from the second (see read_chunk); E2M1 (16 bytes)
// the first chunk.  Registers past the format's size are not read by the MFMA.
template <class C, int FMT>
__device__ __forceinline__ v8i mfma_operand(const v4u* x) {
  v8i v;
  v[0] = x[0][0]; v[1] = x[0][1]; v[2] = x[0][2]; v[3] = x[0][3];
  if constexpr (C::WIDE && FMT == FMT_E4M3) {
    v[4] = x[1][0]; v[5] = x[1][1]; v[6] = x[1][2]; v[7] = x[1][3];
  } else if constexpr (C::WIDE && (FMT == FMT_E2M3 || FMT == FMT_E3M2)) {
    v[4] = x[1][0]; v[5] = x[1][1]; v[6] = 0; v[7] = 0;
  } else {
    v[4] = v[5] = v[6] = v[7] = 0;
  }
  return v;
}

// One MFMA block of C, computed as the transposed product (B block x A block):
// lane l then holds C row (l % MF) and, for each accumulator quad, four
// consecutive columns, which the epilogue stores as one 8-byte run.
template <class C, int OPA, int OPB>
__device__ __forceinline__ void mfma(typename Acc<C>::T& acc, const v4u* a, const v4u* b, int sa, int sb) {
  if constexpr (C::DT == DT_BF16) {
    v8bf va = __builtin_bit_cast(v8bf, a[0]);
    v8bf vb = __builtin_bit_cast(v8bf, b[0]);
    if constexpr (C::MF == 32)
      acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vb, va, acc, 0, 0, 0);
    else
      acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vb, va, acc, 0, 0, 0);
  } else {
    const v8i va = mfma_operand<C, C::FA>(a), vb = mfma_operand<C, C::FB>(b);
    // the first operand is B's block (the transposed product): its format comes first
    if constexpr (C::DT == DT_FP8) {
      // no block scales: with both scale operands 0 (and op_sel 0) the
      // compiler emits the unscaled f8f6f4 instruction, which multiplies by 1
      // and leaves the two scale registers free
      if constexpr (C::MF == 32)
        acc = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(vb, va, acc, C::FB, C::FA, 0, 0, 0, 0);
      else
        acc = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(vb, va, acc, C::FB, C::FA, 0, 0, 0, 0);
    } else if constexpr (C::MF == 32) {
      acc = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(vb, va, acc, C::FB, C::FA, OPB, sb, OPA, sa);
    } else {
      acc = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(vb, va, acc, C::FB, C::FA, OPB, sb, OPA, sa);
    }
  }
}

// ---------------------------------------------------------------- epilogue rounding

typedef __bf16 v2bf __attribute__((ext_vector_type(2)));
typedef float v2f __attribute__((ext_vector_type(2)));

// Four outputs bf16(t[k] + b[k]) of the exact sums, correctly rounded to
// nearest-even, as two packed words.  Each sum is taken twice, rounded toward
// -inf and toward +inf (the wave's fp32 rounding mode is switched around the
// adds and restored to nearest-even).  Of the two, the one with an odd last
// bit is the sum rounded to odd (both are the sum when it is exact), and an
// fp32 rounded to odd carries more than two bits beyond bf16, so converting
// it to bf16 to nearest-even gives the correctly rounded result; NaN, infinity
// and signed zeros come out as the nearest-even sum would give them.  The
// adds are inline asm so that no compiler-scheduled float operation can fall
// between the mode switches; each switch is followed by the two wait states
// a mode change needs before a VALU instruction.
__device__ __forceinline__ v2u round_run(const float t[4], const float b[4]) {
  float dn[4], up[4];
  asm volatile(
      "s_setreg_imm32_b32 hwreg(HW_REG_MODE, 0, 2), 2\n\t"
      "s_nop 1\n\t"
      "v_add_f32 %0, %8, %12\n\t"
      "v_add_f32 %1, %9, %13\n\t"
      "v_add_f32 %2, %10, %14\n\t"
      "v_add_f32 %3, %11, %15\n\t"
      "s_setreg_imm32_b32 hwreg(HW_REG_MODE, 0, 2), 1\n\t"
      "s_nop 1\n\t"
      "v_add_f32 %4, %8, %12\n\t"
      "v_add_f32 %5, %9, %13\n\t"
      "v_add_f32 %6, %10, %14\n\t"
      "v_add_f32 %7, %11, %15\n\t"
      "s_setreg_imm32_b32 hwreg(HW_REG_MODE, 0, 2), 0\n\t"
      "s_nop 1"
      : "=&v"(dn[0]), "=&v"(dn[1]), "=&v"(dn[2]), "=&v"(dn[3]), "=&v"(up[0]), "=&v"(up[1]), "=&v"(up[2]),
        "=&v"(up[3])
      : "v"(t[0]), "v"(t[1]), "v"(t[2]), "v"(t[3]), "v"(b[0]), "v"(b[1]), "v"(b[2]), "v"(b[3]));
  // the odd one of the two: a mask of the low bit of the rounded-down sum
  // (all ones when it is odd), then a bitfield select (two VALU ops)
  float o[4];
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    // (written out: the compiler would turn the plain form back into a compare and a select)
    uint32_t m, r;
    asm("v_bfe_i32 %0, %1, 0, 1" : "=v"(m) : "v"(dn[k]));
    asm("v_bfi_b32 %0, %1, %2, %3" : "=v"(r) : "v"(m), "v"(dn[k]), "v"(up[k]));
    o[k] = __uint_as_float(r);
  }
  v2u h;
  h[0] = __builtin_bit_cast(uint32_t, __builtin_convertvector((v2f{o[0], o[1]}), v2bf));
  h[1] = __builtin_bit_cast(uint32_t, __builtin_convertvector((v2f{o[2], o[3]}), v2bf));
  return h;
}

// Index of this thread's wave; the same for all its lanes, which the compiler
// cannot infer from threadIdx, so it is made explicitly uniform.
__device__ __forceinline__ int wave_id() { return __builtin_amdgcn_readfirstlane(threadIdx.x >> 6); }

// The launch arguments, read afresh from the kernel argument segment at each
// call.  Outside the main loop every argument is fetched where it is used
// instead of being held in scalar registers for the whole kernel (the
// arguments alone would take half of them).  The empty asm hides the pointer's
// origin, so the loads are neither merged nor hoisted; they stay scalar loads.
__device__ __forceinline__ const KArgs& kargs() {
  const __attribute__((address_space(4))) uint8_t* p =
      (const __attribute__((address_space(4))) uint8_t*)__builtin_amdgcn_kernarg_segment_ptr();
  asm volatile("" : "+s"(p));
  return *(const KArgs*)p;
}

// Workgroup barrier for the main loop.  __syncthreads() also waits for every
// outstanding global load (vmcnt(0)), which would drain the direct-to-LDS
// loads issued for later stages; here each wave has already waited for the
// loads of the stage about to be read, so only LDS traffic must settle.
__device__ __forceinline__ void lds_barrier() {
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

template <int N>
__device__ __forceinline__ void wait_vmcnt_n() {
  if constexpr (N == 0) asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  else asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

// s_waitcnt vmcnt(n) for a run-time n in [0, MAX] (the count is an immediate).
template <int MAX>
__device__ __forceinline__ void wait_vmcnt(int n) {
  static_for<MAX + 1>([&](auto c) {
    constexpr int k = decltype(c)::value;
    if (n == k) {
      if constexpr (k == 0) asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
      else asm volatile("s_waitcnt vmcnt(%0)" ::"n"(k) : "memory");
    }
  });
}

// ---------------------------------------------------------------- the kernel body

// DIRECT: MX scales are gathered straight from the caller's [rows][K/32]
// arrays (a k-step's SPR bytes of each row land in LDS as [row][SPR]), with no
// re-layout pass before the launch; a lane then reads its blocks' scale bytes
// one block at a time.  Needs SPR >= 4 (a dword of a row never spans two rows)
// and K a multiple of the k-step (no k-step reads past a row's last scale).
template <class C, bool DIRECT = false>
struct Kernel {
  static constexpr int NT = C::NT;
  static_assert(!DIRECT || (C::MX && C::SPR >= 4), "direct scale reads need MX scales, at least 4 bytes per row");
  static_assert(C::WK == 1 || DIRECT, "k-split kernels read the caller's scales (the re-laid copy has one k-slice per k-step)");

  struct TileCtx {
    v4u ra, rb, rsa, rsb;   // A, B and (MXFP4) their scales, from the tile's first row
  };

  // Per-lane 32-bit buffer offsets of this wave's direct-to-LDS loads, fixed
  // for a launch.  Row group g of a stage is group g % A_GRP of sub-stage
  // g / A_GRP (B likewise), which holds k-slice g / A_GRP of the k-step.  Lane
  // j of a data load fills slot j % CPR of row (group*RG + j / CPR), so it
  // fetches that row's chunk (j % CPR) ^ swz(row) of the k-slice; lane j of a
  // scale load takes bytes [inst*256 + 4j, +4) of the k-slice's scale block
  // ([row][SPR]).  Rows past M or N lie outside the tile's buffer resource and
  // read as zero.
  struct LoadOffs {
    uint32_t a[C::A_PT];     // lane's row offset plus chunk offset, per load
    uint32_t b[C::B_PT];
    // per load: the k-step byte offsets k for which the lane's chunk lies
    // inside the row, k < lim (a chunk at byte c of the k-step: lim = row bytes
    // - c, or 0 for a padding chunk or one past the row at every k)
    uint32_t lim_a[C::A_PT];
    uint32_t lim_b[C::B_PT];
    uint32_t sa[C::SA_PT > 0 ? C::SA_PT : 1];
    uint32_t sb[C::SB_PT > 0 ? C::SB_PT : 1];
  };
  struct Ops {
    v4u a[C::FM][C::NCH];
    v4u b[C::FN][C::NCH];
  };
  // A lane's scale bytes of one k-step: byte i * NU + u is block i's scale in
  // sub-step u (0x7f, a factor of 1, for the unscaled types).
  struct Scales {
    uint32_t a[C::SWA];
    uint32_t b[C::SWB];
  };
  struct LdsPtrs {
    const lds_u8* a;                 // lane's row in block 0 of its A rows
    const lds_u8* b;
    int slot_a[C::NU * C::NCH];      // byte offset of the lane's A chunk for (sub-step, half)
    int slot_b[C::NU * C::NCH];      // the same for B (differs when the formats do)
    int sa, sb;                      // byte offsets of the lane's packed scale bytes inside a stage
  };

  static __device__ __forceinline__ lds_u8* stage_ptr(lds_u8* smem, int s) { return smem + s * C::STAGE; }

  static __device__ __forceinline__ TileCtx tile_ctx(const KArgs& a, int tile) {
    TileCtx t;
    const int tm = tile / a.tiles_n, tn = tile - tm * a.tiles_n;
    const int m0 = tm * C::BM, n0 = tn * C::BN;
    const int rows_a = min(C::BM, a.M - m0);
    const int rows_b = min(C::BN, a.N - n0);
    t.ra = rsrc_words(a.A + (int64_t)m0 * a.row_bytes, (uint32_t)(rows_a * a.row_bytes));
    t.rb = rsrc_words(a.B + (int64_t)n0 * a.row_bytes_b, (uint32_t)(rows_b * a.row_bytes_b));
    if constexpr (DIRECT) {
      // the caller's scales: the tile's rows, [row][s_pitch]; k-step ks reads
      // at scalar offset ks * sa_kstride (its first byte in a row), and since
      // K is a whole number of k-steps every byte read lies inside the tile's rows
      t.rsa = rsrc_words(a.SA + (int64_t)m0 * a.s_pitch, (uint32_t)(rows_a * a.s_pitch));
      t.rsb = rsrc_words(a.SB + (int64_t)n0 * a.s_pitch, (uint32_t)(rows_b * a.s_pitch));
    } else if constexpr (C::MX) {
      // k-step-major scales, a tile's k-step block of BM * SPR bytes at
      // SA + ks * sa_kstride + m0 * SPR in the packed lane order; k-step ks
      // reads at scalar offset ks * sa_kstride.  The scale copy holds whole
      // tiles (rows past M carry 127), so the range ends with the tile's block
      // of the last k-step.
      t.rsa = rsrc_words(a.SA + (int64_t)m0 * C::SPR, (uint32_t)(a.iters - 1) * a.sa_kstride + C::BM * C::SPR);
      t.rsb = rsrc_words(a.SB + (int64_t)n0 * C::SPR, (uint32_t)(a.iters - 1) * a.sb_kstride + C::BN * C::SPR);
    } else {
      t.rsa = t.ra;
      t.rsb = t.rb;
    }
    return t;
  }

  // Byte offset, in a row's k-step in memory, of what LDS chunk c of that row
  // holds, for element format FMT; kNone where the chunk is padding.  A WIDE
  // block of 32 elements takes chunks 2i and 2i+1: E4M3 bytes [32i, +32); a
  // 6-bit block's bytes [24i, +16) and [24i + 8, +16) (so no read goes past
  // the block; the second chunk's upper 8 bytes are the block's bytes 16..23);
  // an E2M1 block's 16 bytes [16i, +16) in the first chunk only.
  static constexpr uint32_t kNone = 0x40000000u;
  template <int FMT>
  static __device__ __forceinline__ uint32_t gchunk(int c) {
    if constexpr (!C::WIDE || FMT == FMT_E4M3) return (uint32_t)(16 * c);
    else if constexpr (FMT == FMT_E2M1) return (c & 1) ? kNone : (uint32_t)(16 * (c >> 1));
    else return (uint32_t)(24 * (c >> 1) + 8 * (c & 1));
  }

  static __device__ __forceinline__ LoadOffs load_offsets(const KArgs& a) {
    const int lane = threadIdx.x & 63, wave = wave_id();
    const int rr = lane / C::CPR, p = lane % C::CPR;
    LoadOffs o;
#pragma unroll
    for (int i = 0; i < C::A_PT; ++i) {
      const int grp = (wave + i * C::NW) % C::A_GROUPS;
      const int row = (grp % C::A_GRP) * C::RG + rr;
      const uint32_t c = gchunk<C::FA>(p ^ swz(row));
      const uint32_t ca = c == kNone ? kNone : (uint32_t)(grp / C::A_GRP) * C::KBG_A + c;
      o.a[i] = c == kNone ? kOob : (uint32_t)row * (uint32_t)a.row_bytes + ca;
      o.lim_a[i] = ca < (uint32_t)a.row_bytes ? (uint32_t)a.row_bytes - ca : 0u;
    }
#pragma unroll
    for (int i = 0; i < C::B_PT; ++i) {
      const int grp = (wave + i * C::NW) % C::B_GROUPS;
      const int row = (grp % C::B_GRP) * C::RG + rr;
      const uint32_t c = gchunk<C::FB>(p ^ swz(row));
      const uint32_t cb = c == kNone ? kNone : (uint32_t)(grp / C::B_GRP) * C::KBG_B + c;
      o.b[i] = c == kNone ? kOob : (uint32_t)row * (uint32_t)a.row_bytes_b + cb;
      o.lim_b[i] = cb < (uint32_t)a.row_bytes_b ? (uint32_t)a.row_bytes_b - cb : 0u;
    }
    if constexpr (C::MX) {
      // the k-slice's scale bytes of the tile's rows are contiguous ([row][SPR])
      // (DIRECT: byte `byte` of the [row][SPR] block of k-slice s is byte
      // s * SPR + byte % SPR of the k-step's scales in row byte / SPR of the
      // caller's array)
      // (SW: byte `byte` of the [row][SROW] area is byte byte % SROW of the
      // k-step's scales in row byte / SROW, 16 bytes per lane)
      auto scale_src = [&](int ins, int rows, int per) -> uint32_t {
        if constexpr (C::SW) {
          const int byte = ins * 1024 + lane * 16;
          return byte < rows * C::SROW ? (uint32_t)(byte / C::SROW) * (uint32_t)a.s_pitch + (uint32_t)(byte % C::SROW)
                                       : kOob;
        } else {
          const int byte = (ins % per) * 256 + lane * 4;
          const uint32_t src = DIRECT ? (uint32_t)(byte / C::SPR) * (uint32_t)a.s_pitch +
                                            (uint32_t)((ins / per) * C::SPR + byte % C::SPR)
                                      : (uint32_t)byte;
          return byte < rows * C::SPR ? src : kOob;
        }
      };
      if constexpr (C::SW) {
        // scale load i of this wave: A's instruction wave + i*NW, else B's, else none
#pragma unroll
        for (int i = 0; i < C::SA_PT; ++i) {
          const int idx = wave + i * C::NW;
          o.sa[i] = idx < C::SA_INST ? scale_src(idx, C::BM, 0)
                  : idx < C::SA_INST + C::SB_INST ? scale_src(idx - C::SA_INST, C::BN, 0) : kOob;
        }
      } else {
#pragma unroll
        for (int i = 0; i < C::SA_PT; ++i) o.sa[i] = scale_src((wave + i * C::NW) % C::SA_INST, C::BM, C::SA_I);
#pragma unroll
        for (int i = 0; i < C::SB_PT; ++i) o.sb[i] = scale_src((wave + i * C::NW) % C::SB_INST, C::BN, C::SB_I);
      }
    }
    return o;
  }

  // Chunk permutation of row r: for 128-byte rows, rows 2k and 2k+1 share the
  // value k (mod 8) and sit on opposite halves of the banks; for 64-byte rows,
  // rows 4k..4k+3 share k (mod 4) and fill the four bank quarters.
  static __device__ __forceinline__ constexpr int swz(int r) {
    return C::KB == 128 ? (r >> 1) & 7 : (r >> 2) & 3;
  }

  static __device__ __forceinline__ LdsPtrs lds_ptrs(const lds_u8* smem) {
    const int lane = threadIdx.x & 63, wave = wave_id();
    const int ow = wave % C::OW, wk = wave / C::OW;   // output wave, k-slice
    const int wm = ow / C::WN, wn = ow % C::WN;
    const int lr = lane % C::MF, g = lane / C::MF;
    LdsPtrs p;
    // Block rows start at multiples of 16, so the lane's permutation is swz(lr).
    const int x = swz(lr);
    // 16-byte chunk of the k-step row that (lane group g, sub-step u, operand
    // half h) reads.  With E4M3 elements the scaled MFMA takes register half h
    // of lane group g as K elements [h*16*NG + 16g, +16) of its K range, and
    // the scale of its 32-element block b from lane group b; so for
    // block-scaled E4M3 each hardware block is filled with the k-step's block
    // b*NU + u, whose scale byte lane group b holds at op_sel u.  E2M1 and the
    // 6-bit formats take a lane group's 32 elements as one contiguous K range
    // (checked on the device), so lane group g's operands are its own blocks
    // g*NU + u, the same k-step block in the same hardware block as above;
    // operands of different formats therefore pair the same K.
    auto chunk = [&](int fmt, int u, int h) {
      if (C::MX && C::WIDE && fmt == FMT_E4M3) return 2 * ((h * (C::NG / 2) + g / 2) * C::NU + u) + g % 2;
      return g * (C::LB / 16) + u * C::NCH + h;
    };
#pragma unroll
    for (int u = 0; u < C::NU; ++u)
#pragma unroll
      for (int h = 0; h < C::NCH; ++h) {
        p.slot_a[u * C::NCH + h] = (chunk(C::FA, u, h) ^ x) * 16;
        p.slot_b[u * C::NCH + h] = (chunk(C::FB, u, h) ^ x) * 16;
      }
    // the wave's k-slice is sub-stage wk of every stage
    p.a = smem + wk * C::SUB + C::A_OFF + (wm * C::WTM + lr) * C::KB;
    p.b = smem + wk * C::SUB + C::B_OFF + (wn * C::WTN + lr) * C::KB;
    if constexpr (DIRECT) {
      // [row][SPR]: the lane's row in block 0, its lane group's NU bytes
      // [row][SROW]: the lane's row in block 0, its k-slice's bytes, its lane group's NU bytes
      const int slice = C::SW ? wk * C::SPR : wk * C::SUB;
      p.sa = slice + C::SA_OFF + (wm * C::WTM + lr) * C::SROW + g * C::NU;
      p.sb = slice + C::SB_OFF + (wn * C::WTN + lr) * C::SROW + g * C::NU;
    } else {
      // packed order of a tile's k-step scales: [wave row][lane row][lane group][block][sub-step]
      p.sa = C::SA_OFF + ((wm * C::MF + lr) * C::NG + g) * C::NSA;
      p.sb = C::SB_OFF + ((wn * C::MF + lr) * C::NG + g) * C::NSB;
    }
    return p;
  }

  // The lane's n packed scale bytes (n = 1, 2, 4, 8 or 16) in one LDS read.
  template <int NB, int NW>
  static __device__ __forceinline__ void read_packed(const lds_u8* p, uint32_t (&w)[NW]) {
    typedef const __attribute__((address_space(3))) uint8_t* P8;
    if constexpr (NB == 1) w[0] = *(P8)p;
    else if constexpr (NB == 2) w[0] = *(const __attribute__((address_space(3))) uint16_t*)p;
    else if constexpr (NB == 4) w[0] = *(const __attribute__((address_space(3))) uint32_t*)p;
    else if constexpr (NB == 8) {
      const v2u x = *(const __attribute__((address_space(3))) v2u*)p;
      w[0] = x[0];
      w[1] = x[1];
    } else {
      const v4u x = *(const __attribute__((address_space(3))) v4u*)p;
      w[0] = x[0];
      w[1] = x[1];
      w[2] = x[2];
      w[3] = x[3];
    }
  }
  // DIRECT: the NU bytes of each of NB blocks (MF rows apart in the [row][SPR]
  // image), placed where the packed read would put them (block i at byte i * NU).
  template <int NB, int NW>
  static __device__ __forceinline__ void read_blocks(const lds_u8* p, uint32_t (&w)[NW]) {
#pragma unroll
    for (int k = 0; k < NW; ++k) w[k] = 0;
#pragma unroll
    for (int i = 0; i < NB; ++i) {
      const lds_u8* q = p + i * C::MF * C::SROW;
      uint32_t x;
      if constexpr (C::NU == 1) x = *q;
      else if constexpr (C::NU == 2) x = *(const __attribute__((address_space(3))) uint16_t*)q;
      else x = *(const __attribute__((address_space(3))) uint32_t*)q;
      w[(i * C::NU) / 4] |= x << (8 * ((i * C::NU) % 4));
    }
  }
  static __device__ __forceinline__ void read_scale_a(const lds_u8* st, const LdsPtrs& p, Scales& sc) {
    if constexpr (DIRECT) read_blocks<C::FM>(st + p.sa, sc.a);
    else if constexpr (C::MX) read_packed<C::NSA>(st + p.sa, sc.a);
  }
  static __device__ __forceinline__ void read_scale_b(const lds_u8* st, const LdsPtrs& p, Scales& sc) {
    if constexpr (DIRECT) read_blocks<C::FN>(st + p.sb, sc.b);
    else if constexpr (C::MX) read_packed<C::NSB>(st + p.sb, sc.b);
  }
  static __device__ __forceinline__ void read_scales(const lds_u8* st, const LdsPtrs& p, Scales& sc) {
    if constexpr (C::MX) {
      read_scale_a(st, p, sc);
      read_scale_b(st, p, sc);
    } else {
      sc.a[0] = 0x7f7f7f7f;   // unit E8M0 block scales
      sc.b[0] = 0x7f7f7f7f;
    }
  }
  // Scale word and op_sel byte of block i in sub-step u.
  static constexpr int sbyte(int i, int u) { return i * C::NU + u; }

  // One operand chunk (half H) of element format FMT from LDS: 16 bytes; the
  // second chunk of a 6-bit block only its upper 8 bytes (the block's bytes
  // 16..23, registers 4 and 5 of the operand); nothing for the empty second
  // chunk of an E2M1 block in a WIDE image.
  template <int FMT, int H>
  static __device__ __forceinline__ void read_chunk(v4u& dst, const lds_u8* q) {
    if constexpr (C::WIDE && FMT == FMT_E2M1 && H == 1) {
    } else if constexpr (C::WIDE && (FMT == FMT_E2M3 || FMT == FMT_E3M2) && H == 1) {
      const v2u x = *(const __attribute__((address_space(3))) v2u*)(q + 8);
      dst[0] = x[0];
      dst[1] = x[1];
    } else {
      dst = *(const __attribute__((address_space(3))) v4u*)q;
    }
  }

  // LDS operands of sub-step U (one MFMA K slice) of the stage at byte offset `so`.
  template <int U>
  static __device__ __forceinline__ void read_ops(int so, const LdsPtrs& p, Ops& o) {
    static_for<C::NCH>([&](auto hc) {
      constexpr int h = decltype(hc)::value;
      const int offa = so + p.slot_a[U * C::NCH + h], offb = so + p.slot_b[U * C::NCH + h];
#pragma unroll
      for (int i = 0; i < C::FM; ++i) read_chunk<C::FA, h>(o.a[i][h], p.a + offa + i * C::MF * C::KB);
#pragma unroll
      for (int j = 0; j < C::FN; ++j) read_chunk<C::FB, h>(o.b[j][h], p.b + offb + j * C::MF * C::KB);
    });
  }

  // The operand reads of one sub-step, one at a time, A and B blocks
  // interleaved (A0, B0, A1, B1, ...) so that the first MFMAs of a sub-step
  // find their operands first.
  static constexpr int NRD = (C::FM + C::FN) * C::NCH;   // operand reads per sub-step
  static constexpr int NSR = C::MX ? 2 : 0;               // packed scale reads per stage (A's, B's)
  struct ReadDesc {
    bool a;
    int blk, h;
  };
  static constexpr ReadDesc read_desc(int r) {
    const int h = r % C::NCH;
    int k = r / C::NCH;
    const int m = C::FM > C::FN ? C::FM : C::FN;
    for (int t = 0; t < m; ++t) {
      if (t < C::FM) {
        if (k == 0) return ReadDesc{true, t, h};
        --k;
      }
      if (t < C::FN) {
        if (k == 0) return ReadDesc{false, t, h};
        --k;
      }
    }
    return ReadDesc{true, 0, 0};
  }
  template <int U, int R>
  static __device__ __forceinline__ void read_op(int so, const LdsPtrs& p, Ops& o) {
    constexpr ReadDesc d = read_desc(R);
    if constexpr (d.a)
      read_chunk<C::FA, d.h>(o.a[d.blk][d.h], p.a + so + p.slot_a[U * C::NCH + d.h] + d.blk * C::MF * C::KB);
    else
      read_chunk<C::FB, d.h>(o.b[d.blk][d.h], p.b + so + p.slot_b[U * C::NCH + d.h] + d.blk * C::MF * C::KB);
  }
  // MFMA order inside a sub-step, in "shells" that follow the read order:
  // once A_t and B_t are in, every block (i, j) with max(i, j) == t can go.
  struct BlockIJ {
    int i, j;
  };
  static constexpr BlockIJ block_of(int b) {
    const int m = C::FM > C::FN ? C::FM : C::FN;
    for (int t = 0; t < m; ++t) {
      for (int j = 0; j < t; ++j)
        if (t < C::FM && j < C::FN) {
          if (b == 0) return BlockIJ{t, j};
          --b;
        }
      for (int i = 0; i < t; ++i)
        if (i < C::FM && t < C::FN) {
          if (b == 0) return BlockIJ{i, t};
          --b;
        }
      if (t < C::FM && t < C::FN) {
        if (b == 0) return BlockIJ{t, t};
        --b;
      }
    }
    return BlockIJ{0, 0};
  }
  // Reads after the barrier, in the order the next k-step's first MFMAs need
  // them: A's packed scales, A_0's operand, B's packed scales, B_0's operand,
  // then A_t's and B_t's operands for t >= 1 (R < NSR + NRD).
  struct PostRead {
    bool scale, a;
    int blk, h;
  };
  static constexpr PostRead post_read(int r) {
    const int m = C::FM > C::FN ? C::FM : C::FN;
    for (int t = 0; t < m; ++t) {
      if (t < C::FM) {
        if (C::MX && t == 0) {
          if (r == 0) return PostRead{true, true, 0, 0};
          --r;
        }
        for (int h = 0; h < C::NCH; ++h) {
          if (r == 0) return PostRead{false, true, t, h};
          --r;
        }
      }
      if (t < C::FN) {
        if (C::MX && t == 0) {
          if (r == 0) return PostRead{true, false, 0, 0};
          --r;
        }
        for (int h = 0; h < C::NCH; ++h) {
          if (r == 0) return PostRead{false, false, t, h};
          --r;
        }
      }
    }
    return PostRead{false, true, 0, 0};
  }
  template <int R>
  static __device__ __forceinline__ void post_read_one(const lds_u8* st, int so, const LdsPtrs& p, Scales& sc, Ops& o) {
    constexpr PostRead d = post_read(R);
    if constexpr (d.scale) {
      if constexpr (d.a) read_scale_a(st, p, sc);
      else read_scale_b(st, p, sc);
    } else {
      if constexpr (d.a)
        read_chunk<C::FA, d.h>(o.a[d.blk][d.h], p.a + so + p.slot_a[d.h] + d.blk * C::MF * C::KB);
      else
        read_chunk<C::FB, d.h>(o.b[d.blk][d.h], p.b + so + p.slot_b[d.h] + d.blk * C::MF * C::KB);
    }
  }

  // MFMA slot B of sub-step U with A's fragments from oa and B's from ob.
  template <int U, int B>
  static __device__ __forceinline__ void mfma_ab(const Ops& oa, const Ops& ob, const Scales& sc, Acc<C>& acc) {
    constexpr BlockIJ bij = block_of(B);
    constexpr int i = bij.i, j = bij.j;
    constexpr int ba = C::MX ? sbyte(i, U) : 0, bb = C::MX ? sbyte(j, U) : 0;
    mfma<C, ba % 4, bb % 4>(acc.v[i][j], oa.a[i], ob.b[j], (int)sc.a[ba / 4], (int)sc.b[bb / 4]);
  }
  // The slot of sub-step order in which A's fragment I is used for the last time.
  static constexpr int last_use_a(int i) {
    int l = -1;
    for (int b = 0; b < C::FM * C::FN; ++b)
      if (block_of(b).i == i) l = b;
    return l;
  }
  // A's fragment I (both halves) / B's fragment J of sub-step U, from the stage at byte offset so.
  template <int U, int I>
  static __device__ __forceinline__ void read_a(int so, const LdsPtrs& p, Ops& o) {
    static_for<C::NCH>([&](auto hc) {
      constexpr int h = decltype(hc)::value;
      read_chunk<C::FA, h>(o.a[I][h], p.a + so + p.slot_a[U * C::NCH + h] + I * C::MF * C::KB);
    });
  }
  template <int U, int J, int H>
  static __device__ __forceinline__ void read_b(int so, const LdsPtrs& p, Ops& o) {
    read_chunk<C::FB, H>(o.b[J][H], p.b + so + p.slot_b[U * C::NCH + H] + J * C::MF * C::KB);
  }

  template <int U, int B>
  static __device__ __forceinline__ void mfma_one(const Ops& o, const Scales& sc, Acc<C>& acc) {
    constexpr BlockIJ bij = block_of(B);
    constexpr int i = bij.i, j = bij.j;
    constexpr int ba = C::MX ? sbyte(i, U) : 0, bb = C::MX ? sbyte(j, U) : 0;
    mfma<C, ba % 4, bb % 4>(acc.v[i][j], o.a[i], o.b[j], (int)sc.a[ba / 4], (int)sc.b[bb / 4]);
  }

  // One direct-to-LDS load of a k-step, by its index P among the k-step's
  // LOADS_PER_STAGE_S loads (A row groups, then B, then the two scale areas;
  // each into the sub-stage of its k-slice).  Past the end of the work list
  // the last k-step's loads are issued again, into a stage nobody reads, so
  // that every k-step issues the same number of loads.
  struct DmaCtx {
    TileCtx t;
    uint32_t kbyte_a, kbyte_b;   // the k-step's byte offset in a row of A and of B
    uint32_t ks_a, ks_b;         // scalar offsets of the k-step's scale bytes
    uint32_t lds;                // LDS address of the target stage
    uint32_t w16, w4;            // ... plus 1 KiB (256 B) per wave below this one (the LIN_ loads' base)
    uint32_t wave;
  };
  template <int P>
  static __device__ __forceinline__ void dma_piece(const DmaCtx& d, const LoadOffs& o) {
    const uint32_t wave = d.wave;
    if constexpr (P < C::A_PT) {
      constexpr int i = P;
      const uint32_t voff = d.kbyte_a < o.lim_a[C::LIM1_A ? 0 : i] ? o.a[i] : kOob;
      if constexpr (C::LIN_A) {
        constexpr uint32_t g0 = i * C::NW;   // wave 0's row group
        dma_load16_at<(g0 / C::A_GRP) * C::SUB + C::A_OFF + (g0 % C::A_GRP) * 1024>(d.t.ra, voff, d.kbyte_a, d.w16);
      } else {
        const uint32_t grp = (wave + i * C::NW) % C::A_GROUPS;
        dma_load16(d.t.ra, voff, d.kbyte_a, d.lds + (grp / C::A_GRP) * C::SUB + C::A_OFF + (grp % C::A_GRP) * 1024);
      }
    } else if constexpr (P < C::A_PT + C::B_PT) {
      constexpr int i = P - C::A_PT;
      const uint32_t voff = d.kbyte_b < o.lim_b[C::LIM1_B ? 0 : i] ? o.b[i] : kOob;
      if constexpr (C::LIN_B) {
        constexpr uint32_t g0 = i * C::NW;
        dma_load16_at<(g0 / C::B_GRP) * C::SUB + C::B_OFF + (g0 % C::B_GRP) * 1024>(d.t.rb, voff, d.kbyte_b, d.w16);
      } else {
        const uint32_t grp = (wave + i * C::NW) % C::B_GROUPS;
        dma_load16(d.t.rb, voff, d.kbyte_b, d.lds + (grp / C::B_GRP) * C::SUB + C::B_OFF + (grp % C::B_GRP) * 1024);
      }
    } else if constexpr (P < C::A_PT + C::B_PT + C::SA_PT) {
      constexpr int i = P - C::A_PT - C::B_PT;
      if constexpr (C::SW) {
        const uint32_t idx = wave + i * C::NW;
        if (idx < C::SA_INST) dma_load16(d.t.rsa, o.sa[i], d.ks_a, d.lds + C::SA_OFF + idx * 1024);
        else if (idx < C::SA_INST + C::SB_INST)
          dma_load16(d.t.rsb, o.sa[i], d.ks_b, d.lds + C::SB_OFF + (idx - C::SA_INST) * 1024);
        else dma_load16(d.t.rsa, kOob, 0u, d.lds + C::JUNK_OFF);
      } else if constexpr (C::LIN_S) {
        constexpr uint32_t n0 = i * C::NW;   // wave 0's instruction
        dma_load4_at<(n0 / C::SA_I) * C::SUB + C::SA_OFF + (n0 % C::SA_I) * 256>(d.t.rsa, o.sa[i], d.ks_a, d.w4);
      } else {
        const uint32_t ins = (wave + i * C::NW) % C::SA_INST;
        dma_load4(d.t.rsa, o.sa[i], d.ks_a, d.lds + (ins / C::SA_I) * C::SUB + C::SA_OFF + (ins % C::SA_I) * 256);
      }
    } else {
      constexpr int i = P - C::A_PT - C::B_PT - C::SA_PT;
      if constexpr (C::LIN_S) {
        constexpr uint32_t n0 = i * C::NW;
        dma_load4_at<(n0 / C::SB_I) * C::SUB + C::SB_OFF + (n0 % C::SB_I) * 256>(d.t.rsb, o.sb[i], d.ks_b, d.w4);
      } else {
        const uint32_t ins = (wave + i * C::NW) % C::SB_INST;
        dma_load4(d.t.rsb, o.sb[i], d.ks_b, d.lds + (ins / C::SB_I) * C::SUB + C::SB_OFF + (ins % C::SB_I) * 256);
      }
    }
  }

  // Program-order anchor for the accumulators: MFMAs count as side-effect-free,
  // so without this the compiler moves all of a k-step's MFMAs behind its LDS
  // reads and barrier.  An empty volatile asm that reads and rewrites every
  // accumulator (kept in AGPRs) and clobbers memory pins both in place.
  static __device__ __forceinline__ void anchor(Acc<C>& acc) {
#pragma unroll
    for (int i = 0; i < C::FM; ++i)
#pragma unroll
      for (int j = 0; j < C::FN; ++j) asm volatile("" : "+a"(acc.v[i][j])::"memory");
  }

  // Partial tiles and flags move between workgroups on different XCDs, whose
  // L2 caches are not coherent with each other.  Rather than agent-scope
  // fences (which write back or invalidate a whole L2, costly for every other
  // workgroup sharing it), only these accesses are made device-coherent: the
  // partials are stored and loaded with the device-scope cache policy (sc1),
  // and the flags are device-scope atomics.
  static constexpr int kDeviceScope = 16;   // buffer cache policy: sc1
  // s_waitcnt vmcnt(0) with the other counters left alone (expcnt 7, lgkmcnt 15)
  static constexpr int kWaitVmcnt0 = 0x0F70;

  // Publish this workgroup's partial: every wave waits until its own
  // device-scope stores of the partial have completed, then the barrier, then
  // one thread writes the flag.  The wait has to be explicit: the barrier's
  // workgroup-scope fence does not wait for global stores, so without it the
  // flag could become visible while some of the partial is still in flight.
  static __device__ __forceinline__ void publish(const KArgs& a, int w) {
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    if (a.delay_seed) {
      uint32_t h = a.delay_seed ^ (0x9e3779b9u * (uint32_t)(w + 1));
      h ^= h >> 15; h *= 0x2c1b3c6du; h ^= h >> 12;
      const int n = (int)(h % 48u);
      for (int i = 0; i < n; ++i) __builtin_amdgcn_s_sleep(127);
    }
    __syncthreads();
    if (threadIdx.x == 0 && w != a.drop_wg)
      __hip_atomic_store(a.locks + w, a.epoch, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }

  // Wait until workgroups first .. w-1 have all published; false if the spin
  // limit ran out.  Wave 0 polls up to 64 of the flags at once, one per lane,
  // so that the round trips of device-scope loads overlap instead of adding
  // up one contributor after another.
  static __device__ __forceinline__ bool wait_all(const KArgs& a, int first, int w, int* s_flag) {
    if (threadIdx.x < 64) {
      const int lane = threadIdx.x;
      const uint64_t t0 = __builtin_amdgcn_s_memrealtime();
      int ok = 1;
      for (int b = first; b < w && ok; b += 64) {
        const int v = b + lane;
        bool done = v >= w;
        for (;;) {
          if (!done) done = __hip_atomic_load(a.locks + v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) == a.epoch;
          if (__builtin_amdgcn_ballot_w64(!done) == 0) break;
          __builtin_amdgcn_s_sleep(2);
          if (__builtin_amdgcn_s_memrealtime() - t0 > a.spin_limit) {
            ok = 0;
            break;
          }
        }
      }
      if (lane == 0) {
        if (!ok) __hip_atomic_store(a.err, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        *s_flag = ok;
      }
    }
    __syncthreads();
    // The flag is the same for every lane; saying so keeps the work loop (and
    // every buffer descriptor derived from it) wave-uniform.
    // (the partials are then read with device-scope loads, issued after this)
    const int ok = __builtin_amdgcn_readfirstlane(*s_flag);
    __syncthreads();
    return ok != 0;
  }

  // Scratch slot of workgroup w in accumulator (register) order, so that each
  // store or load of a wave is one contiguous 1 KiB run:
  // [wave][block][accumulator quad][lane][4 floats].
  static __device__ __forceinline__ uint32_t slot_off(int w) {
    return (uint32_t)w * (uint32_t)(C::P_SLOT * 4) +
           (uint32_t)((wave_id() % C::OW) * C::P_WAVE + (threadIdx.x & 63) * 4) * 4u;
  }

  // Four accumulators (one run of four output columns) copied out of AGPRs.
  // The explicit reads keep the accumulators in AGPRs for their whole life;
  // left to itself the register allocator moves some of them to VGPRs for
  // the epilogue's arithmetic and then runs out of VGPRs in the main loop.
  template <class T>
  static __device__ __forceinline__ v4f read_run(const T& blk, int q) {
    v4f r;
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      float x;
      asm volatile("v_accvgpr_read_b32 %0, %1" : "=v"(x) : "a"(blk[4 * q + k]));
      r[k] = x;
    }
    return r;
  }

  // A VALU read of an MFMA result needs wait states after the MFMA (up to 18
  // for the 16-pass shapes) that the hardware does not enforce.  The compiler
  // inserts them for its own reads but not for the inline-asm reads above, so
  // every path that reads accumulators starts with this.
  static __device__ __forceinline__ void mfma_read_hazard() {
    asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7" ::: "memory");
  }

  static __device__ __forceinline__ uint32_t run_off(int i, int j, int q) {
    return (uint32_t)(((i * C::FN + j) * C::NQ + q) * 1024);
  }

  static __device__ __forceinline__ void store_partial(const KArgs& a, int w, const Acc<C>& acc) {
    const __amdgpu_buffer_rsrc_t rp = make_rsrc(a.P, 0x7fffffffu);
    const uint32_t base = slot_off(w);
    mfma_read_hazard();
#pragma unroll
    for (int i = 0; i < C::FM; ++i)
#pragma unroll
      for (int j = 0; j < C::FN; ++j)
#pragma unroll
        for (int q = 0; q < C::NQ; ++q) {
          const v4f v = read_run(acc.v[i][j], q);
          __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(v4u, v), rp, base + run_off(i, j, q), 0, kDeviceScope);
          __builtin_amdgcn_sched_barrier(0);
        }
  }

  // WK > 1, an item of a split tile: the waves of k-slices 1 .. WK-1 hand their
  // accumulators to the wave of slice 0 with the same output block (through
  // `red`, a free stage), which adds them to its own in slice order; only slice
  // 0's waves then hold the item's sums (to publish as a partial, or to finish
  // with the other workgroups' partials).  Every wave takes part (one barrier).
  static __device__ __forceinline__ void reduce_k(Acc<C>& acc, lds_u8* red) {
    const int lane = threadIdx.x & 63, wave = wave_id();
    const int ow = wave % C::OW, wk = wave / C::OW;
    typedef __attribute__((address_space(3))) v4f* PV;
    mfma_read_hazard();
    if (wk > 0) {
      lds_u8* const mine = red + ((wk - 1) * C::OW + ow) * (C::P_WAVE * 4) + lane * 16;
#pragma unroll
      for (int i = 0; i < C::FM; ++i)
#pragma unroll
        for (int j = 0; j < C::FN; ++j)
#pragma unroll
          for (int q = 0; q < C::NQ; ++q) *(PV)(mine + run_off(i, j, q)) = read_run(acc.v[i][j], q);
    }
    lds_barrier();
    if (wk == 0) {
#pragma unroll
      for (int i = 0; i < C::FM; ++i)
#pragma unroll
        for (int j = 0; j < C::FN; ++j)
#pragma unroll
          for (int q = 0; q < C::NQ; ++q) {
            v4f x = read_run(acc.v[i][j], q);
#pragma unroll
            for (int s = 1; s < C::WK; ++s)
              x += *(const PV)(red + ((s - 1) * C::OW + ow) * (C::P_WAVE * 4) + lane * 16 + run_off(i, j, q));
#pragma unroll
            for (int k = 0; k < 4; ++k) acc.v[i][j][4 * q + k] = x[k];
          }
    }
  }

  // Finishes one tile: C = round(sigma * (acc + P[w-1] + ... + P[first]) + bias),
  // the partials of the lower workgroups added in descending order (none when
  // first >= w).  Each lane holds, per block and run, four consecutive
  // columns of one row.  When N % 8 == 0 the wave rounds MF rows x SC columns
  // at a time into its part of the LDS stage `stg` (free while a tile is
  // finished) and writes them back as 16-byte pieces of whole rows, so each
  // store instruction fills entire 128-byte lines; otherwise (and for wave
  // tiles narrower than 32 columns) each lane stores its runs of four
  // columns, as one 8-byte piece when N % 4 == 0, else element by element.
  // The tile's bias was staged in LDS (as -0 when there is none).
  static __device__ __forceinline__ void epilogue(const KArgs& a, int tile, const Acc<C>& acc, const lds_u8* smem,
                                                  lds_u8* stg, int w, int first) {
    const int lane = threadIdx.x & 63, wave = wave_id() % C::OW;
    const int wm = wave / C::WN, wn = wave % C::WN;
    const int lr = lane % C::MF, g = lane / C::MF;
    const int tm = tile / a.tiles_n, tn = tile - tm * a.tiles_n;
    const int m0 = tm * C::BM, n0 = tn * C::BN;
    const int rows = min(C::BM, a.M - m0);
    const __amdgpu_buffer_rsrc_t rc = make_rsrc(a.C + (int64_t)m0 * a.N, (uint32_t)rows * (uint32_t)a.N * 2u);
    const __amdgpu_buffer_rsrc_t rp = make_rsrc(a.P, 0x7fffffffu);
    float sigma = 1.0f;
    if constexpr (C::DT == DT_FP8) {
      const float x = a.fsa ? *a.fsa : 1.0f;
      const float y = a.fsb ? *a.fsb : 1.0f;
      sigma = x * y;
    }
    const int N = a.N;
    const bool staged = C::STAGED && (N & 7) == 0;
    lds_u8* sw = stg + wave * C::STG_WAVE;
    // The bias of every column this lane touches (the same for all block
    // rows), read from LDS once: FN blocks x NQ runs of four bf16.
    v2u bias[C::FN][C::NQ];
#pragma unroll
    for (int j = 0; j < C::FN; ++j)
#pragma unroll
      for (int q = 0; q < C::NQ; ++q) {
        const int tcol = wn * C::WTN + j * C::MF + (C::MF == 32 ? 8 * q + 4 * g : 4 * g);
        bias[j][q] = *(const __attribute__((address_space(3))) v2u*)(smem + C::BIAS_OFF + tcol * 2);
      }
    // Byte offset in C of this lane's first staged chunk (row wm*WTM + lane/SCH
    // of the tile, column n0 + wn*WTN + 8*(lane%SCH)); each store adds a uniform
    // offset.  Its column, to test against N.
    const int lcol = n0 + wn * C::WTN + (lane % C::SCH) * 8;
    const uint32_t lane_c = ((uint32_t)(wm * C::WTM + lane / C::SCH) * (uint32_t)N + (uint32_t)lcol) * 2u;
    mfma_read_hazard();

    // the rounded run (block i, j; run q) of this lane, partials included
    auto run_bits = [&](int j, int q, const v4f& xq) -> v2u {
      const v2u bb = bias[j][q];
      const float b4[4] = {__uint_as_float(bb[0] << 16), __uint_as_float(bb[0] & 0xffff0000u),
                           __uint_as_float(bb[1] << 16), __uint_as_float(bb[1] & 0xffff0000u)};
      float t[4];
#pragma unroll
      for (int k = 0; k < 4; ++k) t[k] = C::DT == DT_FP8 ? xq[k] * sigma : xq[k];
      return round_run(t, b4);
    };
    // The block's partial sums: own accumulators, then the partials of
    // workgroups w-1, w-2, ..., first in that order.  The loads of CHK
    // contributors are issued together (partials come from memory at device
    // scope, so one at a time would pay a round trip each); the adds keep
    // the fixed order.
    // (8 runs in flight, 4 for eight-wave tiles, whose register file is half)
    constexpr int CHK_RUNS = C::NW >= 8 ? 4 : 8;
    constexpr int CHK = CHK_RUNS / C::NQ > 0 ? CHK_RUNS / C::NQ : 1;
    // Wave tiles of at most 4 runs: the partials of the first PRE contributors
    // (w-1 .. w-PRE), every run of every block, are loaded up front in one
    // batch (at most 16 runs in flight), so the blocks do not each wait a round
    // trip; the rest, if any, follow in chunks as above.
    constexpr int RUNS = C::FM * C::FN * C::NQ;
    constexpr int PRE = RUNS <= 4 ? 16 / RUNS : 0;
    v4u pre[PRE > 0 ? PRE : 1][PRE > 0 ? RUNS : 1];
    if constexpr (PRE > 0) {
#pragma unroll
      for (int c = 0; c < PRE; ++c)
        if (w - 1 - c >= first) {
          const uint32_t base = slot_off(w - 1 - c);
#pragma unroll
          for (int i = 0; i < C::FM; ++i)
#pragma unroll
            for (int j = 0; j < C::FN; ++j)
#pragma unroll
              for (int q = 0; q < C::NQ; ++q)
                pre[c][(i * C::FN + j) * C::NQ + q] =
                    __builtin_amdgcn_raw_buffer_load_b128(rp, base + run_off(i, j, q), 0, kDeviceScope);
        }
    }
    auto block_sums = [&](const typename Acc<C>::T& blk, int i, int j, v4f x[C::NQ]) {
#pragma unroll
      for (int q = 0; q < C::NQ; ++q) x[q] = read_run(blk, q);
      if constexpr (PRE > 0) {
#pragma unroll
        for (int c = 0; c < PRE; ++c)
          if (w - 1 - c >= first) {
#pragma unroll
            for (int q = 0; q < C::NQ; ++q) x[q] += __builtin_bit_cast(v4f, pre[c][(i * C::FN + j) * C::NQ + q]);
          }
      }
      for (int v0 = w - 1 - PRE; v0 >= first; v0 -= CHK) {
        v4u p[CHK][C::NQ];
#pragma unroll
        for (int c = 0; c < CHK; ++c)
          if (v0 - c >= first) {
            const uint32_t base = slot_off(v0 - c);
#pragma unroll
            for (int q = 0; q < C::NQ; ++q)
              p[c][q] = __builtin_amdgcn_raw_buffer_load_b128(rp, base + run_off(i, j, q), 0, kDeviceScope);
          }
#pragma unroll
        for (int c = 0; c < CHK; ++c)
          if (v0 - c >= first) {
#pragma unroll
            for (int q = 0; q < C::NQ; ++q) x[q] += __builtin_bit_cast(v4f, p[c][q]);
          }
      }
    };

    // compile-time block indices throughout: accumulators are only ever
    // indexed by constants (a dynamic index would move them to scratch)
    static_for<C::FM>([&](auto ic_) {
      constexpr int i = decltype(ic_)::value;
      const uint32_t row0 = (uint32_t)(wm * C::WTM + i * C::MF);     // first row of the block row, in the tile
      if (staged) {
        if constexpr (C::STAGED) static_for<C::WTN / C::SC>([&](auto cwc) {
          constexpr int cw = decltype(cwc)::value;
          static_for<C::SC / C::MF>([&](auto jjc) {
            constexpr int jj = decltype(jjc)::value;
            constexpr int j = cw * (C::SC / C::MF) + jj;
            v4f x[C::NQ];
            block_sums(acc.v[i][j], i, j, x);
#pragma unroll
            for (int q = 0; q < C::NQ; ++q) {
              const v2u h = run_bits(j, q, x[q]);
              const int c = jj * C::MF + (C::MF == 32 ? 8 * q + 4 * g : 4 * g);   // column in the window
              const int off = lr * (C::SC * 2) + (((c >> 3) ^ (lr % C::SCH)) << 4) + (((c >> 2) & 1) << 3);
              *(__attribute__((address_space(3))) v2u*)(sw + off) = h;
            }
            __builtin_amdgcn_sched_barrier(0);
          });
          // every lane's writes land before any lane's reads (one wave's LDS
          // operations execute in order; this keeps the compiler from moving
          // them across each other)
          asm volatile("" ::: "memory");
          constexpr int PS = C::MF / C::SRP;
          v4u d[PS];
#pragma unroll
          for (int ps = 0; ps < PS; ++ps) {
            const int r = ps * C::SRP + lane / C::SCH, ch = lane % C::SCH;
            d[ps] = *(const __attribute__((address_space(3))) v4u*)(sw + r * (C::SC * 2) + ((ch ^ (r % C::SCH)) << 4));
          }
          const bool col_ok = lcol + cw * C::SC < N;
#pragma unroll
          for (int ps = 0; ps < PS; ++ps) {
            const uint32_t up = ((uint32_t)(i * C::MF + ps * C::SRP) * (uint32_t)N + (uint32_t)(cw * C::SC)) * 2u;
            __builtin_amdgcn_raw_buffer_store_b128(d[ps], rc, col_ok ? lane_c + up : kOob, 0, 0);
          }
          asm volatile("" ::: "memory");
        });
      } else {
        static_for<C::FN>([&](auto jc) {
          constexpr int j = decltype(jc)::value;
          v4f x[C::NQ];
          block_sums(acc.v[i][j], i, j, x);
#pragma unroll
          for (int q = 0; q < C::NQ; ++q) {
            const v2u h = run_bits(j, q, x[q]);
            const int col = n0 + wn * C::WTN + j * C::MF + (C::MF == 32 ? 8 * q + 4 * g : 4 * g);
            const uint32_t coff = ((row0 + lr) * (uint32_t)N + (uint32_t)col) * 2u;
            if ((N & 3) == 0) {
              // the run's four columns are all inside N or all past it
              __builtin_amdgcn_raw_buffer_store_b64(h, rc, col < N ? coff : kOob, 0, 0);
            } else {
              const uint32_t hv[4] = {h[0] & 0xffffu, h[0] >> 16, h[1] & 0xffffu, h[1] >> 16};
#pragma unroll
              for (int k = 0; k < 4; ++k)
                __builtin_amdgcn_raw_buffer_store_b16((uint16_t)hv[k], rc, col + k < N ? coff + 2u * k : kOob, 0, 0);
            }
          }
          __builtin_amdgcn_sched_barrier(0);
        });
      }
    });
    // The partials are loaded and added under the same conditions, which the
    // compiler does not pair up: it takes a load that was issued and never
    // used as possibly still in flight, and then waits for every outstanding
    // load (the next item's operand stages included) before the first
    // register write of each later k-step.  A wait it can see, once per tile,
    // tells it they have all landed.  (A second copy of the epilogue without
    // partials, for the tiles finished alone, would need no wait, but the
    // pair raises the register pressure around it: more spills in the
    // 8-wave kernels.  The k-split kernels finish such tiles in
    // finish_split.)
    __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);
  }

  // WK > 1, a tile the workgroup finishes alone (no partials): every wave
  // writes its accumulators to `red` (a free stage), and after one barrier
  // each wave takes an equal share of the tile's 4-column runs, adds the WK
  // k-slices' sums of each in slice order (the order reduce_k uses), rounds
  // them with the bias (staged in LDS before the barrier) and stores them:
  // the work after the k-steps is spread over all the waves instead of
  // waiting on slice 0's.  Each lane of a share stores its run as one
  // 8-byte piece when N % 4 == 0, else element by element.
  static __device__ __forceinline__ void finish_split(const KArgs& a, int tile, const Acc<C>& acc, lds_u8* red,
                                                      const lds_u8* smem) {
    typedef __attribute__((address_space(3))) v4f* PV;
    const int lane = threadIdx.x & 63, wave = wave_id();
    constexpr int RUNS = C::FM * C::FN * C::NQ;           // runs of one output wave, 64 lanes each
    constexpr int TOTAL = C::OW * RUNS * 64;              // lane-runs of the tile
    static_assert(TOTAL % C::NW == 0, "equal shares");
    constexpr int SHARE = TOTAL / C::NW;
    mfma_read_hazard();
    lds_u8* const mine = red + wave * (C::P_WAVE * 4) + lane * 16;
#pragma unroll
    for (int i = 0; i < C::FM; ++i)
#pragma unroll
      for (int j = 0; j < C::FN; ++j)
#pragma unroll
        for (int q = 0; q < C::NQ; ++q) *(PV)(mine + run_off(i, j, q)) = read_run(acc.v[i][j], q);
    lds_barrier();
    const int tm = tile / a.tiles_n, tn = tile - tm * a.tiles_n;
    const int m0 = tm * C::BM, n0 = tn * C::BN;
    const int rows = min(C::BM, a.M - m0);
    const int N = a.N;
    const __amdgpu_buffer_rsrc_t rc = make_rsrc(a.C + (int64_t)m0 * N, (uint32_t)rows * (uint32_t)N * 2u);
#pragma unroll
    for (int x0 = 0; x0 < SHARE; x0 += 64) {
      const int x = wave * SHARE + x0 + lane;              // lane-run of the tile
      if (x0 + 64 > SHARE && x0 + lane >= SHARE) break;
      const int ow = x / (RUNS * 64), run = (x / 64) % RUNS, l = x % 64;
      v4f v = *(const PV)(red + ow * (C::P_WAVE * 4) + run * 1024 + l * 16);
#pragma unroll
      for (int k = 1; k < C::WK; ++k) v += *(const PV)(red + (k * C::OW + ow) * (C::P_WAVE * 4) + run * 1024 + l * 16);
      // the run's place: block (i, j), accumulator quad q of output wave ow, lane l
      const int q = run % C::NQ, ij = run / C::NQ, j = ij % C::FN, i = ij / C::FN;
      const int wm = ow / C::WN, wn = ow % C::WN;
      const int row = wm * C::WTM + i * C::MF + l % C::MF;
      const int tcol = wn * C::WTN + j * C::MF + (C::MF == 32 ? 8 * q + 4 * (l / C::MF) : 4 * (l / C::MF));
      const v2u bb = *(const __attribute__((address_space(3))) v2u*)(smem + C::BIAS_OFF + tcol * 2);
      const float b4[4] = {__uint_as_float(bb[0] << 16), __uint_as_float(bb[0] & 0xffff0000u),
                           __uint_as_float(bb[1] << 16), __uint_as_float(bb[1] & 0xffff0000u)};
      const float t[4] = {v[0], v[1], v[2], v[3]};
      const v2u h = round_run(t, b4);
      const int col = n0 + tcol;
      const uint32_t coff = ((uint32_t)row * (uint32_t)N + (uint32_t)col) * 2u;
      if ((N & 3) == 0) {
        __builtin_amdgcn_raw_buffer_store_b64(h, rc, col < N ? coff : kOob, 0, 0);
      } else {
        const uint32_t hv[4] = {h[0] & 0xffffu, h[0] >> 16, h[1] & 0xffffu, h[1] >> 16};
#pragma unroll
        for (int k = 0; k < 4; ++k)
          __builtin_amdgcn_raw_buffer_store_b16((uint16_t)hv[k], rc, col + k < N ? coff + 2u * k : kOob, 0, 0);
      }
    }
  }

  // Position in a workgroup's work list: the WorkIter fields that change as
  // it is walked.  The rest is recomputed from the launch arguments at each
  // step, which keeps two cursors down to six scalar registers.
  struct Cursor {
    int32_t phase, whole, dp;
  };

  static __device__ __forceinline__ Cursor cursor_begin(int w) {
    const KArgs& a = kargs();
    const WorkIter it(w, a.sk_tiles, a.tiles, a.iters, a.q, a.r, a.G);
    return Cursor{it.phase, it.whole, it.dp};
  }

  // Next work item of workgroup w; the item is the same for every lane, and
  // saying so keeps everything derived from it (tile origins, buffer
  // descriptors) in scalar registers.
  static __device__ __forceinline__ bool advance(int w, Cursor& c, WorkItem& x) {
    const KArgs& a = kargs();
    WorkIter it(w, a.sk_tiles, a.tiles, a.iters, a.q, a.r, a.G);
    it.phase = c.phase;
    it.whole = c.whole;
    it.dp = c.dp;
    const bool more = it.next(x);
    c.phase = __builtin_amdgcn_readfirstlane(it.phase);
    c.whole = __builtin_amdgcn_readfirstlane(it.whole);
    c.dp = __builtin_amdgcn_readfirstlane(it.dp);
    x.tile = __builtin_amdgcn_readfirstlane(x.tile);
    x.k0 = __builtin_amdgcn_readfirstlane(x.k0);
    x.k1 = __builtin_amdgcn_readfirstlane(x.k1);
    x.mode = __builtin_amdgcn_readfirstlane(x.mode);
    x.first = __builtin_amdgcn_readfirstlane(x.first);
    return more;
  }

  // Runs the workgroup's whole work list as one stream of k-steps through a
  // ring of STAGES LDS buffers: k-step c (counted over the whole list) lives
  // in stage c % STAGES and its loads are issued STAGES-1 k-steps ahead, also
  // across item boundaries, so the next tile's operands are on their way while
  // a tile is being finished.
  static __device__ __forceinline__ void run_list(lds_u8* smem, int* s_flag) {
    constexpr int S = C::STAGES;
    constexpr int PER_STAGE = C::LOADS_PER_STAGE_S;
    const int w = blockIdx.x;
    const int tid = threadIdx.x;
    // Phase trace (only when the caller passed a buffer): wave 0 of each
    // workgroup stores s_memrealtime stamps at the phase boundaries, at most
    // kTraceItems work items, and nothing else changes.
    uint64_t* const tr = kargs().trace;
    const bool rec = tr != nullptr && tid == 0;
    int item = 0;
    if (rec) tr[w * kTraceWords] = __builtin_amdgcn_s_memrealtime();
    auto stamp = [&](int slot) {
      if (rec && item < kTraceItems) tr[w * kTraceWords + 1 + 4 * item + slot] = __builtin_amdgcn_s_memrealtime();
    };
    const LoadOffs lo = load_offsets(kargs());
    const LdsPtrs lp = lds_ptrs(smem);
    if (rec) tr[w * kTraceWords + 29] = __builtin_amdgcn_s_memrealtime();
    const uint32_t sa_kstride = kargs().sa_kstride, sb_kstride = kargs().sb_kstride;

    // Two cursors over the same work list: one issues loads, one computes.
    Cursor ci = cursor_begin(w);
    Cursor cc = ci;
    WorkItem ii, ic;
    bool have_i = advance(w, ci, ii);
    if (!have_i) return;
    advance(w, cc, ic);
    int ki = ii.k0, ki_end = ii.k1;
    TileCtx ti = tile_ctx(kargs(), ii.tile);
    int issued = 0;   // k-steps issued so far
    int done = 0;     // k-steps computed so far

    // this tile's bias element (one per thread), staged in LDS before the epilogue
    auto load_bias = [&](int tile) -> uint32_t {
      const KArgs& a = kargs();
      const int tn = tile % a.tiles_n;
      const int col = tn * C::BN + tid;
      if (a.bias == nullptr) return 0x8000u;   // -0: adding it changes nothing, not even a zero's sign
      const bool ok = tid < C::BN && col < a.N;
      return __builtin_amdgcn_raw_buffer_load_b16(make_rsrc(a.bias, (uint32_t)(a.N * 2)), ok ? (uint32_t)col * 2 : kOob,
                                                 0, 0);
    };

    // ---- the direct path: one fixed, interleaved schedule per k-step.
    // k-step d reads stage d % S and issues the loads of k-step d + S - 1 (past
    // the end of the list, the last k-step's again) into stage (d + S - 1) % S,
    // which the barrier of k-step d - 1 freed.  Because every k-step issues
    // PER_STAGE loads, the loads of stage d + 1 have landed once at most
    // (S - 2) * PER_STAGE loads are outstanding (loads complete in issue
    // order; other outstanding operations are younger and only lengthen the
    // wait).  Slot b of a sub-step is its b-th MFMA; the k-step's loads go
    // after the slots before the barrier, the next sub-step's operand reads
    // after the first slots of each sub-step, and the barrier that publishes
    // stage d + 1 sits half-way through the last sub-step, after which that
    // stage's scales and first operands are read (inside an item) between the
    // remaining MFMAs.  sched_barrier(0) between slots keeps this order.
    const uint32_t wv = (uint32_t)wave_id();
    auto dma_ctx = [&]() -> DmaCtx {
      DmaCtx d;
      d.t = ti;
      d.kbyte_a = (uint32_t)ki * C::KSA;
      d.kbyte_b = (uint32_t)ki * C::KSB;
      d.ks_a = (uint32_t)ki * sa_kstride;
      d.ks_b = (uint32_t)ki * sb_kstride;
      d.lds = (uint32_t)(uintptr_t)stage_ptr(smem, (int)((uint32_t)issued % S));
      d.w16 = d.lds + wv * 1024u;
      d.w4 = d.lds + wv * 256u;
      d.wave = wv;
      return d;
    };
    // (past the end of the list ki stays on the last k-step, whose loads are
    // then issued again)
    auto advance_issue = [&]() {
      ++issued;
      if (have_i && ++ki == ki_end) {
        WorkItem x;
        have_i = advance(w, ci, x);
        if (have_i) {
          ki = x.k0;
          ki_end = x.k1;
          ti = tile_ctx(kargs(), x.tile);
        } else {
          ki = ki_end - 1;
        }
      }
    };
    constexpr int NB = C::FM * C::FN;                     // MFMA slots per sub-step
    constexpr int HB = NB / 2;                            // slots of the last sub-step before the barrier
    constexpr int PRE = (C::NU - 1) * NB + HB;            // slots before the barrier
    constexpr int POST = NB - HB;
    // The k-step's loads are spread over the slots before the barrier.  With
    // two stages the loads issued in a k-step are waited for at its own
    // barrier, so they all go out in the first slots instead.
    constexpr int DMA_SPAN = S == 2 ? (PRE < PER_STAGE ? PRE : PER_STAGE) : PRE;
    auto kstep_interleaved = [&](int d, Ops& o0, Ops& o1, Scales& sc0, Scales& sc1, Acc<C>& acc) {
      const int cur = (int)((uint32_t)d % S), nxt = (int)((uint32_t)(d + 1) % S);
      const DmaCtx dc = dma_ctx();
      if constexpr (PRE == 0) {
        static_for<PER_STAGE>([&](auto pc) { dma_piece<decltype(pc)::value>(dc, lo); });
      }
      static_for<C::NU>([&](auto uc) {
        constexpr int u = decltype(uc)::value;
        Ops& now = (u & 1) ? o1 : o0;
        Ops& nxo = (u & 1) ? o0 : o1;
        constexpr bool last = u + 1 == C::NU;
        static_for<(last ? HB : NB)>([&](auto bc) {
          constexpr int b = decltype(bc)::value;
          constexpr int slot = u * NB + b;                // among the PRE slots
          mfma_one<u, b>(now, sc0, acc);
          if constexpr (!last) {
            static_for<NRD>([&](auto rc) {
              constexpr int r = decltype(rc)::value;
              // early in the sub-step (front-loaded), so they land well before use
              if constexpr ((NRD <= NB ? r : r * NB / NRD) == b) read_op<u + 1, r>(cur * C::STAGE, lp, nxo);
            });
          }
          static_for<PER_STAGE>([&](auto pc) {
            constexpr int pp = decltype(pc)::value;
            if constexpr (pp * DMA_SPAN / PER_STAGE == slot) dma_piece<pp>(dc, lo);
          });
          __builtin_amdgcn_sched_barrier(0);
        });
        if constexpr (last) {
          wait_vmcnt_n<(S - 2) * PER_STAGE>();
          lds_barrier();
          // The next k-step's scales and first operands, also when it belongs
          // to the next item (the stage is the same either way).
          static_for<POST>([&](auto bc) {
            constexpr int b = decltype(bc)::value;
            mfma_one<u, HB + b>(now, sc0, acc);
            static_for<NSR + NRD>([&](auto rc) {
              constexpr int r = decltype(rc)::value;
              if constexpr (r * POST / (NSR + NRD) == b)
                post_read_one<r>(stage_ptr(smem, nxt), nxt * C::STAGE, lp, sc1, nxo);
            });
            __builtin_amdgcn_sched_barrier(0);
          });
          sc0 = sc1;
          if constexpr ((C::NU & 1) == 1) o0 = o1;   // sub-step 0 always starts in o0
        }
        anchor(acc);
      });
      advance_issue();
    };

    // INPLACE kernels: A's fragments live in o0.a and are refilled one by one
    // right after the MFMA that uses each for the last time in a sub-step; B's
    // alternate between o0.b (even sub-steps) and o1.b (odd), read early in
    // the sub-step before.  In the last sub-step the refills come from the
    // next stage, so those whose slot falls before the barrier wait for it,
    // as do B's fragments and the scales of the next k-step.
    auto kstep_inplace = [&](int d, auto& o0, auto& o1, Scales& sc0, Scales& sc1, Acc<C>& acc) {
      static_assert(!C::INPLACE || PRE > 0, "the in-place schedule issues its loads before the barrier");
      const int cur = (int)((uint32_t)d % S), nxt = (int)((uint32_t)(d + 1) % S);
      const DmaCtx dc = dma_ctx();
      constexpr int NBR = C::FN * C::NCH;   // B reads per sub-step
      static_for<C::NU>([&](auto uc) {
        constexpr int u = decltype(uc)::value;
        constexpr bool last = u + 1 == C::NU;
        auto& bnow = (u & 1) ? o1 : o0;
        auto& bnxt = (u & 1) ? o0 : o1;
        static_for<NB>([&](auto bc) {
          constexpr int b = decltype(bc)::value;
          constexpr int slot = u * NB + b;
          if constexpr (last && b == HB) {
            wait_vmcnt_n<(S - 2) * PER_STAGE>();
            lds_barrier();
            const lds_u8* st = stage_ptr(smem, nxt);
            if constexpr (C::MX) read_scale_a(st, lp, sc1);
            static_for<C::FM>([&](auto ic) {
              constexpr int i = decltype(ic)::value;
              if constexpr (last_use_a(i) < HB) read_a<0, i>(nxt * C::STAGE, lp, o0);
            });
            if constexpr (C::MX) read_scale_b(st, lp, sc1);
            static_for<NBR>([&](auto rc) {
              constexpr int r = decltype(rc)::value;
              read_b<0, r / C::NCH, r % C::NCH>(nxt * C::STAGE, lp, bnxt);
            });
          }
          mfma_ab<u, b>(o0, bnow, sc0, acc);
          static_for<C::FM>([&](auto ic) {
            constexpr int i = decltype(ic)::value;
            if constexpr (last_use_a(i) == b) {
              if constexpr (!last) read_a<u + 1, i>(cur * C::STAGE, lp, o0);
              else if constexpr (b >= HB) read_a<0, i>(nxt * C::STAGE, lp, o0);
            }
          });
          if constexpr (!last) {
            static_for<NBR>([&](auto rc) {
              constexpr int r = decltype(rc)::value;
              if constexpr ((NBR <= NB ? r : r * NB / NBR) == b) read_b<u + 1, r / C::NCH, r % C::NCH>(cur * C::STAGE, lp, bnxt);
            });
          }
          if constexpr (slot < PRE) {
            static_for<PER_STAGE>([&](auto pc) {
              constexpr int pp = decltype(pc)::value;
              if constexpr (pp * DMA_SPAN / PER_STAGE == slot) dma_piece<pp>(dc, lo);
            });
          }
          __builtin_amdgcn_sched_barrier(0);
        });
        anchor(acc);
      });
      sc0 = sc1;
      if constexpr ((C::NU & 1) == 1) {
        // the next k-step's B went to o1 (its sub-step 0 reads o0)
#pragma unroll
        for (int j = 0; j < C::FN; ++j)
#pragma unroll
          for (int h = 0; h < C::NCH; ++h) o0.b[j][h] = o1.b[j][h];
      }
      advance_issue();
    };

    static_for<S - 1>([&](auto) {
      const DmaCtx dc = dma_ctx();
      static_for<PER_STAGE>([&](auto pc) { dma_piece<decltype(pc)::value>(dc, lo); });
      advance_issue();
    });
    uint32_t bias_h = load_bias(ic.tile);
    if (rec) tr[w * kTraceWords + 28] = __builtin_amdgcn_s_memrealtime();
    // stage 0 landed: everything but the loads of the stages after it (and the bias load)
    wait_vmcnt_n<(S - 2) * PER_STAGE>();
    lds_barrier();
    if (rec) tr[w * kTraceWords + 27] = __builtin_amdgcn_s_memrealtime();
    // Operands of the next k-step: each k-step reads the next one's scales
    // and first operands (also across items), so they are read here once.
    Ops o0, o1;
    Scales sc0, sc1;
    read_scales(stage_ptr(smem, 0), lp, sc0);
    sc1 = sc0;   // (the unscaled types never read scales again)
    read_ops<0>(0, lp, o0);
    for (;;) {
      Acc<C> acc;
      acc.zero();
      int n = ic.k1 - ic.k0;   // at least one k-step per item
      stamp(0);
      do {
        if constexpr (C::INPLACE) kstep_inplace(done, o0, o1, sc0, sc1, acc);
        else kstep_interleaved(done, o0, o1, sc0, sc1, acc);
        ++done;
      } while (--n > 0);

      // ---- the item is complete
      stamp(1);
      // the stage of the item's last k-step is free until the next k-step issues into it
      // (k-split kernels: a whole tile goes to finish_split, others add their slices here)
      if constexpr (C::WK > 1) {
        if (ic.mode != WORK_WHOLE) reduce_k(acc, stage_ptr(smem, (int)((uint32_t)(done + S - 1) % S)) + C::RED_OFF);
      }
      const bool holds = C::WK == 1 || wave_id() < C::OW;   // a wave with the item's sums
      if (ic.mode == WORK_CONTRIB) {
        if (holds) store_partial(kargs(), w, acc);
        publish(kargs(), w);
        stamp(2);
      } else {
        bool ok = true;
        int first = w;   // lowest contributing workgroup (w: none)
        if (ic.mode == WORK_OWNER) {
          // every contributor has published before any partial is read
          first = ic.first;
          ok = wait_all(kargs(), first, w, s_flag);
        }
        stamp(2);
        if (ok) {
          lds_barrier();   // every wave is done with the previous tile's bias
          if (tid < C::BN) *(__attribute__((address_space(3))) uint16_t*)(smem + C::BIAS_OFF + tid * 2) = (uint16_t)bias_h;
          lds_u8* const stg = stage_ptr(smem, (int)((uint32_t)(done + S - 1) % S));
          if (C::WK > 1 && ic.mode == WORK_WHOLE) {
            finish_split(kargs(), ic.tile, acc, stg + C::RED_OFF, smem);   // (its barrier also publishes the bias)
          } else {
            lds_barrier();
            if (holds) epilogue(kargs(), ic.tile, acc, smem, stg, w, first);
          }
          lds_barrier();   // the next k-step's loads into the freed stage wait until every wave is done with it
        }
      }
      stamp(3);
      ++item;
      if (!advance(w, cc, ic)) break;
      bias_h = load_bias(ic.tile);
    }
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    if (rec) {
      tr[w * kTraceWords + 30] = (uint64_t)item;
      tr[w * kTraceWords + 31] = __builtin_amdgcn_s_memrealtime();
    }
  }

  static __device__ __forceinline__ void run() {
    __shared__ __attribute__((aligned(16))) uint8_t smem_raw[C::LDS_TOTAL];
    __shared__ int s_flag;
    lds_u8* smem = (lds_u8*)smem_raw;
    run_list(smem, &s_flag);
  }
};

template <class C, int OCC, bool DIRECT>
__global__ __launch_bounds__(C::NT) __attribute__((amdgpu_waves_per_eu(OCC, OCC)))
void sk_gemm_kernel(KArgs a) {
  (void)a;   // read through kargs()
  Kernel<C, DIRECT>::run();
}

template <class C, int OCC, bool DIRECT>
hipError_t launch_variant(int grid, const KArgs& a, hipStream_t s) {
  hipLaunchKernelGGL((sk_gemm_kernel<C, OCC, DIRECT>), dim3(grid), dim3(C::NT), 0, s, a);
  return hipGetLastError();
}

typedef hipError_t (*Launcher)(int, const KArgs&, hipStream_t);

// The direct-scale twin is compiled for the MX kernels with at most 128 rows
// per tile, which serve the small and skinny problems: there the separate
// re-layout launch is a large part of a call (16x8192x8192 MXFP4: 19.1 ->
// 15.3 us; 128x8192x8192: 27.8 -> 24.1 us).  The 256x256 kernels keep the
// re-laid copy: gathering 256 rows' scale bytes per k-step costs them more
// than the pass (8192^3: 258 -> 284 us).
template <class C, int OCC>
constexpr Launcher direct_launcher() {
  if constexpr (C::MX && C::SPR >= 4 && C::BM <= 128) return &launch_variant<C, OCC, true>;
  else return nullptr;
}

#define SK_CFG(DT, BM, BN, KB, MF, WM, WN, ST) Cfg<DT, BM, BN, KB, MF, WM, WN, ST>
#define SK_VARIANT(DT, BM, BN, KB, MF, WM, WN, ST, OCC)                                                   \
  Variant {                                                                                              \
    DT, BM, BN, KB, SK_CFG(DT, BM, BN, KB, MF, WM, WN, ST)::BK, MF, SK_CFG(DT, BM, BN, KB, MF, WM, WN, ST)::NT, \
        SK_CFG(DT, BM, BN, KB, MF, WM, WN, ST)::LDS_TOTAL, WM, WN,                                       \
        SK_CFG(DT, BM, BN, KB, MF, WM, WN, ST)::NG, SK_CFG(DT, BM, BN, KB, MF, WM, WN, ST)::NU, 1,       \
        &launch_variant<SK_CFG(DT, BM, BN, KB, MF, WM, WN, ST), OCC, false>,                             \
        direct_launcher<SK_CFG(DT, BM, BN, KB, MF, WM, WN, ST), OCC>()                                   \
  }

// A k-split kernel (WK groups of waves): direct scale reads only, so no
// re-layout launcher.  Its k-step is WK k-slices of KB bytes per row.
#define SK_CFG_WK(DT, BM, BN, KB, MF, WM, WN, ST, WK) Cfg<DT, BM, BN, KB, MF, WM, WN, ST, WK>
#define SK_VARIANT_WK(DT, BM, BN, KB, MF, WM, WN, ST, WK, OCC)                                               \
  Variant {                                                                                                  \
    DT, BM, BN, (WK) * (KB), SK_CFG_WK(DT, BM, BN, KB, MF, WM, WN, ST, WK)::BK, MF,                           \
        SK_CFG_WK(DT, BM, BN, KB, MF, WM, WN, ST, WK)::NT, SK_CFG_WK(DT, BM, BN, KB, MF, WM, WN, ST, WK)::LDS_TOTAL, \
        WM, WN, SK_CFG_WK(DT, BM, BN, KB, MF, WM, WN, ST, WK)::NG, SK_CFG_WK(DT, BM, BN, KB, MF, WM, WN, ST, WK)::NU, \
        WK, nullptr, &launch_variant<SK_CFG_WK(DT, BM, BN, KB, MF, WM, WN, ST, WK), OCC, true>                 \
  }

}  // namespace sk
