// Stream-K GEMM kernels for gfx950 (MI355X).
//
// One persistent kernel template serves MXFP4, bf16 and fp8.  Each of the G
// workgroups (256 threads = 4 wave64) runs, in order:
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
// Per MAC iteration (k-step) each operand row contributes KB bytes (128 for the
// big tiles: 256 FP4, 128 fp8 or 64 bf16 values).  A and B k-slices are loaded
// with 16-byte buffer loads (out-of-range chunks read as zero), staged through
// registers into a double-buffered LDS tile (16-byte chunks XOR-swizzled by row
// to spread LDS banks), and consumed by MFMA:
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
// is unchanged) and each lane's scale bytes are contiguous in memory.

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

// Buffer resource word 3 for gfx9-family raw (untyped) buffers.
constexpr int kRsrcWord3 = 0x00020000;
// Any offset at or past 2^31 lies beyond every resource built here: reads 0.
constexpr uint32_t kOob = 0x80000000u;

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, kRsrcWord3);
}

template <int N, class F>
__device__ __forceinline__ void static_for(F&& f) {
  if constexpr (N > 0) {
    static_for<N - 1>(f);
    f(std::integral_constant<int, N - 1>{});
  }
}

template <int DT_, int BM_, int BN_, int KB_, int MF_, int WM_, int WN_>
struct Cfg {
  static constexpr int DT = DT_, BM = BM_, BN = BN_, KB = KB_, MF = MF_, WM = WM_, WN = WN_;
  static constexpr int NW = WM * WN;
  static constexpr int NT = 64 * NW;
  static constexpr int WTM = BM / WM, WTN = BN / WN;   // per-wave tile
  static constexpr int FM = WTM / MF, FN = WTN / MF;   // MFMA blocks per wave
  static constexpr int NG = 64 / MF;                   // K groups across the lanes
  static constexpr int LB = KB / NG;                   // bytes per lane per row per k-step
  static constexpr int U = DT == DT_FP8 ? 32 : 16;     // bytes per lane per MFMA
  static constexpr int NU = LB / U;                    // MFMAs per block per k-step
  static constexpr int CPR = KB / 16;                  // 16-byte chunks per row per k-step
  static constexpr int SPR = DT == DT_MXFP4 ? KB / 16 : 0;  // scale bytes per row per k-step
  static constexpr int BK = DT == DT_MXFP4 ? 2 * KB : (DT == DT_BF16 ? KB / 2 : KB);
  static constexpr int ACC = MF == 32 ? 16 : 4;        // fp32 accumulators per block per lane
  static constexpr int A_OFF = 0;
  static constexpr int B_OFF = BM * KB;
  static constexpr int SA_OFF = (BM + BN) * KB;
  static constexpr int SB_OFF = SA_OFF + BM * SPR;
  static constexpr int STAGE = ((BM + BN) * (KB + SPR) + 15) / 16 * 16;
  static constexpr int LDS = 2 * STAGE;
  static constexpr int A_CH = BM * CPR, B_CH = BN * CPR;
  static constexpr int A_PT = (A_CH + NT - 1) / NT, B_PT = (B_CH + NT - 1) / NT;
  static constexpr int SA_PT = DT == DT_MXFP4 ? (BM + NT - 1) / NT : 0;
  static constexpr int SB_PT = DT == DT_MXFP4 ? (BN + NT - 1) / NT : 0;
  static constexpr int P_SLOT = BM * BN;                // floats per scratch slot
  static constexpr int P_WAVE = FM * FN * ACC * 64;     // floats per wave in a slot

  static_assert(MF == 32 || MF == 16, "MFMA shape");
  static_assert(WTM % MF == 0 && WTN % MF == 0, "wave tile must be whole MFMA blocks");
  static_assert(LB % U == 0 && NU >= 1, "k-step must give each lane whole MFMA operands");
  static_assert(KB % 16 == 0 && (CPR & (CPR - 1)) == 0, "k-step is a power-of-two number of chunks");
  static_assert(DT != DT_MXFP4 || SPR == 4 || SPR == 8, "scale bytes per row per k-step");
  static_assert(LDS <= 160 * 1024, "LDS");
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

template <class C, int OP>
__device__ __forceinline__ void mfma(typename Acc<C>::T& acc, const v4u* a, const v4u* b, int sa, int sb) {
  if constexpr (C::DT == DT_BF16) {
    v8bf va = __builtin_bit_cast(v8bf, a[0]);
    v8bf vb = __builtin_bit_cast(v8bf, b[0]);
    if constexpr (C::MF == 32)
      acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(va, vb, acc, 0, 0, 0);
    else
      acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(va, vb, acc, 0, 0, 0);
  } else {
    v8i va, vb;
    va[0] = a[0][0]; va[1] = a[0][1]; va[2] = a[0][2]; va[3] = a[0][3];
    vb[0] = b[0][0]; vb[1] = b[0][1]; vb[2] = b[0][2]; vb[3] = b[0][3];
    if constexpr (C::DT == DT_FP8) {
      va[4] = a[1][0]; va[5] = a[1][1]; va[6] = a[1][2]; va[7] = a[1][3];
      vb[4] = b[1][0]; vb[5] = b[1][1]; vb[6] = b[1][2]; vb[7] = b[1][3];
    } else {
      va[4] = va[5] = va[6] = va[7] = 0;
      vb[4] = vb[5] = vb[6] = vb[7] = 0;
    }
    constexpr int fmt = C::DT == DT_FP8 ? 0 : 4;   // 0 = E4M3, 4 = E2M1
    if constexpr (C::MF == 32)
      acc = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(va, vb, acc, fmt, fmt, OP, sa, OP, sb);
    else
      acc = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(va, vb, acc, fmt, fmt, OP, sa, OP, sb);
  }
}

// ---------------------------------------------------------------- epilogue rounding

// bf16 nearest-even of the exact value t + bias, where t and bias are fp32.
// s = fl(t + bias) carries an error e (TwoSum).  Rounding s to bf16 gives the
// right answer unless s sits exactly on a bf16 midpoint while e != 0: then the
// exact sum lies on e's side of the midpoint.
__device__ __forceinline__ uint16_t round_sum_bf16(float t, float bias) {
#pragma clang fp contract(off)
  const float s = t + bias;
  const float bv = s - t;
  const float av = s - bv;
  const float e = (t - av) + (bias - bv);
  const uint32_t u = __float_as_uint(s);
  if ((u & 0x7f800000u) == 0x7f800000u) return (u & 0x007fffffu) ? (uint16_t)0x7fc0 : (uint16_t)(u >> 16);
  if ((u & 0xffffu) == 0x8000u && e != 0.0f) {
    const uint32_t low = u >> 16;                       // neighbour nearer zero
    return (uint16_t)(((e > 0.0f) == (s > 0.0f)) ? low + 1 : low);
  }
  return (uint16_t)((u + 0x7fffu + ((u >> 16) & 1u)) >> 16);
}

__device__ __forceinline__ float bf16_to_float(uint16_t h) { return __uint_as_float((uint32_t)h << 16); }

// ---------------------------------------------------------------- the kernel body

template <class C>
struct Kernel {
  static constexpr int NT = C::NT;

  // Register staging for one k-step of global loads.
  struct Stage {
    v4u a[C::A_PT];
    v4u b[C::B_PT];
    v2u sa[C::SA_PT > 0 ? C::SA_PT : 1];
    v2u sb[C::SB_PT > 0 ? C::SB_PT : 1];
  };

  struct TileCtx {
    __amdgpu_buffer_rsrc_t ra, rb, rsa, rsb;
    int64_t m0, n0;
  };

  static __device__ __forceinline__ int swz(int row, int c) { return c ^ (row & (C::CPR - 1)); }

  static __device__ __forceinline__ TileCtx tile_ctx(const KArgs& a, int64_t tile) {
    TileCtx t;
    const int64_t tm = tile / a.tiles_n, tn = tile - tm * a.tiles_n;
    t.m0 = tm * C::BM;
    t.n0 = tn * C::BN;
    const int64_t rows_a = min((int64_t)C::BM, a.M - t.m0);
    const int64_t rows_b = min((int64_t)C::BN, a.N - t.n0);
    t.ra = make_rsrc(a.A + t.m0 * a.a_pitch, (uint32_t)(rows_a * a.a_pitch));
    t.rb = make_rsrc(a.B + t.n0 * a.b_pitch, (uint32_t)(rows_b * a.b_pitch));
    if constexpr (C::DT == DT_MXFP4) {
      t.rsa = make_rsrc(a.SA + t.m0 * a.s_pitch, (uint32_t)(rows_a * a.s_pitch));
      t.rsb = make_rsrc(a.SB + t.n0 * a.s_pitch, (uint32_t)(rows_b * a.s_pitch));
    } else {
      t.rsa = t.ra;
      t.rsb = t.rb;
    }
    return t;
  }

  // 8 scale bytes of one row for k-step ks; bytes past K/32 read as 127 (x1) so
  // that they never turn the zero padding into NaN.
  static __device__ __forceinline__ v2u load_scales(const KArgs& a, __amdgpu_buffer_rsrc_t rs, int row, int ks) {
    const uint32_t off = (uint32_t)(row * a.s_pitch) + (uint32_t)(ks * C::SPR);
    if (a.scale_fast) {
      if constexpr (C::SPR == 8) return __builtin_amdgcn_raw_buffer_load_b64(rs, off, 0, 0);
      else return v2u{__builtin_amdgcn_raw_buffer_load_b32(rs, off, 0, 0), 0u};
    }
    uint32_t w[2] = {0u, 0u};
#pragma unroll
    for (int j = 0; j < C::SPR; ++j) {
      const bool in = (int64_t)ks * C::SPR + j < a.s_pitch;
      uint32_t v = __builtin_amdgcn_raw_buffer_load_b8(rs, in ? off + j : kOob, 0, 0);
      if (!in) v = 127u;
      w[j >> 2] |= v << (8 * (j & 3));
    }
    return v2u{w[0], w[1]};
  }

  static __device__ __forceinline__ void gload(const KArgs& a, const TileCtx& t, int ks, Stage& st) {
    const int tid = threadIdx.x;
    const int64_t kbyte = (int64_t)ks * C::KB;
#pragma unroll
    for (int i = 0; i < C::A_PT; ++i) {
      const int id = tid + i * NT;
      if (C::A_CH % NT == 0 || id < C::A_CH) {
        const int row = id / C::CPR, c = id % C::CPR;
        const bool in = kbyte + c * 16 < a.row_bytes;
        const uint32_t off = in ? (uint32_t)(row * a.a_pitch + kbyte + c * 16) : kOob;
        st.a[i] = __builtin_amdgcn_raw_buffer_load_b128(t.ra, off, 0, 0);
      }
    }
#pragma unroll
    for (int i = 0; i < C::B_PT; ++i) {
      const int id = tid + i * NT;
      if (C::B_CH % NT == 0 || id < C::B_CH) {
        const int row = id / C::CPR, c = id % C::CPR;
        const bool in = kbyte + c * 16 < a.row_bytes;
        const uint32_t off = in ? (uint32_t)(row * a.b_pitch + kbyte + c * 16) : kOob;
        st.b[i] = __builtin_amdgcn_raw_buffer_load_b128(t.rb, off, 0, 0);
      }
    }
    if constexpr (C::DT == DT_MXFP4) {
#pragma unroll
      for (int i = 0; i < C::SA_PT; ++i) {
        const int row = tid + i * NT;
        if (C::BM % NT == 0 || row < C::BM) st.sa[i] = load_scales(a, t.rsa, row, ks);
      }
#pragma unroll
      for (int i = 0; i < C::SB_PT; ++i) {
        const int row = tid + i * NT;
        if (C::BN % NT == 0 || row < C::BN) st.sb[i] = load_scales(a, t.rsb, row, ks);
      }
    }
  }

  static __device__ __forceinline__ void sstore(uint8_t* stage, const Stage& st) {
    const int tid = threadIdx.x;
#pragma unroll
    for (int i = 0; i < C::A_PT; ++i) {
      const int id = tid + i * NT;
      if (C::A_CH % NT == 0 || id < C::A_CH) {
        const int row = id / C::CPR, c = id % C::CPR;
        *(v4u*)(stage + C::A_OFF + row * C::KB + swz(row, c) * 16) = st.a[i];
      }
    }
#pragma unroll
    for (int i = 0; i < C::B_PT; ++i) {
      const int id = tid + i * NT;
      if (C::B_CH % NT == 0 || id < C::B_CH) {
        const int row = id / C::CPR, c = id % C::CPR;
        *(v4u*)(stage + C::B_OFF + row * C::KB + swz(row, c) * 16) = st.b[i];
      }
    }
    if constexpr (C::DT == DT_MXFP4) {
#pragma unroll
      for (int i = 0; i < C::SA_PT; ++i) {
        const int row = tid + i * NT;
        if (C::BM % NT == 0 || row < C::BM) {
          if constexpr (C::SPR == 8) *(v2u*)(stage + C::SA_OFF + row * 8) = st.sa[i];
          else *(uint32_t*)(stage + C::SA_OFF + row * 4) = st.sa[i][0];
        }
      }
#pragma unroll
      for (int i = 0; i < C::SB_PT; ++i) {
        const int row = tid + i * NT;
        if (C::BN % NT == 0 || row < C::BN) {
          if constexpr (C::SPR == 8) *(v2u*)(stage + C::SB_OFF + row * 8) = st.sb[i];
          else *(uint32_t*)(stage + C::SB_OFF + row * 4) = st.sb[i][0];
        }
      }
    }
  }

  // Lane's NU scale bytes of one operand row, packed little-endian.
  static __device__ __forceinline__ int lane_scales(const uint8_t* base, int row, int g) {
    const uint8_t* p = base + row * C::SPR + g * C::NU;
    if constexpr (C::NU == 4) return *(const int*)p;
    else if constexpr (C::NU == 2) return (int)*(const uint16_t*)p;
    else return (int)*p;
  }

  static __device__ __forceinline__ void compute(const uint8_t* stage, Acc<C>& acc) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int wm = wave / C::WN, wn = wave % C::WN;
    const int lr = lane % C::MF, g = lane / C::MF;
    int sa[C::FM], sb[C::FN];
    if constexpr (C::DT == DT_MXFP4) {
#pragma unroll
      for (int i = 0; i < C::FM; ++i) sa[i] = lane_scales(stage + C::SA_OFF, wm * C::WTM + i * C::MF + lr, g);
#pragma unroll
      for (int j = 0; j < C::FN; ++j) sb[j] = lane_scales(stage + C::SB_OFF, wn * C::WTN + j * C::MF + lr, g);
    } else {
#pragma unroll
      for (int i = 0; i < C::FM; ++i) sa[i] = 0x7f7f7f7f;   // unit E8M0 block scales
#pragma unroll
      for (int j = 0; j < C::FN; ++j) sb[j] = 0x7f7f7f7f;
    }
    static_for<C::NU>([&](auto uc) {
      constexpr int u = decltype(uc)::value;
      constexpr int NCH = C::U / 16;
      v4u av[C::FM][NCH], bv[C::FN][NCH];
#pragma unroll
      for (int i = 0; i < C::FM; ++i) {
        const int row = wm * C::WTM + i * C::MF + lr;
#pragma unroll
        for (int h = 0; h < NCH; ++h) {
          const int c = (g * C::LB + u * C::U) / 16 + h;
          av[i][h] = *(const v4u*)(stage + C::A_OFF + row * C::KB + swz(row, c) * 16);
        }
      }
#pragma unroll
      for (int j = 0; j < C::FN; ++j) {
        const int row = wn * C::WTN + j * C::MF + lr;
#pragma unroll
        for (int h = 0; h < NCH; ++h) {
          const int c = (g * C::LB + u * C::U) / 16 + h;
          bv[j][h] = *(const v4u*)(stage + C::B_OFF + row * C::KB + swz(row, c) * 16);
        }
      }
#pragma unroll
      for (int i = 0; i < C::FM; ++i)
#pragma unroll
        for (int j = 0; j < C::FN; ++j) mfma<C, (C::DT == DT_MXFP4 ? u : 0)>(acc.v[i][j], av[i], bv[j], sa[i], sb[j]);
    });
  }

  // MAC iterations [k0, k1) of one tile into acc (which the caller zeroed).
  static __device__ __forceinline__ void mac(const KArgs& a, int64_t tile, int k0, int k1, Acc<C>& acc,
                                             uint8_t* smem) {
    const TileCtx t = tile_ctx(a, tile);
    Stage st;
    gload(a, t, k0, st);
    sstore(smem, st);
    __syncthreads();
    for (int ks = k0; ks < k1; ++ks) {
      uint8_t* cur = smem + ((ks - k0) & 1) * C::STAGE;
      uint8_t* nxt = smem + (((ks - k0) & 1) ^ 1) * C::STAGE;
      const bool more = ks + 1 < k1;
      if (more) gload(a, t, ks + 1, st);
      compute(cur, acc);
      if (more) sstore(nxt, st);
      __syncthreads();
    }
  }

  static __device__ __forceinline__ float* slot(const KArgs& a, int w) {
    return a.P + (int64_t)w * C::P_SLOT + (threadIdx.x >> 6) * C::P_WAVE;
  }

  static __device__ __forceinline__ void store_partial(const KArgs& a, int w, const Acc<C>& acc) {
    float* p = slot(a, w);
    const int lane = threadIdx.x & 63;
#pragma unroll
    for (int i = 0; i < C::FM; ++i)
#pragma unroll
      for (int j = 0; j < C::FN; ++j)
#pragma unroll
        for (int q = 0; q < C::ACC / 4; ++q) {
          v4f v;
          v[0] = acc.v[i][j][4 * q + 0]; v[1] = acc.v[i][j][4 * q + 1];
          v[2] = acc.v[i][j][4 * q + 2]; v[3] = acc.v[i][j][4 * q + 3];
          *(v4f*)(p + (((i * C::FN + j) * (C::ACC / 4) + q) * 64 + lane) * 4) = v;
        }
  }

  static __device__ __forceinline__ void add_partial(const KArgs& a, int w, Acc<C>& acc) {
    const float* p = slot(a, w);
    const int lane = threadIdx.x & 63;
#pragma unroll
    for (int i = 0; i < C::FM; ++i)
#pragma unroll
      for (int j = 0; j < C::FN; ++j)
#pragma unroll
        for (int q = 0; q < C::ACC / 4; ++q) {
          const v4f v = *(const v4f*)(p + (((i * C::FN + j) * (C::ACC / 4) + q) * 64 + lane) * 4);
          acc.v[i][j][4 * q + 0] += v[0]; acc.v[i][j][4 * q + 1] += v[1];
          acc.v[i][j][4 * q + 2] += v[2]; acc.v[i][j][4 * q + 3] += v[3];
        }
  }

  // Publish this workgroup's partial: every thread's stores become visible at
  // device scope before the flag does.
  static __device__ __forceinline__ void publish(const KArgs& a, int w) {
    if (a.delay_seed) {
      uint32_t h = a.delay_seed ^ (0x9e3779b9u * (uint32_t)(w + 1));
      h ^= h >> 15; h *= 0x2c1b3c6du; h ^= h >> 12;
      const int n = (int)(h % 48u);
      for (int i = 0; i < n; ++i) __builtin_amdgcn_s_sleep(127);
    }
    __threadfence();
    __syncthreads();
    if (threadIdx.x == 0 && w != a.drop_wg)
      __hip_atomic_store(a.locks + w, a.epoch, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_AGENT);
  }

  // Wait until workgroup v has published; false if the spin limit ran out.
  static __device__ __forceinline__ bool wait_for(const KArgs& a, int v, int* s_flag) {
    if (threadIdx.x == 0) {
      const uint64_t t0 = __builtin_amdgcn_s_memrealtime();
      int ok = 1;
      while (__hip_atomic_load(a.locks + v, __ATOMIC_ACQUIRE, __HIP_MEMORY_SCOPE_AGENT) != a.epoch) {
        __builtin_amdgcn_s_sleep(2);
        if (__builtin_amdgcn_s_memrealtime() - t0 > a.spin_limit) {
          ok = 0;
          break;
        }
      }
      if (!ok) __hip_atomic_store(a.err, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      *s_flag = ok;
    }
    __syncthreads();
    const int ok = *s_flag;
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
    __syncthreads();
    return ok != 0;
  }

  static __device__ __forceinline__ void epilogue(const KArgs& a, int64_t tile, const Acc<C>& acc) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int wm = wave / C::WN, wn = wave % C::WN;
    const int lr = lane % C::MF, g = lane / C::MF;
    const int64_t tm = tile / a.tiles_n, tn = tile - tm * a.tiles_n;
    const int64_t m0 = tm * C::BM + wm * C::WTM, n0 = tn * C::BN + wn * C::WTN;
    float sigma = 1.0f;
    if constexpr (C::DT == DT_FP8) {
      const float x = a.fsa ? *a.fsa : 1.0f;
      const float y = a.fsb ? *a.fsb : 1.0f;
      sigma = x * y;
    }
#pragma unroll
    for (int j = 0; j < C::FN; ++j) {
      const int64_t col = n0 + j * C::MF + lr;
      const bool col_ok = col < a.N;
      const float bias = (a.bias && col_ok) ? bf16_to_float(a.bias[col]) : 0.0f;
#pragma unroll
      for (int i = 0; i < C::FM; ++i) {
#pragma unroll
        for (int e = 0; e < C::ACC; ++e) {
          const int r = C::MF == 32 ? 8 * (e / 4) + 4 * g + (e % 4) : 4 * g + e;
          const int64_t row = m0 + i * C::MF + r;
          if (col_ok && row < a.M) {
            float t = acc.v[i][j][e];
            if constexpr (C::DT == DT_FP8) t = t * sigma;
            a.C[row * a.N + col] = round_sum_bf16(t, bias);
          }
        }
      }
    }
  }

  static __device__ void run(const KArgs& a) {
    __shared__ __attribute__((aligned(16))) uint8_t smem[C::LDS];
    __shared__ int s_flag;
    const int w = blockIdx.x;
    Acc<C> acc;
    WorkIter work(w, a.sk_tiles, a.tiles, a.iters, a.q, a.r, a.G);
    WorkItem it;
    while (work.next(it)) {
      acc.zero();
      mac(a, it.tile, it.k0, it.k1, acc, smem);
      if (it.mode == WORK_CONTRIB) {
        store_partial(a, w, acc);
        publish(a, w);
        continue;
      }
      bool ok = true;
      if (it.mode == WORK_OWNER) {
        // Partials are added in descending workgroup order, a fixed order.
        for (int v = w - 1; v >= it.first; --v) {
          if (!wait_for(a, v, &s_flag)) {
            ok = false;
            break;
          }
          add_partial(a, v, acc);
        }
      }
      if (ok) epilogue(a, it.tile, acc);
    }
  }
};

template <class C, int OCC>
__global__ __launch_bounds__(C::NT) __attribute__((amdgpu_waves_per_eu(OCC, OCC)))
void sk_gemm_kernel(KArgs a) {
  Kernel<C>::run(a);
}

template <class C, int OCC>
hipError_t launch_variant(int grid, const KArgs& a, hipStream_t s) {
  hipLaunchKernelGGL((sk_gemm_kernel<C, OCC>), dim3(grid), dim3(C::NT), 0, s, a);
  return hipGetLastError();
}

#define SK_VARIANT(DT, BM, BN, KB, MF, WM, WN, OCC)                                                     \
  Variant {                                                                                              \
    DT, BM, BN, KB, Cfg<DT, BM, BN, KB, MF, WM, WN>::BK, MF, Cfg<DT, BM, BN, KB, MF, WM, WN>::NT,       \
        Cfg<DT, BM, BN, KB, MF, WM, WN>::LDS, &launch_variant<Cfg<DT, BM, BN, KB, MF, WM, WN>, OCC>     \
  }

static const Variant kVariants[] = {
    // MXFP4
    SK_VARIANT(DT_MXFP4, 256, 256, 128, 32, 2, 2, 1),
    SK_VARIANT(DT_MXFP4, 128, 128, 128, 32, 2, 2, 1),
    SK_VARIANT(DT_MXFP4, 64, 64, 64, 32, 2, 2, 2),
    SK_VARIANT(DT_MXFP4, 16, 256, 128, 16, 1, 4, 1),
    SK_VARIANT(DT_MXFP4, 16, 128, 128, 16, 1, 4, 1),
    // bf16
    SK_VARIANT(DT_BF16, 256, 256, 128, 32, 2, 2, 1),
    SK_VARIANT(DT_BF16, 128, 128, 128, 32, 2, 2, 1),
    SK_VARIANT(DT_BF16, 128, 192, 128, 32, 2, 2, 1),
    SK_VARIANT(DT_BF16, 64, 64, 64, 32, 2, 2, 2),
    // fp8
    SK_VARIANT(DT_FP8, 256, 256, 128, 32, 2, 2, 1),
    SK_VARIANT(DT_FP8, 128, 128, 128, 32, 2, 2, 1),
    SK_VARIANT(DT_FP8, 64, 64, 64, 32, 2, 2, 2),
    SK_VARIANT(DT_FP8, 16, 256, 128, 16, 1, 4, 1),
};

int num_variants() { return (int)(sizeof(kVariants) / sizeof(kVariants[0])); }
const Variant* variant(int index) {
  return (index >= 0 && index < num_variants()) ? &kVariants[index] : nullptr;
}

}  // namespace sk
