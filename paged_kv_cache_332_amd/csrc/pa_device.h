// Device helpers for the gfx950 kernels: element types, conversions and
// wave64 cross-lane reductions.
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>

namespace pa {

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x4 __attribute__((ext_vector_type(4)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kNegInf = -__builtin_huge_valf();

// Storage element tags.  `bits` is the raw storage type.
struct F32 {
  using bits = uint32_t;
  static constexpr int kBytes = 4;
  __device__ static float to_f32(uint32_t b) { return __uint_as_float(b); }
  __device__ static uint32_t from_f32(float x) { return __float_as_uint(x); }
};
struct F16 {
  using bits = uint16_t;
  static constexpr int kBytes = 2;
  __device__ static float to_f32(uint32_t b) {
    return static_cast<float>(__builtin_bit_cast(_Float16, static_cast<uint16_t>(b)));
  }
  __device__ static uint32_t from_f32(float x) {
    return __builtin_bit_cast(uint16_t, static_cast<_Float16>(x));
  }
  // two packed elements of a 32-bit word -> floats
  __device__ static float lo(uint32_t w) { return to_f32(w & 0xFFFFu); }
  __device__ static float hi(uint32_t w) { return to_f32(w >> 16); }
  __device__ static float dot2(uint32_t a, uint32_t b, float c) {
    return __builtin_amdgcn_fdot2(__builtin_bit_cast(f16x2, a), __builtin_bit_cast(f16x2, b), c,
                                  false);
  }
};
struct BF16 {
  using bits = uint16_t;
  static constexpr int kBytes = 2;
  __device__ static float to_f32(uint32_t b) { return __uint_as_float(b << 16); }
  __device__ static uint32_t from_f32(float x) {
    return __builtin_bit_cast(uint16_t, static_cast<__bf16>(x));
  }
  __device__ static float lo(uint32_t w) { return __uint_as_float(w << 16); }
  __device__ static float hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }
  __device__ static float dot2(uint32_t a, uint32_t b, float c) {
    return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, a),
                                           __builtin_bit_cast(bf16x2, b), c, false);
  }
};

// ---------------------------------------------------------------- lanes
__device__ __forceinline__ int lane_id() { return __builtin_amdgcn_mbcnt_hi(~0u, __builtin_amdgcn_mbcnt_lo(~0u, 0u)); }

template <int CTRL>
__device__ __forceinline__ float dpp(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xF, 0xF, true));
}
// DPP controls (all stay inside a 16-lane row)
constexpr int kQuadXor1 = 0xB1;     // quad_perm [1,0,3,2]
constexpr int kQuadXor2 = 0x4E;     // quad_perm [2,3,0,1]
constexpr int kRowHalfMirror = 0x141;
constexpr int kRowMirror = 0x140;
constexpr int kRowRor8 = 0x128;     // lane i <- lane (i+8) mod 16 == i ^ 8

struct OpSum {
  __device__ static float op(float a, float b) { return a + b; }
};
struct OpMax {
  __device__ static float op(float a, float b) { return fmaxf(a, b); }
};

// Combine with the lane whose id differs in bit 4 (xor 16) or bit 5 (xor 32).
// The gfx950 permlane swaps exchange 16-lane rows / 32-lane halves between
// two registers; combining the two results is symmetric, so every lane ends
// with op(x[l], x[l ^ 16]) (resp. x[l ^ 32]).
template <class Op>
__device__ __forceinline__ float xor16(float x) {
  auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return Op::op(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
template <class Op>
__device__ __forceinline__ float xor32(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return Op::op(__uint_as_float(r[0]), __uint_as_float(r[1]));
}

// All-reduce over the lanes that differ only in bits [0, NBITS) of the lane
// id (groups of 2^NBITS consecutive lanes).  The mirror patterns pair whole
// already-reduced sub-groups, so bits are taken in increasing order.
template <class Op, int NBITS>
__device__ __forceinline__ float reduce_low_bits(float x) {
  if constexpr (NBITS > 0) x = Op::op(x, dpp<kQuadXor1>(x));
  if constexpr (NBITS > 1) x = Op::op(x, dpp<kQuadXor2>(x));
  if constexpr (NBITS > 2) x = Op::op(x, dpp<kRowHalfMirror>(x));
  if constexpr (NBITS > 3) x = Op::op(x, dpp<kRowMirror>(x));
  if constexpr (NBITS > 4) x = xor16<Op>(x);
  if constexpr (NBITS > 5) x = xor32<Op>(x);
  return x;
}

// All-reduce over lane-id bits [LO, 6) with LO >= 3 (the other bits are
// left as they are): exact xor partners for bits 3, 4, 5.
template <class Op, int LO>
__device__ __forceinline__ float reduce_high_bits(float x) {
  static_assert(LO >= 3, "only bits 3..5 have exact xor partners here");
  if constexpr (LO <= 3) x = Op::op(x, dpp<kRowRor8>(x));
  if constexpr (LO <= 4) x = xor16<Op>(x);
  if constexpr (LO <= 5) x = xor32<Op>(x);
  return x;
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

template <int N>
struct ilog2 {
  static constexpr int value = 1 + ilog2<N / 2>::value;
};
template <>
struct ilog2<1> {
  static constexpr int value = 0;
};

// Keeps the compiler from moving LDS accesses of one wave across this point
// (the LDS unit itself executes one wave's operations in order).
__device__ __forceinline__ void wave_lds_fence() {
  __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
  __builtin_amdgcn_wave_barrier();
}

// Work-item order: items are ranked (kv head, partition, sequence) with the
// sequence fastest, and consecutive ranks are kept on one XCD (workgroups
// are dealt round-robin over the 8 XCDs by id), so the 64 sharers of one
// prefix block read it through the same L2.
constexpr int kNumXcd = 8;
__device__ __forceinline__ int64_t xcd_rank(int64_t total) {
  int64_t per = (total + kNumXcd - 1) / kNumXcd;
  int64_t bid = blockIdx.x;
  return (bid % kNumXcd) * per + bid / kNumXcd;
}
inline int64_t xcd_grid(int64_t total) { return ((total + kNumXcd - 1) / kNumXcd) * kNumXcd; }

// ---------------------------------------------------------------- matrix cores
// v_mfma_f32_16x16x32 for S^T = K Q^T (A: 8 key dims of a token per lane,
// B: 8 query dims of a column per lane) and v_mfma_f32_16x16x16 for
// O^T += V^T P^T (A: 4 tokens of a V row, B: 4 probabilities of a column).
template <class T>
struct MfmaOps;

template <>
struct MfmaOps<BF16> {
  using v8 = bf16x8;
  using v4 = bf16x4;
  using e = __bf16;
  __device__ static f32x4 qk(u32x4 a, u32x4 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(v8, a), __builtin_bit_cast(v8, b),
                                                   c, 0, 0, 0);
  }
  __device__ static f32x4 pv(u32x2 a, v4 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(__builtin_bit_cast(v4, a), b, c, 0, 0, 0);
  }
  // the P.V product over 32 keys at the full rate of the 16x16x32 form
  __device__ static f32x4 pv32(u32x4 a, v8 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(v8, a), b, c, 0, 0, 0);
  }
  // p = hi + lo to about 2^-16 relative: hi is p with its low 16 bits cut
  // off (a bf16 value, packed two a word by one byte permute), lo the exact
  // remainder rounded to bf16
  __device__ static void split(const float (&p)[8], v8& hi, v8& lo) {
    u32x4 h;
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const uint32_t x0 = __float_as_uint(p[2 * k]), x1 = __float_as_uint(p[2 * k + 1]);
      h[k] = __builtin_amdgcn_perm(x1, x0, 0x07060302u);
      lo[2 * k] = static_cast<e>(p[2 * k] - __uint_as_float(x0 & 0xFFFF0000u));
      lo[2 * k + 1] = static_cast<e>(p[2 * k + 1] - __uint_as_float(x1 & 0xFFFF0000u));
    }
    hi = __builtin_bit_cast(v8, h);
  }
};

template <>
struct MfmaOps<F16> {
  using v8 = f16x8;
  using v4 = f16x4;
  using e = _Float16;
  __device__ static f32x4 qk(u32x4 a, u32x4 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(v8, a), __builtin_bit_cast(v8, b), c,
                                                  0, 0, 0);
  }
  __device__ static f32x4 pv(u32x2 a, v4 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x16f16(__builtin_bit_cast(v4, a), b, c, 0, 0, 0);
  }
  __device__ static f32x4 pv32(u32x4 a, v8 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(v8, a), b, c, 0, 0, 0);
  }
  // p = hi + lo: hi is p rounded to f16, lo the exact remainder rounded to f16
  __device__ static void split(const float (&p)[8], v8& hi, v8& lo) {
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      hi[i] = static_cast<e>(p[i]);
      lo[i] = static_cast<e>(p[i] - static_cast<float>(hi[i]));
    }
  }
};

typedef const void __attribute__((address_space(1)))* gptr_t;
typedef void __attribute__((address_space(3)))* lptr_t;

// 16 bytes per lane from src into LDS at dst + 16 * lane.
__device__ __forceinline__ void dma16(const void* src, void* dst) {
  __builtin_amdgcn_global_load_lds((gptr_t)src, (lptr_t)dst, 16, 0, 0);
}

// The same load with a streaming cache policy: the "nt" bit of gfx950
// memory instructions (the caches treat the line as data that will not be
// read again) and "sc0" (the load is not kept in the compute unit's L1).  For
// bytes a launch reads exactly once (the K/V tiles of a decode pass); lines
// that are read again (block tables, lengths, code) then keep their place.
// (nt alone measured about 1 us slower per batch-64 pass; adding sc1 no
// better.)
constexpr int kCpolSc0 = 1, kCpolNt = 2;
constexpr int kCpolStreamOnce = kCpolSc0 | kCpolNt;
__device__ __forceinline__ void dma16_once(const void* src, void* dst) {
  __builtin_amdgcn_global_load_lds((gptr_t)src, (lptr_t)dst, 16, 0, kCpolStreamOnce);
}

// x as an opaque fp32 value: converting the result to 16 bits rounds this
// fp32 value, as converting a stored fp32 output would.  Left visible, the
// multiply that produced x can be fused with the conversion into one
// mixed-precision fma that rounds the exact product once; where the fp32
// product is a tie between two 16-bit values, that can pick the other one.
// The empty asm emits no instruction.
__device__ __forceinline__ float opaque_f32(float x) {
  asm volatile("" : "+v"(x));
  return x;
}

// Wait until at most N vector-memory operations of this wave are outstanding.
// The memory clobber keeps LDS reads of the landed tile below the wait.
template <int N>
__device__ __forceinline__ void vm_wait() {
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

__device__ __forceinline__ void lgkm_wait0() { asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory"); }

// Workgroup barrier without the memory fence of __syncthreads, which would
// wait for every outstanding load of the wave (prefetches into LDS included);
// each wave waits for its own accesses with an explicit count first.  The
// clobber keeps the compiler from moving memory accesses across it.
__device__ __forceinline__ void wg_barrier() { asm volatile("s_barrier" ::: "memory"); }

__device__ __forceinline__ int uniform(int x) { return __builtin_amdgcn_readfirstlane(x); }

}  // namespace pa
