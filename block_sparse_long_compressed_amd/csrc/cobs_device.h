// Device-side helpers for the gfx950 kernels: element types, 16-byte vector
// loads, MFMA wrappers and wave-level reductions.  Wavefronts are 64 lanes.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace cobs {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int kBlock = 64;      // keys per block (the method's block size)
constexpr int kWave = 64;       // lanes per wavefront

__device__ __forceinline__ float bf16_bits_to_f32(uint32_t h16) { return __uint_as_float(h16 << 16); }

// Round-to-nearest-even float -> bf16 bits (inputs are finite).
__device__ __forceinline__ uint32_t f32_to_bf16_bits(float f) {
  uint32_t u = __float_as_uint(f);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return u >> 16;
}

// Two floats rounded to nearest-even bf16, packed (lo in bits 0..15): one
// v_cvt_pk_bf16_f32 on gfx950.
typedef float f32x2_t __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2_t{lo, hi}), bf16x2_t));
}

// Element traits.  A 16-byte chunk holds kPer16 elements.
struct EltBF16 {
  typedef uint16_t storage;
  static constexpr int kPer16 = 8;
  static constexpr int kBytes = 2;
  // unpack element e (0..7) of a 16-byte chunk
  __device__ static __forceinline__ float get(const u32x4& c, int e) {
    uint32_t w = c[e >> 1];
    return (e & 1) ? __uint_as_float(w & 0xFFFF0000u) : __uint_as_float(w << 16);
  }
};
struct EltF32 {
  typedef float storage;
  static constexpr int kPer16 = 4;
  static constexpr int kBytes = 4;
  __device__ static __forceinline__ float get(const u32x4& c, int e) { return __uint_as_float(c[e]); }
};

__device__ __forceinline__ u32x4 ld16(const void* p) {
  return *reinterpret_cast<const u32x4*>(p);
}
__device__ __forceinline__ void st16(void* p, const u32x4& v) {
  *reinterpret_cast<u32x4*>(p) = v;
}
__device__ __forceinline__ f32x4 ld_f32x4(const float* p) {
  return *reinterpret_cast<const f32x4*>(p);
}
__device__ __forceinline__ void st_f32x4(float* p, const f32x4& v) {
  *reinterpret_cast<f32x4*>(p) = v;
}

// D = A(16x32 bf16) * B(32x16 bf16) + C.  Lane l supplies A[l%16][8*(l/16)+j]
// and B[8*(l/16)+j][l%16] (j = 0..7), and holds C[4*(l/16)+i][l%16] (i = 0..3).
__device__ __forceinline__ f32x4 mfma_bf16_16x16x32(const u32x4& a, const u32x4& b, const f32x4& c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                 __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}
// D = A(16x4 f32) * B(4x16 f32) + C.  Lane l supplies A[l%16][l/16] and
// B[l/16][l%16], and holds C[4*(l/16)+i][l%16].
__device__ __forceinline__ f32x4 mfma_f32_16x16x4(float a, float b, const f32x4& c) {
  return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ float shfl_xor_f(float v, int m) { return __shfl_xor(v, m, kWave); }

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }
__device__ __forceinline__ float fast_log2(float x) { return __builtin_amdgcn_logf(x); }

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr float kLnBlock = 4.1588830833596715f;   // ln 64: a full block's ln n_b

// Order-preserving map of a float to uint32 (larger float -> larger key); -0 maps as +0.
__device__ __forceinline__ uint32_t orderable(float f) {
  uint32_t u = __float_as_uint(f + 0.0f);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}


// Inclusive prefix sum across the 64 lanes of a wave with DPP row shifts and
// row broadcasts (no LDS round trips).
__device__ __forceinline__ int wave_inclusive_sum(int x) {
  x += __builtin_amdgcn_update_dpp(0, x, 0x111, 0xf, 0xf, false);   // row_shr:1
  x += __builtin_amdgcn_update_dpp(0, x, 0x112, 0xf, 0xf, false);   // row_shr:2
  x += __builtin_amdgcn_update_dpp(0, x, 0x114, 0xf, 0xf, false);   // row_shr:4
  x += __builtin_amdgcn_update_dpp(0, x, 0x118, 0xf, 0xf, false);   // row_shr:8
  x += __builtin_amdgcn_update_dpp(0, x, 0x142, 0xa, 0xf, false);   // row_bcast:15
  x += __builtin_amdgcn_update_dpp(0, x, 0x143, 0xc, 0xf, false);   // row_bcast:31
  return x;
}

// ---------------------------------------------------------------------------
// Hand-off between workgroups of one launch.  The XCDs of the chip have
// separate L2 caches, so data one workgroup leaves for another is written and
// read with the sc1 cache policy (coherent at device scope; what device-scope
// atomic loads and stores compile to), which avoids the whole-L2 write-back and
// invalidate of a device-scope fence.  A writer waits for its stores to be
// acknowledged (s_waitcnt vmcnt(0)) before the workgroup bumps the counter.
// ---------------------------------------------------------------------------
constexpr int kCoherent = 16;   // CPol SC1

struct Coherent {
  __amdgpu_buffer_rsrc_t rsrc;
  __device__ __forceinline__ explicit Coherent(const void* base, uint32_t bytes)
      : rsrc(__builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, bytes, 0x00020000)) {}
  __device__ __forceinline__ void st4(uint32_t byte_off, const f32x4& v) const {
    __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, v), rsrc, byte_off, 0, kCoherent);
  }
  __device__ __forceinline__ void st1(uint32_t byte_off, float v) const {
    __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(v), rsrc, byte_off, 0, kCoherent);
  }
  __device__ __forceinline__ f32x4 ld4(uint32_t byte_off) const {
    return __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(rsrc, byte_off, 0, kCoherent));
  }
  __device__ __forceinline__ float ld1(uint32_t byte_off) const {
    return __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(rsrc, byte_off, 0, kCoherent));
  }
  // the same load marked volatile (bit 31 of the cache-policy operand), for a value
  // another workgroup publishes while this one polls: it is re-read on every call
  __device__ __forceinline__ uint32_t poll1(uint32_t byte_off) const {
    return __builtin_amdgcn_raw_buffer_load_b32(rsrc, byte_off, 0, kCoherent | (int)0x80000000u);
  }
};

// All threads: wait until this thread's coherent stores are acknowledged, then
// the workgroup synchronises and one thread increments the counter.  Returns
// true in every thread of the workgroup that arrived last (of `expected`).
__device__ __forceinline__ bool arrive_last(uint32_t* counter, uint32_t expected, int* lds_flag) {
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  if (threadIdx.x == 0) {
    const uint32_t prev = __hip_atomic_fetch_add(counter, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    *lds_flag = (prev == expected - 1) ? 1 : 0;
  }
  __syncthreads();
  return *lds_flag != 0;
}

__device__ __forceinline__ void reset_counter(uint32_t* counter) {
  __hip_atomic_store(counter, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

}  // namespace cobs
