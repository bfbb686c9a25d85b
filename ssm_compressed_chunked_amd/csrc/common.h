// Device helpers shared by the HIP kernels of libattamba (gfx950, wave64).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace attamba {

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.69314718055994531f;
constexpr int kWave = 64;

// Storage types: float32 or bf16 activations; arithmetic is always float32.
__device__ __forceinline__ float to_f32(float v) { return v; }
__device__ __forceinline__ float to_f32(__bf16 v) { return static_cast<float>(v); }
template <typename T> __device__ __forceinline__ T from_f32(float v);
template <> __device__ __forceinline__ float from_f32<float>(float v) { return v; }
// gfx950 converts with v_cvt_pk_bf16_f32: round to nearest even.
template <> __device__ __forceinline__ __bf16 from_f32<__bf16>(float v) { return static_cast<__bf16>(v); }

// Hardware transcendental instructions: v_exp_f32 (2^x), v_log_f32 (log2 x), v_rcp_f32.
__device__ __forceinline__ float hw_exp2(float x) { return __builtin_amdgcn_exp2f(x); }
__device__ __forceinline__ float hw_log2(float x) { return __builtin_amdgcn_logf(x); }
__device__ __forceinline__ float hw_rcp(float x) { return __builtin_amdgcn_rcpf(x); }

// softplus(z) = ln(1 + e^z) with e = e^z and w = fl(1 + e). For e < 1 the rounding error of that
// sum, c = e - (w - 1), is exact (Dekker's Fast2Sum: |1| >= |e|, and w - 1 is exact by Sterbenz's
// lemma), and ln(1 + e) = ln(w) + ln(1 + c / w) = ln(w) + c to within c e, which keeps full
// relative accuracy when e is small. For e >= 1 the correction (at most 2^-24) is about one ulp
// of the result or less and is left out; for z > 20 the result is z to float32 precision.
__device__ __forceinline__ float softplus_f32(float z) {
  const float e = hw_exp2(z * kLog2e);
  const float w = 1.0f + e;
  const float c = e < 1.0f ? e - (w - 1.0f) : 0.0f;
  const float r = fmaf(hw_log2(w), kLn2, c);
  return z > 20.0f ? z : r;
}

// silu(v) = v sigmoid(v) = v / (1 + e^-v), with the hardware exponential and reciprocal (each
// within about one ulp); for v far below zero e^-v is +inf and the result is -0.
__device__ __forceinline__ float silu_f32(float v) {
  return v * hw_rcp(1.0f + hw_exp2(-v * kLog2e));
}

__host__ __device__ __forceinline__ int ceil_div(int a, int b) { return (a + b - 1) / b; }

// Per-lane access to channel c of a token-major [T, d] tensor. With BUF (bf16 only) the tensor
// goes through a buffer resource: the lane's byte offset 2c is fixed and the token's offset 2td
// is a scalar, so no per-token vector address arithmetic is issued (T d < 2^31, so both offsets
// and the size fit in 32 bits). Otherwise plain pointers.
template <typename T, bool BUF>
struct Column {
  const T* p;
  __amdgpu_buffer_rsrc_t r;
  __device__ __forceinline__ void init(const T* q, int T_rows, int d) {
    p = q;
    if constexpr (BUF)
      r = __builtin_amdgcn_make_buffer_rsrc(const_cast<T*>(q), (short)0,
                                            static_cast<int>(2u * static_cast<uint32_t>(T_rows) *
                                                             static_cast<uint32_t>(d)),
                                            0x00020000);
  }
  // element (t, c): row offset rd = t d (wave-uniform), channel c
  __device__ __forceinline__ float load(int rd, int c) const {
    if constexpr (BUF) {
      const unsigned short v = __builtin_amdgcn_raw_buffer_load_b16(r, 2u * c, 2u * rd, 0);
      return __uint_as_float(static_cast<uint32_t>(v) << 16);
    } else {
      return to_f32(p[rd + c]);
    }
  }
  __device__ __forceinline__ void store(float v, int rd, int c) const {
    if constexpr (BUF) {
      const __bf16 b = from_f32<__bf16>(v);
      __builtin_amdgcn_raw_buffer_store_b16(__builtin_bit_cast(unsigned short, b), r, 2u * c,
                                            2u * rd, 0);
    } else {
      const_cast<T*>(p)[rd + c] = from_f32<T>(v);
    }
  }
};


}  // namespace attamba
