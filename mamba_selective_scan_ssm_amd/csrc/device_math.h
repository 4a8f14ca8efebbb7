// device_math.h -- small float32 device helpers shared by the scan kernels.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace ssm {

// Debug builds with SSM_POISON_LDS defined fill the workgroup's whole static
// LDS with NaN bit patterns at kernel entry, so that a read of LDS that no
// thread of the workgroup wrote first (a missing store or barrier) shows up
// as NaN in the parity tests instead of reading whatever an earlier
// workgroup left there.  Release builds: nothing.
#ifdef SSM_POISON_LDS
__device__ __forceinline__ void poison_lds() {
  typedef __attribute__((address_space(3))) uint32_t lds_u32;
  const uint32_t words = __builtin_amdgcn_groupstaticsize() / 4;
  const uint32_t nthr = blockDim.x * blockDim.y * blockDim.z;
  for (uint32_t i = threadIdx.x; i < words; i += nthr) ((lds_u32*)0)[i] = 0xffffffffu;
  __syncthreads();
}
#define SSM_POISON_LDS_AT_ENTRY() ::ssm::poison_lds()
#else
#define SSM_POISON_LDS_AT_ENTRY() ((void)0)
#endif

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }
__device__ __forceinline__ float fast_log2(float x) { return __builtin_amdgcn_logf(x); }
__device__ __forceinline__ float fast_rcp(float x) { return __builtin_amdgcn_rcpf(x); }

// max(x, 0) for a float that is not NaN, as an integer max of its bits
// (negative floats, -0 included, are negative integers): one instruction,
// with no canonicalisation of x as a float max may need.
__device__ __forceinline__ float relu_bits(float x) {
  return __int_as_float(max(__float_as_int(x), 0));
}

// softplus(x) = log(1 + e^x) = max(x, 0) + log1p(e^{-|x|}).
// log1p(w) for w in (0, 1] is ln(s) + (w - (s - 1)) / s with s = fl(1 + w);
// the correction term is below 2^-24 and is used without the division by s
// (relative error < 2^-24 / ln 2), which keeps small w accurate.
__device__ __forceinline__ float softplus_f(float x) {
  const float w = fast_exp2(-fabsf(x) * kLog2e);
  const float s = 1.0f + w;
  const float corr = w - (s - 1.0f);
  return relu_bits(x) + __builtin_fmaf(fast_log2(s), kLn2, corr);
}

// softplus(x) with log1p(w) taken as ln(fl(1 + w)): the rounding of 1 + w
// leaves an absolute error below 2^-24 in the result (relative error grows
// only where softplus(x) itself is below ~1e-4).  Used for bfloat16 inputs,
// whose own resolution is 2^-9 relative; two VALU instructions fewer.
__device__ __forceinline__ float softplus_short_f(float x) {
  const float w = fast_exp2(-fabsf(x) * kLog2e);
  return __builtin_fmaf(fast_log2(1.0f + w), kLn2, relu_bits(x));
}

// log2(e) softplus(x) from x2 = log2(e) x: max(x2, 0) + log2(fl(1 + 2^{-|x2|}))
// (the bfloat16 form above in log2 units: the same rounding of 1 + w).
__device__ __forceinline__ float softplus_log2_short(float x2) {
  return relu_bits(x2) + fast_log2(1.0f + fast_exp2(-fabsf(x2)));
}

// silu(z) = z * sigmoid(z) = z / (1 + e^{-z})
__device__ __forceinline__ float silu_f(float z) {
  return z * fast_rcp(1.0f + fast_exp2(-z * kLog2e));
}

__device__ __forceinline__ float bf16_bits_to_f32(uint32_t bits16) {
  return __uint_as_float(bits16 << 16);
}

// float -> bf16 bits, round to nearest even (finite inputs).
__device__ __forceinline__ uint16_t f32_to_bf16_bits(float x) {
  return __builtin_bit_cast(uint16_t, static_cast<__bf16>(x));
}

// Two floats -> two bf16 (round to nearest even) in one 32-bit word, lo in
// the low half: a two-wide vector conversion, one v_cvt_pk_bf16_f32.
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  typedef float f32x2_t __attribute__((ext_vector_type(2)));
  typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
  const f32x2_t v = {lo, hi};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2_t));
}

}  // namespace ssm
