// scan_common.h -- device helpers shared by the Mamba-1 scan kernels
// (forward, backward): element access for float32 / bfloat16 rows, raw
// 16-byte chunk loads, and DPP exchanges inside groups of 1, 2 or 4 lanes.
// Internal; not part of the public ABI.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

#include "device_math.h"

namespace ssm {
namespace scan {

// ---- element access ------------------------------------------------------

template <typename In> struct Elem;
template <> struct Elem<float> {
  static constexpr int kPer16B = 4;
  __device__ static float load(const float* p, int64_t i) { return p[i]; }
  __device__ static void unpack(const uint4& v, float* o) {
    o[0] = __uint_as_float(v.x); o[1] = __uint_as_float(v.y);
    o[2] = __uint_as_float(v.z); o[3] = __uint_as_float(v.w);
  }
  __device__ static void store(float* p, int64_t i, float x) { p[i] = x; }
  __device__ static uint4 pack(const float* x) {
    return make_uint4(__float_as_uint(x[0]), __float_as_uint(x[1]),
                      __float_as_uint(x[2]), __float_as_uint(x[3]));
  }
};
template <> struct Elem<uint16_t> {  // bfloat16 bit pattern
  static constexpr int kPer16B = 8;
  __device__ static float widen(uint32_t bits16) { return __uint_as_float(bits16 << 16); }
  __device__ static float load(const uint16_t* p, int64_t i) { return widen(p[i]); }
  __device__ static void unpack(const uint4& v, float* o) {
    const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      o[2 * k] = __uint_as_float(w[k] << 16);
      o[2 * k + 1] = __uint_as_float(w[k] & 0xffff0000u);
    }
  }
  // float -> bf16, round to nearest even (inputs are finite here).
  __device__ static uint16_t narrow(float x) {
    const __bf16 h = static_cast<__bf16>(x);
    return __builtin_bit_cast(uint16_t, h);
  }
  __device__ static void store(uint16_t* p, int64_t i, float x) { p[i] = narrow(x); }
  // Eight floats -> eight bf16 (round to nearest even), one conversion per pair.
  __device__ static uint4 pack(const float* x) {
    return make_uint4(pack_bf16x2(x[0], x[1]), pack_bf16x2(x[2], x[3]),
                      pack_bf16x2(x[4], x[5]), pack_bf16x2(x[6], x[7]));
  }
};

// Raw (undecoded) input words for K consecutive elements of one row, held in
// registers between the load of a time chunk and its use one chunk later.
template <typename In, int K>
struct RawSeg {
  static constexpr int kWords = (K * (int)sizeof(In) + 3) / 4;
  uint32_t w[kWords];
};

// Load p[base + t0 .. base + t0 + K) into raw words, zero past `limit`.
// 16-byte loads when the segment is 16-byte aligned and complete.
template <typename In, int K>
__device__ __forceinline__ void load_raw(const In* __restrict__ p, int64_t base, int t0,
                                         int limit, RawSeg<In, K>& r) {
  constexpr int V = Elem<In>::kPer16B;
  if constexpr (K % V == 0) {
    if (((base + t0) % V) == 0 && t0 + K <= limit) {
      const uint4* q = reinterpret_cast<const uint4*>(p + base + t0);
#pragma unroll
      for (int k = 0; k < K / V; ++k) {
        const uint4 v = q[k];
        r.w[4 * k] = v.x; r.w[4 * k + 1] = v.y; r.w[4 * k + 2] = v.z; r.w[4 * k + 3] = v.w;
      }
      return;
    }
  }
  if constexpr (K * sizeof(In) == 8) {  // one 8-byte load
    if (((base + t0) % (8 / sizeof(In))) == 0 && t0 + K <= limit) {
      const uint2 v = *reinterpret_cast<const uint2*>(p + base + t0);
      r.w[0] = v.x; r.w[1] = v.y;
      return;
    }
  }
  if constexpr (sizeof(In) == 4) {
#pragma unroll
    for (int k = 0; k < K; ++k)
      r.w[k] = (t0 + k < limit) ? reinterpret_cast<const uint32_t*>(p)[base + t0 + k] : 0u;
  } else {
#pragma unroll
    for (int k = 0; k < r.kWords; ++k) r.w[k] = 0u;
#pragma unroll
    for (int k = 0; k < K; ++k)
      if (t0 + k < limit) r.w[k / 2] |= (uint32_t)p[base + t0 + k] << (16 * (k & 1));
  }
}

template <typename In, int K>
__device__ __forceinline__ void decode_raw(const RawSeg<In, K>& r, float (&out)[K]) {
  if constexpr (sizeof(In) == 4) {
#pragma unroll
    for (int k = 0; k < K; ++k) out[k] = __uint_as_float(r.w[k]);
  } else {
#pragma unroll
    for (int k = 0; k < K; ++k)
      out[k] = __uint_as_float((k & 1) ? (r.w[k / 2] & 0xffff0000u) : (r.w[k / 2] << 16));
  }
}

// Element I (compile-time) of a raw segment, widened to float.
template <typename In, int K, int I>
__device__ __forceinline__ float raw_elem(const RawSeg<In, K>& r) {
  static_assert(I >= 0 && I < K, "element index");
  if constexpr (sizeof(In) == 4) {
    return __uint_as_float(r.w[I]);
  } else {
    return __uint_as_float((I & 1) ? (r.w[I / 2] & 0xffff0000u) : (r.w[I / 2] << 16));
  }
}

template <typename In, int K>
__device__ __forceinline__ void store_seg(In* __restrict__ p, int64_t base, int t0, int limit,
                                          const float (&v)[K]) {
  constexpr int V = Elem<In>::kPer16B;
  if constexpr (K % V == 0) {
    if (((base + t0) % V) == 0 && t0 + K <= limit) {
      uint4* q = reinterpret_cast<uint4*>(p + base + t0);
#pragma unroll
      for (int k = 0; k < K / V; ++k) q[k] = Elem<In>::pack(v + k * V);
      return;
    }
  }
#pragma unroll
  for (int k = 0; k < K; ++k)
    if (t0 + k < limit) Elem<In>::store(p, base + t0 + k, v[k]);
}

// softplus for a row of the given input type: exact log1p for float32
// inputs, the shorter form for bfloat16 inputs.
template <typename In>
__device__ __forceinline__ float softplus_in(float x) {
  if constexpr (sizeof(In) == 2) return softplus_short_f(x);
  else return softplus_f(x);
}

// ---- lane-group exchange (DPP) ---------------------------------------------

constexpr int quad_perm(int a, int b, int c, int d) { return a | (b << 2) | (c << 4) | (d << 6); }
constexpr int kSwapPairs = quad_perm(1, 0, 3, 2);   // lane ^ 1
constexpr int kSwapHalves = quad_perm(2, 3, 0, 1);  // lane ^ 2

// Every lane of a group of LPC (1, 2 or 4) consecutive lanes reads slot s of
// its group.
template <int LPC>
constexpr int group_bcast(int s) {
  return LPC == 4 ? quad_perm(s, s, s, s) : LPC == 2 ? quad_perm(s, s, 2 + s, 2 + s)
                                                     : quad_perm(0, 1, 2, 3);
}

// A DPP quad permute of v.  Written with bound_ctrl and a zero "old" value so
// that the compiler can fold it into the VALU instruction that consumes it.
template <int CTRL>
__device__ __forceinline__ float dpp_f(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xF, 0xF, true));
}

template <int I, int E, class F>
__device__ __forceinline__ void static_for(F&& f) {
  if constexpr (I < E) {
    f(std::integral_constant<int, I>{});
    static_for<I + 1, E>(f);
  }
}

}  // namespace scan
}  // namespace ssm
