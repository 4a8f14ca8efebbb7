// state_update.hip -- one decode step of the Mamba-1 recurrence for gfx950.
//
// Sources (web pages; cited by title and section/equation):
//   [SPEC]      "ТЕХНИЧЕСКОЕ ЗАДАНИЕ: Реализовать selective scan (Mamba)",
//               Stage 1 items 3-4 (recurrence, softplus, D skip, silu gate).
//   [EXPLAINED] "Mamba CUDA 实现解析", eqs. (5)-(7) (one step of the
//               diagonal recurrence).
//   [BLELLOCH]  "从顺序到并行用PyTorch实现Blelloch算法加速Mamba状态空间模型",
//               section 1 (the sequential form serves online inference).
//
// One new token per row: h = exp(delta*A) h + delta*B*u, y = C.h + D*u,
// y *= silu(z), with the state read and written in place.  The work is a
// few flops per state entry, so the kernel is bound by the state traffic
// (8 bytes per entry): each lane owns 4 consecutive states of a row (one
// 16-byte load and store), the LPR lanes of a row are consecutive, and the
// readout is summed over them with lane shuffles.  B and C may be given per
// group of channels ([batch, ngroups, dstate]; ngroups = dim: per channel).
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "device_math.h"
#include "selective_scan_launch.h"

namespace ssm {
namespace {

template <typename In>
__device__ __forceinline__ float load_in(const In* p, int64_t i);
template <>
__device__ __forceinline__ float load_in<float>(const float* p, int64_t i) { return p[i]; }
template <>
__device__ __forceinline__ float load_in<uint16_t>(const uint16_t* p, int64_t i) {
  return bf16_bits_to_f32(p[i]);
}
__device__ __forceinline__ void store_out(float* p, int64_t i, float v) { p[i] = v; }
__device__ __forceinline__ void store_out(uint16_t* p, int64_t i, float v) {
  p[i] = f32_to_bf16_bits(v);
}

// LPR: lanes per row (power of two, 4*LPR >= dstate).
template <typename In, int LPR>
__global__ void __launch_bounds__(256) selective_state_update_kernel(StepParams prm) {
  const int64_t gid = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int64_t row = gid / LPR;
  const int slot = (int)(gid % LPR);
  const int64_t rows = (int64_t)prm.batch * prm.dim;
  const bool ok = row < rows;
  const int64_t r = ok ? row : 0;
  const int b = (int)(r / prm.dim), d = (int)(r % prm.dim);
  const int N = prm.dstate;
  const In* __restrict__ u = static_cast<const In*>(prm.u);
  const In* __restrict__ dl = static_cast<const In*>(prm.delta);
  const In* __restrict__ Bm = static_cast<const In*>(prm.B);
  const In* __restrict__ Cm = static_cast<const In*>(prm.C);
  const In* __restrict__ z = static_cast<const In*>(prm.z);

  const float ut = load_in<In>(u, r);
  float dt = load_in<In>(dl, r) + (prm.delta_bias ? prm.delta_bias[d] : 0.0f);
  if (prm.delta_softplus) dt = softplus_f(dt);
  const float dtu = dt * ut;

  // B, C of the row's group
  const int64_t bc = ((int64_t)b * prm.ngroups + d / (prm.dim / prm.ngroups)) * N;
  float* st = prm.state + r * N;
  const int n0 = 4 * slot;
  float h[4], acc = 0.0f;
  const bool full = n0 + 4 <= N && (N & 3) == 0;  // 16-byte aligned, complete
  if (full) {
    const float4 v = *reinterpret_cast<const float4*>(st + n0);
    h[0] = v.x; h[1] = v.y; h[2] = v.z; h[3] = v.w;
  } else {
#pragma unroll
    for (int k = 0; k < 4; ++k) h[k] = (n0 + k < N) ? st[n0 + k] : 0.0f;
  }
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const int n = n0 + k;
    if (n < N) {
      // [EXPLAINED] eqs. (5)-(7): a = exp(delta*A), v = a v + delta B u
      const float a = fast_exp2(dt * prm.A[(int64_t)d * N + n] * kLog2e);
      h[k] = __builtin_fmaf(a, h[k], dtu * load_in<In>(Bm, bc + n));
      acc = __builtin_fmaf(load_in<In>(Cm, bc + n), h[k], acc);
    }
  }
  if (ok) {
    if (full) {
      *reinterpret_cast<float4*>(st + n0) = make_float4(h[0], h[1], h[2], h[3]);
    } else {
#pragma unroll
      for (int k = 0; k < 4; ++k)
        if (n0 + k < N) st[n0 + k] = h[k];
    }
  }
  // readout y = sum_n C[n] h[n] over the row's lanes, then skip and gate
#pragma unroll
  for (int off = LPR / 2; off > 0; off >>= 1) acc += __shfl_xor(acc, off, LPR);
  if (ok && slot == 0) {
    float y = acc + (prm.D ? prm.D[d] : 0.0f) * ut;
    if (z) y *= silu_f(load_in<In>(z, r));
    store_out(static_cast<In*>(prm.y), r, y);
  }
}

template <typename In, int LPR>
hipError_t launch_step(const StepParams& p, hipStream_t stream) {
  const int64_t threads = (int64_t)p.batch * p.dim * LPR;
  dim3 grid((unsigned)((threads + 255) / 256));
  hipLaunchKernelGGL((selective_state_update_kernel<In, LPR>), grid, dim3(256), 0, stream, p);
  return hipGetLastError();
}

template <typename In>
hipError_t launch_step_typed(const StepParams& p, hipStream_t stream) {
  const int q = (p.dstate + 3) / 4;
  if (q <= 1) return launch_step<In, 1>(p, stream);
  if (q <= 2) return launch_step<In, 2>(p, stream);
  if (q <= 4) return launch_step<In, 4>(p, stream);
  if (q <= 8) return launch_step<In, 8>(p, stream);
  return launch_step<In, 16>(p, stream);
}

}  // namespace

hipError_t launch_state_update(const StepParams& p, bool bf16, hipStream_t stream) {
  return bf16 ? launch_step_typed<uint16_t>(p, stream) : launch_step_typed<float>(p, stream);
}

}  // namespace ssm
