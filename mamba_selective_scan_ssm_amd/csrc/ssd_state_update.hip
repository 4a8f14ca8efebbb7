// ssd_state_update.hip -- one decode step of the Mamba-2 (SSD) recurrence
// for gfx950.
//
// Source: "Прорыв в оптимизации SSM-моделей" (aikraft.ru digest of the cuTile
// Mamba-2 forward kernels), "Технические детали": the recurrence
// h_t = exp(A dt_t) h_{t-1} + dt_t B_t x_t with a scalar A per head; the
// output y_t = C_t . h_t + D x_t follows the skip term of "Mamba CUDA 实现解析"
// eq. (2).
//
// One new token per (batch, head): for every p,
//   S[p, n] = exp(dt A_h) S[p, n] + dt x[p] B[n];   y[p] = sum_n C[n] S[p, n] + D_h x[p]
// with the state read and written in place.  A few flops per state entry,
// so the step is bound by the state traffic (8 bytes per entry): each lane
// owns 4 consecutive states of one (batch, head, p) row (one 16-byte load
// and store), the LPR lanes of a row are consecutive, the decay is one exp
// per lane (a scalar per head), and the readout is summed over the row's
// lanes with shuffles.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "device_math.h"
#include "ssd_launch.h"

namespace ssm {
namespace {

template <typename In> __device__ __forceinline__ float ld(const In* p, int64_t i);
template <> __device__ __forceinline__ float ld<float>(const float* p, int64_t i) { return p[i]; }
template <> __device__ __forceinline__ float ld<uint16_t>(const uint16_t* p, int64_t i) {
  return bf16_bits_to_f32(p[i]);
}
__device__ __forceinline__ void st_out(float* p, int64_t i, float v) { p[i] = v; }
__device__ __forceinline__ void st_out(uint16_t* p, int64_t i, float v) {
  p[i] = f32_to_bf16_bits(v);
}

// LPR: lanes per (batch, head, p) row (power of two, 4*LPR >= dstate).
template <typename In, int LPR>
__global__ void __launch_bounds__(256) ssd_state_update_kernel(SsdStepParams prm) {
  const int64_t gid = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int64_t row = gid / LPR;  // (b*nheads + h)*headdim + p
  const int slot = (int)(gid % LPR);
  const int H = prm.nheads, P = prm.headdim, N = prm.dstate;
  const int64_t rows = (int64_t)prm.batch * H * P;
  const bool ok = row < rows;
  const int64_t r = ok ? row : 0;
  const int64_t bh = r / P;
  const int b = (int)(bh / H), h = (int)(bh % H);
  const int g = h / (H / prm.ngroups);
  const In* __restrict__ x = static_cast<const In*>(prm.x);
  const In* __restrict__ dtp = static_cast<const In*>(prm.dt);
  const In* __restrict__ Bm = static_cast<const In*>(prm.B);
  const In* __restrict__ Cm = static_cast<const In*>(prm.C);

  const float xv = ld<In>(x, r);
  float dt = ld<In>(dtp, bh) + (prm.dt_bias ? prm.dt_bias[h] : 0.0f);
  if (prm.dt_softplus) dt = softplus_f(dt);
  const float a = fast_exp2(dt * prm.A[h] * kLog2e);  // one decay per (batch, head)
  const float dtx = dt * xv;
  const int64_t bc = ((int64_t)b * prm.ngroups + g) * N;

  float* st = prm.state + r * N;
  const int n0 = 4 * slot;
  float s[4], acc = 0.0f;
  const bool full = n0 + 4 <= N && (N & 3) == 0;  // 16-byte aligned, complete
  if (full) {
    const float4 v = *reinterpret_cast<const float4*>(st + n0);
    s[0] = v.x; s[1] = v.y; s[2] = v.z; s[3] = v.w;
  } else {
#pragma unroll
    for (int k = 0; k < 4; ++k) s[k] = (n0 + k < N) ? st[n0 + k] : 0.0f;
  }
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const int n = n0 + k;
    if (n < N) {
      s[k] = __builtin_fmaf(a, s[k], dtx * ld<In>(Bm, bc + n));
      acc = __builtin_fmaf(ld<In>(Cm, bc + n), s[k], acc);
    }
  }
  if (ok) {
    if (full) {
      *reinterpret_cast<float4*>(st + n0) = make_float4(s[0], s[1], s[2], s[3]);
    } else {
#pragma unroll
      for (int k = 0; k < 4; ++k)
        if (n0 + k < N) st[n0 + k] = s[k];
    }
  }
  // readout y[p] = sum_n C[n] S[p, n] over the row's lanes, then the skip term
#pragma unroll
  for (int off = LPR / 2; off > 0; off >>= 1) acc += __shfl_xor(acc, off, LPR);
  if (ok && slot == 0)
    st_out(static_cast<In*>(prm.y), r, acc + (prm.D ? prm.D[h] : 0.0f) * xv);
}

template <typename In, int LPR>
hipError_t launch(const SsdStepParams& p, hipStream_t stream) {
  const int64_t threads = (int64_t)p.batch * p.nheads * p.headdim * LPR;
  dim3 grid((unsigned)((threads + 255) / 256));
  hipLaunchKernelGGL((ssd_state_update_kernel<In, LPR>), grid, dim3(256), 0, stream, p);
  return hipGetLastError();
}

template <typename In>
hipError_t launch_typed(const SsdStepParams& p, hipStream_t stream) {
  const int q = (p.dstate + 3) / 4;
  if (q <= 1) return launch<In, 1>(p, stream);
  if (q <= 2) return launch<In, 2>(p, stream);
  if (q <= 4) return launch<In, 4>(p, stream);
  if (q <= 8) return launch<In, 8>(p, stream);
  if (q <= 16) return launch<In, 16>(p, stream);
  if (q <= 32) return launch<In, 32>(p, stream);
  return launch<In, 64>(p, stream);
}

}  // namespace

hipError_t launch_ssd_state_update(const SsdStepParams& p, bool bf16, hipStream_t stream) {
  return bf16 ? launch_typed<uint16_t>(p, stream) : launch_typed<float>(p, stream);
}

}  // namespace ssm
