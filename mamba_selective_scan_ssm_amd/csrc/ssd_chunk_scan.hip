// ssd_chunk_scan.hip -- Mamba-2 (SSD) chunked scan, forward, for gfx950.
//
// Source: "Прорыв в оптимизации SSM-моделей" (aikraft.ru digest of the cuTile
// Mamba-2 forward kernels), sections "Три оптимизированных ядра" and
// "Технические детали оптимизации": the recurrence
// h_t = exp(A dt_t) h_{t-1} + dt_t B_t x_t, cumulative sums of the log-decay
// within chunks, chunk states advanced across chunks with the jump formula,
// and one fused output step combining the carried state, the causal-masked
// intra-chunk interaction and the skip connection.  The output rule
// y_t = C_t . h_t + D_h x_t follows the skip term of "Mamba CUDA 实现解析"
// eq. (2).
//
// Three launches on one stream, all matrix products on MFMA
// (v_mfma_f32_16x16x32_bf16: bf16 operands, fp32 accumulation):
//   1. ssd_chunk_state_kernel   per (chunk, batch, head group):
//        dt -> softplus -> within-chunk inclusive cumsum of A*dt (cs),
//        S_c[p][n] = sum_s exp(cs_last - cs_s) dt_s x_s[p] B_s[n]
//        (MFMA, K = chunk positions), stored as bf16, and exp(cs_last).
//   2. ssd_state_pass_kernel    per (batch, head, state slice):
//        S = exp(cs_last_c) S + S_c across chunks (fp32 in registers); the
//        state entering each chunk overwrites S_c in place (bf16); the last
//        state is final_state (fp32).
//   3. ssd_chunk_out_kernel     per (chunk, 64-row block, batch, head group):
//        G^T[s][l] = B_s . C_l (MFMA, once per workgroup, shared by its heads)
//        M^T[s][l] = G^T[s][l] exp(cs_l - cs_s) dt_s for s <= l (registers)
//        Y^T[p][l] = sum_s x^T[p][s] M^T[s][l]                (MFMA)
//                  + sum_n S_in[p][n] exp(cs_l) C_l[n]        (MFMA)
//        y[l][p]   = Y^T[p][l] + D_h x[l][p]
//   The cumsum is recomputed where needed (it is a 256-element scan per
//   chunk and head) instead of being stored.
//
// MFMA operand layout (checked on the device): for A (16x32), lane i holds
// A[i%16][8(i/16) .. 8(i/16)+7]; for B (32x16), lane i holds
// B[8(i/16) .. +7][i%16]; the 16x16 result gives lane i rows 4(i/16)..+3 of
// column i%16.  Any consistent assignment of the 32 contraction indices to
// the (lane group, slot) pairs is valid, which lets the result of one
// product feed the next as an operand without moving data between lanes.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <cstdio>

#include "device_math.h"
#include "ssd_launch.h"

namespace ssm {

ssm_status ssd_validate_shape(int64_t batch, int64_t seqlen, int64_t nheads, int64_t headdim,
                              int64_t dstate, int64_t ngroups, int64_t chunk, SsdShape* out,
                              std::string* msg) {
  auto bad = [&](ssm_status st, const char* what) {
    *msg = what;
    return st;
  };
  if (batch <= 0 || seqlen <= 0 || nheads <= 0 || headdim <= 0 || dstate <= 0 || ngroups <= 0 ||
      chunk <= 0)
    return bad(SSM_ERR_INVALID_ARG, "all sizes must be >= 1");
  if (nheads % ngroups != 0) return bad(SSM_ERR_INVALID_ARG, "nheads must be a multiple of ngroups");
  if (chunk != 64 && chunk != 128 && chunk != 256)
    return bad(SSM_ERR_UNSUPPORTED, "chunk_size must be 64, 128 or 256");
  if (headdim != 32 && headdim != 64 && headdim != 128)
    return bad(SSM_ERR_UNSUPPORTED, "headdim must be 32, 64 or 128");
  if (dstate != 32 && dstate != 64 && dstate != 128 && dstate != 256)
    return bad(SSM_ERR_UNSUPPORTED, "dstate must be 32, 64, 128 or 256");
  if (batch > 65535 || nheads > 65535 || seqlen > (1 << 30))
    return bad(SSM_ERR_UNSUPPORTED, "batch and nheads must be <= 65535, seqlen <= 2^30");
  out->batch = (int)batch;
  out->seqlen = (int)seqlen;
  out->nheads = (int)nheads;
  out->headdim = (int)headdim;
  out->dstate = (int)dstate;
  out->ngroups = (int)ngroups;
  out->chunk = (int)chunk;
  out->nchunks = (int)((seqlen + chunk - 1) / chunk);
  return SSM_OK;
}

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int kQMax = 256;          // largest chunk
constexpr int kRowQ = kQMax + 8;    // LDS row stride (bf16) of [row][position] tiles

struct SsdArgs {
  const uint16_t* x;
  const uint16_t* dt;
  const float* A;
  const uint16_t* B;
  const uint16_t* C;
  const float* D;
  const float* dt_bias;
  uint16_t* y;
  float* final_state;
  uint16_t* states;
  float* decay;
  int dt_softplus;
  int batch, seqlen, nheads, headdim, dstate, ngroups, chunk, nchunks;
  int heads_per_wg_state, heads_per_wg_out;
};

__device__ __forceinline__ f32x4 mfma_bf16(const bf16x8& a, const bf16x8& b, const f32x4& c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ uint4 load16(const uint16_t* p) {
  return *reinterpret_cast<const uint4*>(p);
}

__device__ __forceinline__ bf16x8 as_bf16x8(const uint4& v) {
  return __builtin_bit_cast(bf16x8, v);
}

// Interleave rows r0 (position s) and r1 (position s+1), 8 bf16 each, into
// eight 32-bit words: word i = (r0[i], r1[i]).
__device__ __forceinline__ void interleave_pairs(const uint4& r0, const uint4& r1, uint32_t (&w)[8]) {
  const uint32_t a[4] = {r0.x, r0.y, r0.z, r0.w};
  const uint32_t b[4] = {r1.x, r1.y, r1.z, r1.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    w[2 * i] = (a[i] & 0xffffu) | (b[i] << 16);
    w[2 * i + 1] = (a[i] >> 16) | (b[i] & 0xffff0000u);
  }
}

// Raw dt of this thread's position (thread t <-> position t of the chunk),
// zero past the chunk or the sequence; loaded one head ahead of its use.
__device__ __forceinline__ uint32_t load_dt_bits(const SsdArgs& a, int b, int c, int h) {
  const int t = threadIdx.x;
  const int64_t pos = (int64_t)c * a.chunk + t;
  if (t < a.chunk && pos < a.seqlen) return a.dt[((int64_t)b * a.seqlen + pos) * a.nheads + h];
  return 0u;
}

// For one (batch, chunk, head): sDt[s] = dt_s after bias and softplus and
// sCs2[s] = log2(e) * sum_{m <= s} A_h dt_m (inclusive, within the chunk), for
// s < chunk; positions past the sequence end have dt = 0.  `dt_bits` is this
// thread's raw dt (from load_dt_bits).  Every thread of the block calls it;
// threads at or past the chunk length contribute nothing.
__device__ void chunk_log_decay(const SsdArgs& a, int c, int h, uint32_t dt_bits, float* sCs2,
                                float* sDt, float* sTmp) {
  const int t = threadIdx.x;
  const int lane = t & 63, wv = t >> 6;
  const int64_t pos = (int64_t)c * a.chunk + t;
  float dtv = 0.0f;
  if (t < a.chunk && pos < a.seqlen) {
    float v = bf16_bits_to_f32(dt_bits);
    if (a.dt_bias) v += a.dt_bias[h];
    dtv = a.dt_softplus ? softplus_f(v) : v;
  }
  float v = a.A[h] * kLog2e * dtv;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const float o = __shfl_up(v, off, 64);
    if (lane >= off) v += o;
  }
  if (lane == 63 && wv < kQMax / 64) sTmp[wv] = v;
  __syncthreads();
  if (t < a.chunk) {
    float add = 0.0f;
    for (int w = 0; w < wv; ++w) add += sTmp[w];
    sCs2[t] = v + add;
    sDt[t] = dtv;
  }
  __syncthreads();
}

// ---- 1. chunk states ---------------------------------------------------------

// One workgroup (NW waves) per (chunk, batch, head group).  B^T of the chunk is
// staged once; each head's (w x)^T is staged from registers loaded while the
// previous head was computing.
template <int P, int NB, int NW>
__global__ void __launch_bounds__(64 * NW) ssd_chunk_state_kernel(SsdArgs a) {
  __shared__ alignas(16) uint16_t sBt[NB][kRowQ];  // B^T of one state block: [n][s]
  __shared__ alignas(16) uint16_t sXt[P][kRowQ];   // (w x)^T of one head: [p][s]
  __shared__ float sCs2[kQMax], sDt[kQMax], sW[kQMax], sTmp[4];
  constexpr int NTHR = 64 * NW;
  constexpr int NT = NB / 16, PT = P / 16, TILES = NT * PT, TPW = (TILES + NW - 1) / NW;
  constexpr int XTASKS = (P / 8) * (kQMax / 2);
  constexpr int XPT = (XTASKS + NTHR - 1) / NTHR;  // x staging tasks per thread (at Q = 256)

  const int c = blockIdx.x, b = blockIdx.y;
  const int hpg = a.nheads / a.ngroups;
  const int h0 = blockIdx.z * a.heads_per_wg_state;
  const int nh = min(a.heads_per_wg_state, a.nheads - h0);
  const int g = h0 / hpg;
  const int Q = a.chunk, N = a.dstate, L = a.seqlen;
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int r16 = lane & 15, q4 = lane >> 4;
  const int64_t pos0 = (int64_t)c * Q;
  const int xtasks = (P / 8) * (Q / 2);

  // Per-head inputs held in registers one head ahead.
  uint4 xr0[XPT], xr1[XPT];
  uint32_t dtb = 0;
  auto prefetch = [&](int h) {
    dtb = load_dt_bits(a, b, c, h);
#pragma unroll
    for (int k = 0; k < XPT; ++k) {
      const int task = tid + k * NTHR;
      xr0[k] = xr1[k] = make_uint4(0, 0, 0, 0);
      if (task < xtasks) {
        const int sp = task % (Q / 2), po = task / (Q / 2);
        const int s = 2 * sp;
        const int64_t row = ((int64_t)b * L + pos0 + s) * a.nheads + h;
        if (pos0 + s < L) xr0[k] = load16(a.x + row * P + 8 * po);
        if (pos0 + s + 1 < L) xr1[k] = load16(a.x + (row + a.nheads) * P + 8 * po);
      }
    }
  };

  for (int nb0 = 0; nb0 < N; nb0 += NB) {
    prefetch(h0);
    __syncthreads();  // earlier readers of sBt are done
    // B^T[n][s] for this state block, two positions per 32-bit LDS word.
    for (int task = tid; task < (NB / 8) * (Q / 2); task += NTHR) {
      const int sp = task % (Q / 2), no = task / (Q / 2);
      const int s = 2 * sp;
      const int64_t row = ((int64_t)b * L + pos0 + s) * a.ngroups + g;
      uint4 r0 = make_uint4(0, 0, 0, 0), r1 = r0;
      if (pos0 + s < L) r0 = load16(a.B + row * N + nb0 + 8 * no);
      if (pos0 + s + 1 < L) r1 = load16(a.B + (row + a.ngroups) * N + nb0 + 8 * no);
      uint32_t w[8];
      interleave_pairs(r0, r1, w);
#pragma unroll
      for (int i = 0; i < 8; ++i) *reinterpret_cast<uint32_t*>(&sBt[8 * no + i][s]) = w[i];
    }
    for (int hh = 0; hh < nh; ++hh) {
      const int h = h0 + hh;
      chunk_log_decay(a, c, h, dtb, sCs2, sDt, sTmp);
      const float cs_last = sCs2[Q - 1];
      if (tid < Q) sW[tid] = fast_exp2(cs_last - sCs2[tid]) * sDt[tid];
      if (nb0 == 0 && tid == 0)
        a.decay[((int64_t)b * a.nheads + h) * a.nchunks + c] = fast_exp2(cs_last);
      __syncthreads();
      // (w x)^T[p][s], rounded to bf16, from the prefetched rows.
#pragma unroll
      for (int k = 0; k < XPT; ++k) {
        const int task = tid + k * NTHR;
        if (task < xtasks) {
          const int sp = task % (Q / 2), po = task / (Q / 2);
          const int s = 2 * sp;
          const float w0 = sW[s], w1 = sW[s + 1];
          const uint32_t e0[4] = {xr0[k].x, xr0[k].y, xr0[k].z, xr0[k].w};
          const uint32_t e1[4] = {xr1[k].x, xr1[k].y, xr1[k].z, xr1[k].w};
#pragma unroll
          for (int i = 0; i < 8; ++i) {
            const uint32_t b0 = (i & 1) ? (e0[i / 2] >> 16) : (e0[i / 2] & 0xffffu);
            const uint32_t b1 = (i & 1) ? (e1[i / 2] >> 16) : (e1[i / 2] & 0xffffu);
            const uint32_t v0 = f32_to_bf16_bits(bf16_bits_to_f32(b0) * w0);
            const uint32_t v1 = f32_to_bf16_bits(bf16_bits_to_f32(b1) * w1);
            *reinterpret_cast<uint32_t*>(&sXt[8 * po + i][s]) = v0 | (v1 << 16);
          }
        }
      }
      __syncthreads();
      if (hh + 1 < nh) prefetch(h + 1);
      // S_c^T[n][p] = sum_s B^T[n][s] (w x)^T[p][s]
      f32x4 acc[TPW];
#pragma unroll
      for (int t = 0; t < TPW; ++t) acc[t] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
      for (int ks = 0; ks < Q / 32; ++ks) {
        const int s = ks * 32 + 8 * q4;
#pragma unroll
        for (int t = 0; t < TPW; ++t) {
          const int tile = wv + NW * t;
          if (tile < TILES) {
            const int nt = tile / PT, pt = tile % PT;
            const bf16x8 av = as_bf16x8(*reinterpret_cast<const uint4*>(&sBt[nt * 16 + r16][s]));
            const bf16x8 bv = as_bf16x8(*reinterpret_cast<const uint4*>(&sXt[pt * 16 + r16][s]));
            acc[t] = mfma_bf16(av, bv, acc[t]);
          }
        }
      }
      // lane holds S_c[p][n .. n+3] with p = pt*16 + r16, n = nt*16 + 4*q4
      uint16_t* st = a.states + (((int64_t)b * a.nchunks + c) * a.nheads + h) * P * N;
#pragma unroll
      for (int t = 0; t < TPW; ++t) {
        const int tile = wv + NW * t;
        if (tile < TILES) {
          const int nt = tile / PT, pt = tile % PT;
          const int p = pt * 16 + r16, n = nb0 + nt * 16 + 4 * q4;
          uint2 o;
          o.x = (uint32_t)f32_to_bf16_bits(acc[t][0]) | ((uint32_t)f32_to_bf16_bits(acc[t][1]) << 16);
          o.y = (uint32_t)f32_to_bf16_bits(acc[t][2]) | ((uint32_t)f32_to_bf16_bits(acc[t][3]) << 16);
          *reinterpret_cast<uint2*>(st + (int64_t)p * N + n) = o;
        }
      }
    }
  }
}

// ---- 2. state passing across chunks (the jump formula) ----------------------

__global__ void __launch_bounds__(256) ssd_state_pass_kernel(SsdArgs a) {
  const int bh = blockIdx.y;
  const int b = bh / a.nheads, h = bh % a.nheads;
  const int64_t PN = (int64_t)a.headdim * a.dstate;
  const int64_t e0 = ((int64_t)blockIdx.x * 256 + threadIdx.x) * 8;
  if (e0 >= PN) return;
  float S[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) S[i] = 0.0f;
  for (int c = 0; c < a.nchunks; ++c) {
    uint16_t* ptr = a.states + (((int64_t)b * a.nchunks + c) * a.nheads + h) * PN + e0;
    const uint4 raw = *reinterpret_cast<const uint4*>(ptr);
    uint32_t o[4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
      o[i] = (uint32_t)f32_to_bf16_bits(S[2 * i]) | ((uint32_t)f32_to_bf16_bits(S[2 * i + 1]) << 16);
    *reinterpret_cast<uint4*>(ptr) = make_uint4(o[0], o[1], o[2], o[3]);
    const float dec = a.decay[((int64_t)b * a.nheads + h) * a.nchunks + c];
    const uint32_t r[4] = {raw.x, raw.y, raw.z, raw.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      S[2 * i] = __builtin_fmaf(dec, S[2 * i], bf16_bits_to_f32(r[i] & 0xffffu));
      S[2 * i + 1] = __builtin_fmaf(dec, S[2 * i + 1], __uint_as_float(r[i] & 0xffff0000u));
    }
  }
  if (a.final_state) {
    float4* f = reinterpret_cast<float4*>(a.final_state + (int64_t)bh * PN + e0);
    f[0] = make_float4(S[0], S[1], S[2], S[3]);
    f[1] = make_float4(S[4], S[5], S[6], S[7]);
  }
}

// ---- 3. chunk output ---------------------------------------------------------

// One workgroup of 16 waves per (chunk, batch, head group); wave w owns the
// 16 output positions l = 16w .. 16w+15 of the chunk (waves past the chunk
// length only help staging) and needs the s-tiles 0..w (causality).  G^T = B C^T is built once per workgroup from B staged
// 32 states at a time and kept (bf16) in registers for all heads of the
// group; each head's x^T and carried state are staged in LDS from registers
// loaded while the previous head was computing.
template <int P, int N>
__global__ void __launch_bounds__(1024) ssd_chunk_out_kernel(SsdArgs a) {
  constexpr int KN = N / 32;         // contraction steps over the state axis
  constexpr int ST = kQMax / 16;     // most s-tiles a wave can need
  constexpr int PT = P / 16;
  constexpr int kRowN = N + 8;       // LDS row stride (bf16) of [p][n]
  constexpr int NTHR = 1024;
  constexpr int XPT = ((P / 8) * (kQMax / 2) + NTHR - 1) / NTHR;
  constexpr int SPT = (P * N / 8 + NTHR - 1) / NTHR;
  __shared__ alignas(16) uint16_t sXt[P][kRowQ];   // x^T of one head: [p][s]
  __shared__ alignas(16) uint16_t sS[P][kRowN];    // S_in of one head: [p][n]
  __shared__ alignas(16) uint16_t sBk[kQMax][40];  // 32 states of B: [s][n] (+pad)
  __shared__ float sCs2[kQMax], sDt[kQMax], sTmp[4];

  const int Q = a.chunk, L = a.seqlen;
  const int c = blockIdx.x, b = blockIdx.y;
  const int hpg = a.nheads / a.ngroups;
  const int h0 = blockIdx.z * a.heads_per_wg_out;
  const int nh = min(a.heads_per_wg_out, a.nheads - h0);
  const int g = h0 / hpg;
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int r16 = lane & 15, q4 = lane >> 4;
  const int l = 16 * wv + r16;       // this lane's output position within the chunk
  const bool active = 16 * wv < Q;   // wave owns positions inside the chunk
  const int ns = active ? wv + 1 : 0;  // s-tiles 0..wv cover every s <= l
  const int64_t pos0 = (int64_t)c * Q;
  const bool l_ok = active && pos0 + l < L;
  const int xtasks = (P / 8) * (Q / 2);

  const uint16_t* crow = a.C + (((int64_t)b * L + pos0 + (l_ok ? l : 0)) * a.ngroups + g) * N;

  // Per-head inputs held in registers one head ahead.
  uint4 xr0[XPT], xr1[XPT], sr[SPT];
  uint32_t dtb = 0;
  auto prefetch = [&](int h) {
    dtb = load_dt_bits(a, b, c, h);
#pragma unroll
    for (int k = 0; k < XPT; ++k) {
      const int task = tid + k * NTHR;
      xr0[k] = xr1[k] = make_uint4(0, 0, 0, 0);
      if (task < xtasks) {
        const int sp = task % (Q / 2), po = task / (Q / 2);
        const int s = 2 * sp;
        const int64_t row = ((int64_t)b * L + pos0 + s) * a.nheads + h;
        if (pos0 + s < L) xr0[k] = load16(a.x + row * P + 8 * po);
        if (pos0 + s + 1 < L) xr1[k] = load16(a.x + (row + a.nheads) * P + 8 * po);
      }
    }
    const uint16_t* sin = a.states + (((int64_t)b * a.nchunks + c) * a.nheads + h) * P * N;
#pragma unroll
    for (int k = 0; k < SPT; ++k) {
      const int task = tid + k * NTHR;
      sr[k] = (c > 0 && task < P * N / 8) ? load16(sin + 8 * task) : make_uint4(0, 0, 0, 0);
    }
  };
  prefetch(h0);

  // G^T[s][l] = sum_n B[s][n] C[l][n] for s-tiles 0..ns-1, B staged 32
  // states at a time.
  f32x4 gacc[ST];
#pragma unroll
  for (int st = 0; st < ST; ++st) gacc[st] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
  for (int kk = 0; kk < KN; ++kk) {
    __syncthreads();  // earlier readers of sBk are done
    for (int task = tid; task < Q * 4; task += NTHR) {
      const int s = task >> 2, part = task & 3;
      uint4 v = make_uint4(0, 0, 0, 0);
      if (pos0 + s < L)
        v = load16(a.B + (((int64_t)b * L + pos0 + s) * a.ngroups + g) * N + kk * 32 + 8 * part);
      *reinterpret_cast<uint4*>(&sBk[s][8 * part]) = v;
    }
    const bf16x8 bop =
        as_bf16x8(l_ok ? load16(crow + kk * 32 + 8 * q4) : make_uint4(0, 0, 0, 0));
    __syncthreads();
#pragma unroll
    for (int st = 0; st < ST; ++st) {
      if (st < ns) {
        const bf16x8 av = as_bf16x8(*reinterpret_cast<const uint4*>(&sBk[st * 16 + r16][8 * q4]));
        gacc[st] = mfma_bf16(av, bop, gacc[st]);
      }
    }
  }
  // Keep G^T as bf16: pair j holds tiles 2j (slots 0-3) and 2j+1 (slots 4-7).
  bf16x8 gpk[ST / 2];
#pragma unroll
  for (int j = 0; j < ST / 2; ++j)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      gpk[j][i] = static_cast<__bf16>(gacc[2 * j][i]);
      gpk[j][4 + i] = static_cast<__bf16>(gacc[2 * j + 1][i]);
    }

  for (int hh = 0; hh < nh; ++hh) {
    const int h = h0 + hh;
    // C row of this lane's position for the carried-state product (loaded
    // early; its latency overlaps the scan and the staging).
    uint4 cr[KN];
#pragma unroll
    for (int kk = 0; kk < KN; ++kk)
      cr[kk] = (l_ok && c > 0) ? load16(crow + kk * 32 + 8 * q4) : make_uint4(0, 0, 0, 0);
    chunk_log_decay(a, c, h, dtb, sCs2, sDt, sTmp);
    // stage x^T[p][s] (exact bf16) and S_in[p][n] from the prefetched registers
#pragma unroll
    for (int k = 0; k < XPT; ++k) {
      const int task = tid + k * NTHR;
      if (task < xtasks) {
        const int sp = task % (Q / 2), po = task / (Q / 2);
        uint32_t w[8];
        interleave_pairs(xr0[k], xr1[k], w);
#pragma unroll
        for (int i = 0; i < 8; ++i) *reinterpret_cast<uint32_t*>(&sXt[8 * po + i][2 * sp]) = w[i];
      }
    }
#pragma unroll
    for (int k = 0; k < SPT; ++k) {
      const int task = tid + k * NTHR;
      if (task < P * N / 8) {
        const int p = task / (N / 8), n8 = task % (N / 8);
        *reinterpret_cast<uint4*>(&sS[p][8 * n8]) = sr[k];
      }
    }
    __syncthreads();
    if (hh + 1 < nh) prefetch(h + 1);

    const float cs_l = active ? sCs2[l] : 0.0f;
    f32x4 yacc[PT];
#pragma unroll
    for (int pt = 0; pt < PT; ++pt) yacc[pt] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
    // Y^T[p][l] = sum_n S_in[p][n] exp(cs_l) C[l][n]   (S_in = 0 for chunk 0)
    if (c > 0 && active) {
      const float el = fast_exp2(cs_l);
#pragma unroll
      for (int kk = 0; kk < KN; ++kk) {
        const bf16x8 craw = as_bf16x8(cr[kk]);
        bf16x8 cop;
#pragma unroll
        for (int i = 0; i < 8; ++i) cop[i] = static_cast<__bf16>(static_cast<float>(craw[i]) * el);
#pragma unroll
        for (int pt = 0; pt < PT; ++pt) {
          const bf16x8 av =
              as_bf16x8(*reinterpret_cast<const uint4*>(&sS[pt * 16 + r16][kk * 32 + 8 * q4]));
          yacc[pt] = mfma_bf16(av, cop, yacc[pt]);
        }
      }
    }
    // Y^T[p][l] += sum_s x^T[p][s] M^T[s][l], M^T built pair by pair:
    // slot (q4, half*4 + i) of pair j holds s = 32j + 16*half + 4*q4 + i.
#pragma unroll
    for (int j = 0; j < ST / 2; ++j) {
      if (2 * j < ns) {
        bf16x8 mop;
#pragma unroll
        for (int half = 0; half < 2; ++half) {
          const int st = 2 * j + half;
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const int s = st * 16 + 4 * q4 + i;
            float v = 0.0f;
            if (st < ns && s <= l)
              v = static_cast<float>(gpk[j][half * 4 + i]) * fast_exp2(cs_l - sCs2[s]) * sDt[s];
            mop[half * 4 + i] = static_cast<__bf16>(v);
          }
        }
#pragma unroll
        for (int pt = 0; pt < PT; ++pt) {
          const uint16_t* row = &sXt[pt * 16 + r16][0];
          const uint2 lo = *reinterpret_cast<const uint2*>(row + 32 * j + 4 * q4);
          const uint2 hi = *reinterpret_cast<const uint2*>(row + 32 * j + 16 + 4 * q4);
          const bf16x8 av = as_bf16x8(make_uint4(lo.x, lo.y, hi.x, hi.y));
          yacc[pt] = mfma_bf16(av, mop, yacc[pt]);
        }
      }
    }
    // y[l][p .. p+3] = Y^T[p .. p+3][l] + D_h x[l][p .. p+3]
    if (l_ok) {
      const float Dh = a.D ? a.D[h] : 0.0f;
      uint16_t* yrow = a.y + (((int64_t)b * L + pos0 + l) * a.nheads + h) * P;
#pragma unroll
      for (int pt = 0; pt < PT; ++pt) {
        const int p = pt * 16 + 4 * q4;
        float v[4];
#pragma unroll
        for (int i = 0; i < 4; ++i)
          v[i] = __builtin_fmaf(Dh, bf16_bits_to_f32(sXt[p + i][l]), yacc[pt][i]);
        uint2 o;
        o.x = (uint32_t)f32_to_bf16_bits(v[0]) | ((uint32_t)f32_to_bf16_bits(v[1]) << 16);
        o.y = (uint32_t)f32_to_bf16_bits(v[2]) | ((uint32_t)f32_to_bf16_bits(v[3]) << 16);
        *reinterpret_cast<uint2*>(yrow + p) = o;
      }
    }
  }
}

// Largest divisor of `hpg` (heads per group) that still leaves at least
// `target` workgroups, so that a workgroup's heads share one group.
int heads_per_workgroup(int hpg, int nheads, int64_t base_wgs, int64_t target) {
  int best = 1;
  for (int d = 1; d <= hpg && d <= 8; ++d)
    if (hpg % d == 0 && base_wgs * (nheads / d) >= target) best = d;
  return best;
}

template <int P, int N>
hipError_t launch_pn(const SsdParams& p, hipStream_t stream) {
  const SsdShape& s = p.shape;
  const SsdLayout lay = ssd_layout(s);
  SsdArgs a;
  a.x = static_cast<const uint16_t*>(p.x);
  a.dt = static_cast<const uint16_t*>(p.dt);
  a.A = p.A;
  a.B = static_cast<const uint16_t*>(p.B);
  a.C = static_cast<const uint16_t*>(p.C);
  a.D = p.D;
  a.dt_bias = p.dt_bias;
  a.y = static_cast<uint16_t*>(p.y);
  a.final_state = p.final_state;
  a.states = reinterpret_cast<uint16_t*>(static_cast<char*>(p.workspace) + lay.states_off);
  a.decay = reinterpret_cast<float*>(static_cast<char*>(p.workspace) + lay.decay_off);
  a.dt_softplus = p.dt_softplus;
  a.batch = s.batch; a.seqlen = s.seqlen; a.nheads = s.nheads; a.headdim = s.headdim;
  a.dstate = s.dstate; a.ngroups = s.ngroups; a.chunk = s.chunk; a.nchunks = s.nchunks;
  const int hpg = s.nheads / s.ngroups;
  a.heads_per_wg_state = heads_per_workgroup(hpg, s.nheads, (int64_t)s.nchunks * s.batch, 256);
  a.heads_per_wg_out = heads_per_workgroup(hpg, s.nheads, (int64_t)s.nchunks * s.batch, 256);

  constexpr int NB = N > 128 ? 128 : N;
  dim3 g1(s.nchunks, s.batch, (s.nheads + a.heads_per_wg_state - 1) / a.heads_per_wg_state);
  hipLaunchKernelGGL((ssd_chunk_state_kernel<P, NB, 16>), g1, dim3(1024), 0, stream, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int64_t PN = (int64_t)P * N;
  dim3 g2((unsigned)((PN / 8 + 255) / 256), (unsigned)(s.batch * s.nheads));
  hipLaunchKernelGGL(ssd_state_pass_kernel, g2, dim3(256), 0, stream, a);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  dim3 g3(s.nchunks, s.batch, (s.nheads + a.heads_per_wg_out - 1) / a.heads_per_wg_out);
  hipLaunchKernelGGL((ssd_chunk_out_kernel<P, N>), g3, dim3(1024), 0, stream, a);
  return hipGetLastError();
}

template <int P>
hipError_t launch_p(const SsdParams& p, hipStream_t stream) {
  switch (p.shape.dstate) {
    case 32: return launch_pn<P, 32>(p, stream);
    case 64: return launch_pn<P, 64>(p, stream);
    case 128: return launch_pn<P, 128>(p, stream);
    case 256: return launch_pn<P, 256>(p, stream);
  }
  return hipErrorInvalidValue;
}

}  // namespace

hipError_t launch_ssd(const SsdParams& p, hipStream_t stream) {
  switch (p.shape.headdim) {
    case 32: return launch_p<32>(p, stream);
    case 64: return launch_p<64>(p, stream);
    case 128: return launch_p<128>(p, stream);
  }
  return hipErrorInvalidValue;
}

}  // namespace ssm
