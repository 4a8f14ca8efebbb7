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
#include <type_traits>

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
  if (headdim > 128) return bad(SSM_ERR_UNSUPPORTED, "headdim must be <= 128");
  if (dstate > 256) return bad(SSM_ERR_UNSUPPORTED, "dstate must be <= 256");
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
  out->kheaddim = headdim <= 32 ? 32 : headdim <= 64 ? 64 : 128;
  out->kdstate = dstate <= 32 ? 32 : dstate <= 64 ? 64 : dstate <= 128 ? 128 : 256;
  return SSM_OK;
}

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int kQMax = 256;          // largest chunk

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
  const float* init;  // initial state [b, h, P, N] or null (zero)
  uint16_t* states;
  float* decay;
  int dt_softplus;
  // nheads counts the heads the kernels see; with hshift = 1 a head of 128
  // channels runs as two heads of 64 (x, y and the states are the same
  // bytes), whose dt, A, D and dt_bias are those of head >> hshift of the
  // dt_heads real heads.
  int hshift, dt_heads;
  int batch, seqlen, nheads, headdim, dstate, ngroups, chunk, nchunks;
  int heads_per_wg_state, heads_per_wg_out;
  int out_halves;   // output workgroups per (chunk, batch, head group): 1 or 2
  int out_hgroups;  // head groups of the output kernel
};

__device__ __forceinline__ f32x4 mfma_bf16(const bf16x8& a, const bf16x8& b, const f32x4& c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ uint4 load16(const uint16_t* p) {
  return *reinterpret_cast<const uint4*>(p);
}

// Sequence position for a load: positions past the end read the last row
// instead.  Those rows only ever meet a weight of zero (dt = 0 past the end)
// or feed outputs that are not stored, so every load can be issued
// unconditionally; a load under a condition makes the compiler wait for it
// (and for every load issued before it) right away.
__device__ __forceinline__ int64_t load_pos(int64_t pos, int L) { return pos < L ? pos : L - 1; }

__device__ __forceinline__ bf16x8 as_bf16x8(const uint4& v) {
  return __builtin_bit_cast(bf16x8, v);
}

typedef short v4i16 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) v4i16 lds_v4i16;

// Transposed read of a row-major 16-bit LDS tile T[k][m] (ds_read_b64_tr_b16).
// Within each 16-lane group, lane L addresses row k0 + L/4, columns
// m0 + 4*(L%4) .. +3; lane j of the group then receives T[k0 .. k0+3][m0 + j]
// (checked on the device).  k0 may differ between lane groups.
__device__ __forceinline__ uint2 lds_col4(const uint16_t* tile, int stride, int k0, int m0) {
  const int L = threadIdx.x & 15;
  const uint16_t* p = tile + (k0 + (L >> 2)) * stride + m0 + 4 * (L & 3);
  const v4i16 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (lds_v4i16*)((__attribute__((address_space(3))) uint16_t*)p));
  return __builtin_bit_cast(uint2, v);
}

// MFMA operand with contraction index k over rows of a row-major LDS tile:
// lane group q gets T[kb + 8q .. kb + 8q + 7][m0 + lane%16].
__device__ __forceinline__ bf16x8 lds_kop(const uint16_t* tile, int stride, int kb, int m0) {
  const int q = (threadIdx.x & 63) >> 4;
  const uint2 lo = lds_col4(tile, stride, kb + 8 * q, m0);
  const uint2 hi = lds_col4(tile, stride, kb + 8 * q + 4, m0);
  return as_bf16x8(make_uint4(lo.x, lo.y, hi.x, hi.y));
}

constexpr int kHGMax = 8;           // most heads one workgroup handles
constexpr int kHGState = 6;         // most heads per chunk-state workgroup

template <int I, int E, class F>
__device__ __forceinline__ void static_for(F&& f) {
  if constexpr (I < E) {
    f(std::integral_constant<int, I>{});
    static_for<I + 1, E>(f);
  }
}

// Most heads per output-kernel workgroup: the largest shape keeps fewer so
// that its per-head decay tables fit in LDS beside the x and state tiles.
constexpr int out_heads_max(int P, int N) { return P * N >= 128 * 256 ? 4 : kHGMax; }

// Most heads per workgroup of the four-wave output kernel.
constexpr int kHGSmall = 6;

// Raw dt for the log-decay of every head of a workgroup's group: NTHR
// threads form NTHR/256 groups of 256; round r covers heads
// r*(NTHR/256) .. and thread t of a group owns chunk position t.  Loaded
// early so that the latency overlaps other work.
template <int NTHR>
struct GroupRaw {
  static constexpr int ROUNDS = kHGMax / (NTHR / 256);
  uint32_t dt[ROUNDS];             // raw dt (bf16 bits) of this thread's position
  float A[ROUNDS], bias[ROUNDS], D[ROUNDS];  // per-head scalars (uniform per wave)
};

template <int NTHR>
__device__ __forceinline__ void load_group_dt(const SsdArgs& a, int b, int c, int h0, int nh,
                                              GroupRaw<NTHR>& g) {
  constexpr int NGRP = NTHR / 256, ROUNDS = GroupRaw<NTHR>::ROUNDS;
  const int tid = threadIdx.x, t = tid & 255;
  const int grp = __builtin_amdgcn_readfirstlane(tid >> 8);
  const int64_t pos = (int64_t)c * a.chunk + t;
#pragma unroll
  for (int r = 0; r < ROUNDS; ++r) {
    const int hh = min(NGRP * r + grp, nh - 1);  // the consumer skips hh >= nh
    const int hr = (h0 + hh) >> a.hshift;        // the real head
    g.dt[r] = a.dt[((int64_t)b * a.seqlen + load_pos(pos, a.seqlen)) * a.dt_heads + hr];
    g.A[r] = a.A[hr];
    g.bias[r] = a.dt_bias ? a.dt_bias[hr] : 0.0f;
    g.D[r] = a.D ? a.D[hr] : 0.0f;
  }
}

// Log-decay of every head of the group for one (batch, chunk):
// sDt[hh][s] = dt after bias and softplus, sCs2[hh][s] = log2(e) * inclusive
// within-chunk cumsum of A_h dt (positions past the sequence end have
// dt = 0).
//
// With sW given, also sW[hh][t] = dt_t exp2(cs[t | 31] - cs[t]): dt times the
// decay from position t to the end of its 32-position group.  With sHead
// given, sHead[hh] = (A_h, D_h).
template <int NTHR>
__device__ void group_log_decay(const SsdArgs& a, int c, int nh, const GroupRaw<NTHR>& g,
                                float (*sCs2)[kQMax], float (*sDt)[kQMax], float* sTmp,
                                float (*sW)[kQMax] = nullptr, float2* sHead = nullptr) {
  constexpr int NGRP = NTHR / 256, ROUNDS = GroupRaw<NTHR>::ROUNDS;
  const int tid = threadIdx.x;
  const int grp = tid >> 8, t = tid & 255, lane = tid & 63, w4 = (tid >> 6) & 3;
  const int64_t pos = (int64_t)c * a.chunk + t;
#pragma unroll
  for (int r = 0; r < ROUNDS; ++r) {
    if (NGRP * r >= nh) break;
    const int hh = NGRP * r + grp;
    float dtv = 0.0f, ah = 0.0f;
    if (hh < nh) {
      ah = g.A[r] * kLog2e;
      if (t < a.chunk && pos < a.seqlen) {
        const float v = bf16_bits_to_f32(g.dt[r]) + g.bias[r];
        dtv = a.dt_softplus ? softplus_f(v) : v;
      }
      if (sHead && t == 0) sHead[hh] = make_float2(g.A[r], g.D[r]);
    }
    float v = ah * dtv;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
      const float o = __shfl_up(v, off, 64);
      if (lane >= off) v += o;
    }
    if (lane == 63) sTmp[grp * 4 + w4] = v;
    __syncthreads();
    float add = 0.0f;
    for (int w = 0; w < w4; ++w) add += sTmp[grp * 4 + w];
    const float cs = v + add;
    const float cs_end = __shfl(cs, lane | 31, 64);
    if (hh < nh) {
      sCs2[hh][t] = cs;
      sDt[hh][t] = dtv;
      if (sW) sW[hh][t] = dtv * fast_exp2(cs_end - cs);
    }
    __syncthreads();
  }
}

// ---- 1. chunk states ---------------------------------------------------------

// One 1024-thread workgroup per (chunk, batch, head group).  B of the chunk
// (one state block at a time) and each head's w*x are kept in LDS in their
// natural row-major layouts, written with coalesced 16-byte loads; the MFMA
// operands, whose contraction index runs over rows, are read back with the
// transposing LDS read.  Every global load that does not depend on earlier
// results is issued at the start, and each head's x is loaded into
// registers PD heads ahead of its use (a ring of PD + 1 register sets,
// indexed statically by unrolling the head loop by the ring size), so that
// several heads' loads are in flight while the small per-head product runs.
template <int P, int NB, int QT>
__global__ void __launch_bounds__(1024) ssd_chunk_state_kernel(SsdArgs a) {
  SSM_POISON_LDS_AT_ENTRY();
  constexpr int NTHR = 1024, NW = 16;
  // LDS row strides (bf16), in bytes 32 and 16 modulo 128 past the row
  // (B: NB + 16 elements; x: P + 8): the four rows that a 16-lane group of
  // the transposing read touches then fall on disjoint bank groups of B and
  // x; rows stay 16-byte aligned for the staging stores.  With the decay
  // tables of at most kHGState heads the x tile stays double-buffered within
  // 156 KB at P = 64, NB = 128, Q = 256.
  constexpr int kRowB = NB + 16;
  constexpr int kRowX = P + 8;
  constexpr bool DB = (size_t)QT * (kRowB + 2 * kRowX) * 2 + 2 * kHGState * kQMax * 4 <= 156 * 1024;
  constexpr int NBUF = DB ? 2 : 1;
  __shared__ alignas(16) uint16_t sB[QT][kRowB];         // B[s][n] of one state block
  __shared__ alignas(16) uint16_t sX[NBUF][QT][kRowX];   // (w x)[s][p] of one head
  __shared__ alignas(16) float sCs2[kHGState][kQMax];
  __shared__ alignas(16) float sDt[kHGState][kQMax];
  __shared__ float sTmp[16];
  constexpr int NT = NB / 16, PT = P / 16, TILES = NT * PT, TPW = (TILES + NW - 1) / NW;
  constexpr bool kAllTiles = TILES % NW == 0;  // every wave owns TPW tiles
  // a wave's tiles come in pairs on the same rows p (16-byte state stores)
  constexpr bool kPairStores = kAllTiles && TPW % 2 == 0 && NW % PT == 0;
  constexpr int XTASKS = QT * P / 8, BTASKS = QT * NB / 8;
  constexpr int XPT = (XTASKS + NTHR - 1) / NTHR;
  constexpr int BPT = (BTASKS + NTHR - 1) / NTHR;
  constexpr int PD = XPT <= 2 ? 2 : 1;  // heads of x in flight
  constexpr int RING = PD + 1;

  const int c = blockIdx.x, b = blockIdx.y;
  const int hpg = a.nheads / a.ngroups;
  const int h0 = blockIdx.z * a.heads_per_wg_state;
  const int nh = min(a.heads_per_wg_state, a.nheads - h0);
  const int g = h0 / hpg;
  const int N = a.dstate, L = a.seqlen;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave index (uniform)
  const int r16 = lane & 15, q4 = lane >> 4;
  const int64_t pos0 = (int64_t)c * QT;

  // Every global load is issued unconditionally (clamped task, position and
  // head indices): a load under a condition, or a loop whose memory
  // operations depend on a runtime count, makes the compiler wait for every
  // load in flight instead of the one it needs.
  uint4 xr[RING][XPT], br[BPT];
  const uint16_t* xsrc[XPT];  // this thread's x pieces of the group's first head
#pragma unroll
  for (int k = 0; k < XPT; ++k) {
    const int task = min(tid + k * NTHR, XTASKS - 1);
    const int s = task / (P / 8), po = task % (P / 8);
    xsrc[k] = a.x + (((int64_t)b * L + load_pos(pos0 + s, L)) * a.nheads + h0) * P + 8 * po;
  }
  // x of head hh (clamped to the group) into ring slot SLOT
  auto prefetch = [&](auto slot, int hh) {
    constexpr int SLOT = decltype(slot)::value;
    const int64_t off = (int64_t)min(hh, nh - 1) * P;
#pragma unroll
    for (int k = 0; k < XPT; ++k) xr[SLOT][k] = load16(xsrc[k] + off);
  };
  auto prefetch_first = [&]() {
    static_for<0, PD>([&](auto jc) { prefetch(jc, decltype(jc)::value); });
  };
  auto load_b = [&](int nb0) {
#pragma unroll
    for (int k = 0; k < BPT; ++k) {
      const int task = min(tid + k * NTHR, BTASKS - 1);
      const int s = task / (NB / 8), part = task % (NB / 8);
      br[k] = load16(a.B + (((int64_t)b * L + load_pos(pos0 + s, L)) * a.ngroups + g) * N + nb0 +
                     8 * part);
    }
  };
  // (w x)[s][p] = x[s][p] exp2(cs_last - cs_s) dt_s, rounded to bf16.
  auto stage = [&](auto slot, int hh, int buf) {
    constexpr int SLOT = decltype(slot)::value;
    const float cs_last = sCs2[hh][QT - 1];
#pragma unroll
    for (int k = 0; k < XPT; ++k) {
      const int task = tid + k * NTHR;
      if (XTASKS % NTHR == 0 || task < XTASKS) {
        const int s = task / (P / 8), po = task % (P / 8);
        const float w = fast_exp2(cs_last - sCs2[hh][s]) * sDt[hh][s];
        const uint32_t e[4] = {xr[SLOT][k].x, xr[SLOT][k].y, xr[SLOT][k].z, xr[SLOT][k].w};
        uint32_t o[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          o[i] = pack_bf16x2(bf16_bits_to_f32(e[i] & 0xffffu) * w,
                             __uint_as_float(e[i] & 0xffff0000u) * w);
        }
        *reinterpret_cast<uint4*>(&sX[buf][s][8 * po]) = make_uint4(o[0], o[1], o[2], o[3]);
      }
    }
  };

  GroupRaw<NTHR> graw;
  load_group_dt<NTHR>(a, b, c, h0, nh, graw);
  load_b(0);
  prefetch_first();
  group_log_decay<NTHR>(a, c, nh, graw, sCs2, sDt, sTmp);
  if (tid < nh)
    a.decay[((int64_t)b * a.nheads + h0 + tid) * a.nchunks + c] = fast_exp2(sCs2[tid][QT - 1]);

  for (int nb0 = 0; nb0 < N; nb0 += NB) {
    if (nb0 > 0) {
      load_b(nb0);
      prefetch_first();
      __syncthreads();  // earlier readers of sB and sX are done
    }
#pragma unroll
    for (int k = 0; k < BPT; ++k) {
      const int task = tid + k * NTHR;
      if (BTASKS % NTHR == 0 || task < BTASKS) {
        const int s = task / (NB / 8), part = task % (NB / 8);
        *reinterpret_cast<uint4*>(&sB[s][8 * part]) = br[k];
      }
    }
    // one head: stage its (w x), prefetch the head PD ahead, S_c^T = B^T (w x)
    auto head = [&](auto jc, int hh) {
      constexpr int J = decltype(jc)::value;
      const int h = h0 + hh;
      const int buf = DB ? (hh & 1) : 0;
      // a single buffer's previous readers are done (the barrier after the
      // last head's product); two buffers alternate
      stage(jc, hh, buf);
      prefetch(std::integral_constant<int, (J + PD) % RING>{}, hh + PD);
      __syncthreads();
      // S_c^T[n][p] = sum_s B[s][n] (w x)[s][p]
      f32x4 acc[TPW];
#pragma unroll
      for (int t = 0; t < TPW; ++t) acc[t] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll 2
      for (int ks = 0; ks < QT / 32; ++ks) {
#pragma unroll
        for (int t = 0; t < TPW; ++t) {
          const int tile = wv + NW * t;
          if (kAllTiles || tile < TILES) {
            const int nt = tile / PT, pt = tile % PT;
            const bf16x8 av = lds_kop(&sB[0][0], kRowB, ks * 32, nt * 16);
            const bf16x8 bv = lds_kop(&sX[buf][0][0], kRowX, ks * 32, pt * 16);
            acc[t] = mfma_bf16(av, bv, acc[t]);
          }
        }
      }
      if constexpr (!DB) __syncthreads();  // readers of the single sX buffer are done
      // lane holds S_c[p][n .. n+3] with p = pt*16 + r16, n = nt*16 + 4*q4
      uint16_t* st = a.states + (((int64_t)b * a.nchunks + c) * a.nheads + h) * P * N;
      if constexpr (kPairStores) {
        // a wave's tiles t = 2j, 2j+1 share their rows p: swapping with the
        // lane 16 apart (v_permlane16_swap) gives every lane eight
        // consecutive n of one of them, stored as 16 bytes
#pragma unroll
        for (int j = 0; j < TPW / 2; ++j) {
          uint2 o[2];
#pragma unroll
          for (int u = 0; u < 2; ++u) {
            o[u].x = pack_bf16x2(acc[2 * j + u][0], acc[2 * j + u][1]);
            o[u].y = pack_bf16x2(acc[2 * j + u][2], acc[2 * j + u][3]);
          }
          const auto lo = __builtin_amdgcn_permlane16_swap(o[0].x, o[1].x, false, false);
          const auto hi = __builtin_amdgcn_permlane16_swap(o[0].y, o[1].y, false, false);
          const int tile = wv + NW * (2 * j + (q4 & 1));
          const int nt = tile / PT, pt = tile % PT;
          const int p = pt * 16 + r16, n = nb0 + nt * 16 + 8 * (q4 >> 1);
          *reinterpret_cast<uint4*>(st + (int64_t)p * N + n) = make_uint4(lo[0], hi[0], lo[1], hi[1]);
        }
      } else {
#pragma unroll
        for (int t = 0; t < TPW; ++t) {
          const int tile = wv + NW * t;
          if (kAllTiles || tile < TILES) {
            const int nt = tile / PT, pt = tile % PT;
            const int p = pt * 16 + r16, n = nb0 + nt * 16 + 4 * q4;
            uint2 o;
            o.x = pack_bf16x2(acc[t][0], acc[t][1]);
            o.y = pack_bf16x2(acc[t][2], acc[t][3]);
            *reinterpret_cast<uint2*>(st + (int64_t)p * N + n) = o;
          }
        }
      }
    };
    int hb = 0;
    for (; hb + RING <= nh; hb += RING)
      static_for<0, RING>([&](auto jc) { head(jc, hb + decltype(jc)::value); });
    static_for<0, RING>([&](auto jc) {
      if (hb + decltype(jc)::value < nh) head(jc, hb + decltype(jc)::value);
    });
    if constexpr (DB) __syncthreads();  // readers of sX and sB are done
  }
}

// ---- 2. state passing across chunks (the jump formula) ----------------------

// The chunk states of one thread's 8 entries and the chunk decays are
// loaded RING chunks ahead of their use (clamped chunk index, no condition
// on the loads), so that the latencies of the loads overlap instead of
// adding up chunk after chunk.
__global__ void __launch_bounds__(256) ssd_state_pass_kernel(SsdArgs a) {
  constexpr int RING = 8;
  const int64_t bh = blockIdx.x;
  const int b = (int)(bh / a.nheads), h = (int)(bh % a.nheads);
  const int64_t PN = (int64_t)a.headdim * a.dstate;
  const int64_t e0 = ((int64_t)blockIdx.y * 256 + threadIdx.x) * 8;
  if (e0 >= PN) return;
  // the state entering the sequence: the given initial state, else zero
  float S[8];
  if (a.init) {
    const float4* s0 = reinterpret_cast<const float4*>(a.init + bh * PN + e0);
    const float4 lo = s0[0], hi = s0[1];
    S[0] = lo.x; S[1] = lo.y; S[2] = lo.z; S[3] = lo.w;
    S[4] = hi.x; S[5] = hi.y; S[6] = hi.z; S[7] = hi.w;
  } else {
#pragma unroll
    for (int i = 0; i < 8; ++i) S[i] = 0.0f;
  }
  const int nc = a.nchunks;
  const int64_t cstride = (int64_t)a.nheads * PN;  // elements between chunks
  uint16_t* base = a.states + ((int64_t)b * nc * a.nheads + h) * PN + e0;
  const float* dec = a.decay + bh * nc;
  uint4 raw[RING];
  float dv[RING];
#pragma unroll
  for (int i = 0; i < RING; ++i) {
    const int c = min(i, nc - 1);
    raw[i] = *reinterpret_cast<const uint4*>(base + c * cstride);
    dv[i] = dec[c];
  }
  for (int c0 = 0; c0 < nc; c0 += RING) {
#pragma unroll
    for (int i = 0; i < RING; ++i) {
      // Chunks past the end (the last ring's tail) are identity steps whose
      // store is skipped; the loads stay unconditional.
      const int c = c0 + i;
      const bool live = c < nc;
      const uint4 r = raw[i];
      const float d = live ? dv[i] : 1.0f;
      // refill this ring slot with chunk c + RING (this thread writes that
      // chunk's entry only later, after this read)
      const int cn = min(c + RING, nc - 1);
      raw[i] = *reinterpret_cast<const uint4*>(base + cn * cstride);
      dv[i] = dec[cn];
      uint32_t o[4];
#pragma unroll
      for (int k = 0; k < 4; ++k) o[k] = pack_bf16x2(S[2 * k], S[2 * k + 1]);
      if (live) *reinterpret_cast<uint4*>(base + c * cstride) = make_uint4(o[0], o[1], o[2], o[3]);
      const uint32_t rw[4] = {live ? r.x : 0u, live ? r.y : 0u, live ? r.z : 0u, live ? r.w : 0u};
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        S[2 * k] = __builtin_fmaf(d, S[2 * k], bf16_bits_to_f32(rw[k] & 0xffffu));
        S[2 * k + 1] = __builtin_fmaf(d, S[2 * k + 1], __uint_as_float(rw[k] & 0xffff0000u));
      }
    }
  }
  if (a.final_state) {
    float4* f = reinterpret_cast<float4*>(a.final_state + bh * PN + e0);
    f[0] = make_float4(S[0], S[1], S[2], S[3]);
    f[1] = make_float4(S[4], S[5], S[6], S[7]);
  }
}

// ---- 3. chunk output ---------------------------------------------------------

// One 512-thread workgroup (8 waves) per (chunk, batch, head group).  The
// chunk's 16-position output tiles are paired so every wave does the same
// causal work: wave w owns tiles A = w and B = Q/16-1-w and needs s-tiles
// 0..A for A and 0..B for B, which pack into exactly Q/32 + 1 pairs of
// s-tiles (9 for Q = 256).  G^T = B C^T for those pairs is built once per
// workgroup (B staged up to 128 states at a time) and kept as bf16 in
// registers for every head of the group.  The log-decays of all heads are
// computed up front; each head's x^T and carried state are staged from
// registers loaded while the previous head computed, into one of two LDS
// buffers when both fit, so a head costs one barrier.  The carried-state
// product uses C as loaded and is scaled by exp(cs_l) once per column.
//
// W = 4 (the shapes whose tiles fit twice in a CU's LDS): the same work with
// four-wave workgroups, two per (chunk, batch, head group) at Q = 256, each
// taking half of the chunk's output-tile pairs (workgroup ids i and i + 8 of
// each block of 16, so both halves run on one XCD and share its L2).  One
// head buffer and up to 64 states of B per staging round keep a workgroup
// within half of the LDS, so two workgroups share a CU and one stages or
// stores while the other computes.
template <int W>
constexpr int out_kb(int N) { return W == 8 ? (N < 128 ? N : 128) : (N < 64 ? N : 64); }

template <int P, int N, int W>
__global__ void __launch_bounds__(64 * W, 8 / W) ssd_chunk_out_kernel(SsdArgs a) {
  SSM_POISON_LDS_AT_ENTRY();
  constexpr int KN = N / 32;         // contraction steps over the state axis
  constexpr int NPN = kQMax / 32 - 1; // off-diagonal s-tile pairs per wave (at Q = 256)
  constexpr int PT = P / 16;
  constexpr int KB = out_kb<W>(N);   // states of B per staging round
  constexpr int kRowB = KB + 8;
  constexpr int kRowN = N + 8;       // LDS row stride (bf16) of [p][n]
  constexpr int NTHR = 64 * W;
  constexpr int kRowX = P + 16;      // LDS row stride (bf16) of x [s][p]
  constexpr int XPT = (kQMax * P / 8 + NTHR - 1) / NTHR;
  constexpr int SPT = (P * N / 8 + NTHR - 1) / NTHR;
  constexpr int BPT = (kQMax * KB / 8 + NTHR - 1) / NTHR;
  // Staging tasks that cover their tile exactly need no per-thread condition
  // (rows past the chunk are written but never read).
  constexpr bool kXExact = kQMax * P / 8 == XPT * NTHR;
  constexpr bool kSExact = P * N / 8 == SPT * NTHR;
  constexpr bool kBExact = kQMax * KB / 8 == BPT * NTHR;
  // LDS: x [s][p] and S_in [p][n] of one head (two buffers when they fit);
  // B [s][n] for the G^T phase shares the same bytes (it is only used before
  // the first head is staged).
  constexpr size_t kXtBytes = (size_t)kQMax * kRowX * 2;
  constexpr size_t kSBytes = (size_t)P * kRowN * 2;
  constexpr size_t kBBytes = (size_t)kQMax * kRowB * 2;
  constexpr int HG = W == 8 ? out_heads_max(P, N) : kHGSmall;  // most heads per workgroup
  constexpr size_t kFixed = 3 * HG * kQMax * 4 + 64;
  constexpr bool DB = W == 8 && 2 * (kXtBytes + kSBytes) + kFixed <= 156 * 1024;
  constexpr int NBUF = DB ? 2 : 1;
  constexpr size_t kBufBytes = NBUF * (kXtBytes + kSBytes);
  constexpr size_t kRawBytes = kBufBytes > kBBytes ? kBufBytes : kBBytes;
  __shared__ alignas(16) uint8_t sRaw[kRawBytes];
  __shared__ alignas(16) float sCs2[HG][kQMax];
  __shared__ alignas(16) float sDt[HG][kQMax];
  __shared__ alignas(16) float sW[HG][kQMax];
  __shared__ float2 sHead[HG];
  __shared__ float sTmp[16];
  auto sX = reinterpret_cast<uint16_t (*)[kQMax][kRowX]>(sRaw);
  auto sS = reinterpret_cast<uint16_t (*)[P][kRowN]>(sRaw + NBUF * kXtBytes);
  auto sBs = reinterpret_cast<uint16_t (*)[kRowB]>(sRaw);

  const int Q = a.chunk, L = a.seqlen;
  int c, b, zg, half;
  if constexpr (W == 8) {
    c = blockIdx.x;
    b = blockIdx.y;
    zg = blockIdx.z;
    half = 0;
  } else {
    // one-dimensional grid: (pair of halves) -> (chunk, batch, head group)
    const int id = blockIdx.x;
    int pr;
    if (a.out_halves == 2) {
      pr = (id / 16) * 8 + id % 8;
      half = (id / 8) % 2;
    } else {
      pr = id;
      half = 0;
    }
    if (pr >= a.nchunks * a.batch * a.out_hgroups) return;  // (uniform per workgroup)
    c = pr % a.nchunks;
    b = (pr / a.nchunks) % a.batch;
    zg = pr / (a.nchunks * a.batch);
  }
  const int hpg = a.nheads / a.ngroups;
  const int h0 = zg * a.heads_per_wg_out;
  const int nh = min(a.heads_per_wg_out, a.nheads - h0);
  const int g = h0 / hpg;
  const int tid = threadIdx.x, lane = tid & 63;
  // index of this wave's pair of output tiles within the chunk (uniform)
  const int wv = __builtin_amdgcn_readfirstlane(tid >> 6) + W * half;
  const int r16 = lane & 15, q4 = lane >> 4;
  const int nlt = Q / 16;                    // output tiles in the chunk
  const bool active = wv < nlt / 2;
  const int ltile[2] = {wv, nlt - 1 - wv};   // this wave's two output tiles
  const int npA = (wv + 2) / 2;              // s-tile pairs of tile A (ceil((A+1)/2))
  const int npB = (nlt - wv + 1) / 2;        // s-tile pairs of tile B
  const int64_t pos0 = (int64_t)c * Q;
  const int lcol[2] = {16 * ltile[0] + r16, 16 * ltile[1] + r16};  // this lane's positions
  const bool lok[2] = {active && pos0 + lcol[0] < L, active && pos0 + lcol[1] < L};
  const int xtasks = Q * P / 8;
  const int btasks = Q * KB / 8;

  uint4 xr[XPT], sr[SPT], br[BPT], cr[2][KN];
  auto prefetch = [&](int hh) {
    const int h = h0 + hh;
#pragma unroll
    for (int k = 0; k < XPT; ++k) {
      const int task = tid + k * NTHR;
      const int s = task / (P / 8), po = task % (P / 8);
      xr[k] = load16(a.x + (((int64_t)b * L + load_pos(pos0 + s, L)) * a.nheads + h) * P + 8 * po);
    }
    const uint16_t* sin = a.states + (((int64_t)b * a.nchunks + c) * a.nheads + h) * P * N;
#pragma unroll
    for (int k = 0; k < SPT; ++k) {
      const int task = tid + k * NTHR;
      sr[k] = load16(sin + 8 * min(task, P * N / 8 - 1));  // unused for chunk 0 from zero
    }
  };
  // B[s][kb0 .. kb0+KB) rows, 16 bytes per task.
  auto load_b = [&](int kb0) {
#pragma unroll
    for (int k = 0; k < BPT; ++k) {
      const int task = tid + k * NTHR;
      const int s = task / (KB / 8), part = task % (KB / 8);
      br[k] = load16(a.B + (((int64_t)b * L + load_pos(pos0 + s, L)) * a.ngroups + g) * N + kb0 +
                     8 * part);
    }
  };
  // x[s][p] and S_in[p][n] from the prefetched registers.
  auto stage = [&](int buf) {
#pragma unroll
    for (int k = 0; k < XPT; ++k) {
      const int task = tid + k * NTHR;
      if (kXExact || task < xtasks) {
        const int s = task / (P / 8), po = task % (P / 8);
        *reinterpret_cast<uint4*>(&sX[buf][s][8 * po]) = xr[k];
      }
    }
#pragma unroll
    for (int k = 0; k < SPT; ++k) {
      const int task = tid + k * NTHR;
      if (kSExact || task < P * N / 8) {
        const int p = task / (N / 8), n8 = task % (N / 8);
        *reinterpret_cast<uint4*>(&sS[buf][p][8 * n8]) = sr[k];
      }
    }
  };

  // Issue the independent loads: dt and the head scalars first (their wait
  // covers nothing else), then C rows of this lane's two positions, B, and
  // the first head's x and carried state.
  GroupRaw<NTHR> graw;
  load_group_dt<NTHR>(a, b, c, h0, nh, graw);
#pragma unroll
  for (int t = 0; t < 2; ++t) {
    const uint16_t* crow =
        a.C + (((int64_t)b * L + pos0 + (lok[t] ? lcol[t] : 0)) * a.ngroups + g) * N;
#pragma unroll
    for (int kk = 0; kk < KN; ++kk)
      cr[t][kk] = load16(crow + kk * 32 + 8 * q4);  // rows past the end feed unstored columns
  }
  load_b(0);
  // (the four-wave kernel loads each head right before staging it: its
  // second workgroup on the CU covers the latency)
  if constexpr (W == 8) prefetch(0);
  group_log_decay<NTHR>(a, c, nh, graw, sCs2, sDt, sTmp, sW, sHead);

  // Pairs of s-tiles: the last pair of each output tile touches its diagonal
  // and has its own registers; of the others, tile A takes slots 0 .. npA-2
  // (s-tiles 2p, 2p+1) and tile B slots NPN-1-j for j < npB-1 (s-tiles 2j,
  // 2j+1).  npA + npB <= NPN + 2 keeps the two ranges apart, so every
  // register index below is static.  s-tiles past the diagonal are zero.
  const int ltA = ltile[0], ltB = ltile[1];

  // G^T[s][l] = sum_n B[s][n] C[l][n] for this wave's pairs.
  f32x4 gacc[2 * NPN], gdacc[4];
#pragma unroll
  for (int k = 0; k < 2 * NPN; ++k) gacc[k] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
  for (int k = 0; k < 4; ++k) gdacc[k] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
  auto gt_pair = [&](f32x4& g0, f32x4& g1, int st0, int lt, const uint4 (&cv)[KN], int kb0) {
#pragma unroll
    for (int half = 0; half < 2; ++half) {
      const int st = st0 + half;
      if (st > lt) continue;
      f32x4& acc = half ? g1 : g0;
#pragma unroll
      for (int kq = 0; kq < KB / 32; ++kq) {
        const bf16x8 av =
            as_bf16x8(*reinterpret_cast<const uint4*>(&sBs[st * 16 + r16][kq * 32 + 8 * q4]));
        acc = mfma_bf16(av, as_bf16x8(cv[kb0 / 32 + kq]), acc);
      }
    }
  };
  for (int kb0 = 0; kb0 < N; kb0 += KB) {
    if (kb0 > 0) __syncthreads();  // earlier readers of sBs are done
#pragma unroll
    for (int k = 0; k < BPT; ++k) {
      const int task = tid + k * NTHR;
      if (kBExact || task < btasks) {
        const int s = task / (KB / 8), part = task % (KB / 8);
        *reinterpret_cast<uint4*>(&sBs[s][8 * part]) = br[k];
      }
    }
    __syncthreads();
    if (kb0 + KB < N) load_b(kb0 + KB);
    if (active) {
#pragma unroll
      for (int p = 0; p < NPN; ++p)
        if (p < npA - 1) gt_pair(gacc[2 * p], gacc[2 * p + 1], 2 * p, ltA, cr[0], kb0);
#pragma unroll
      for (int j = 0; j < NPN; ++j)
        if (j < npB - 1)
          gt_pair(gacc[2 * (NPN - 1 - j)], gacc[2 * (NPN - 1 - j) + 1], 2 * j, ltB, cr[1], kb0);
      gt_pair(gdacc[0], gdacc[1], 2 * (npA - 1), ltA, cr[0], kb0);
      gt_pair(gdacc[2], gdacc[3], 2 * (npB - 1), ltB, cr[1], kb0);
    }
  }
  // Keep G^T as bf16: a pair holds s-tiles st0 (slots 0-3) and st0+1 (slots 4-7).
  auto pack_pair = [](const f32x4& lo, const f32x4& hi) {
    return as_bf16x8(make_uint4(pack_bf16x2(lo[0], lo[1]), pack_bf16x2(lo[2], lo[3]),
                                pack_bf16x2(hi[0], hi[1]), pack_bf16x2(hi[2], hi[3])));
  };
  bf16x8 gpk[NPN], gdk[2];
#pragma unroll
  for (int p = 0; p < NPN; ++p) gpk[p] = pack_pair(gacc[2 * p], gacc[2 * p + 1]);
#pragma unroll
  for (int t = 0; t < 2; ++t) gdk[t] = pack_pair(gdacc[2 * t], gdacc[2 * t + 1]);

  __syncthreads();  // readers of sBs are done before the head buffers reuse its bytes
  if constexpr (W == 8) {
    stage(0);
    if (nh > 1) prefetch(1);
  } else {
    prefetch(0);
    stage(0);
  }
  __syncthreads();

  for (int hh = 0; hh < nh; ++hh) {
    const int h = h0 + hh;
    const int buf = DB ? (hh & 1) : 0;
    const float csl[2] = {active ? sCs2[hh][lcol[0]] : 0.0f, active ? sCs2[hh][lcol[1]] : 0.0f};
    // the decay never grows within the chunk: dt >= 0 (softplus) and A_h <= 0
    const bool fact = a.dt_softplus && sHead[hh].x <= 0.0f;
    f32x4 yacc[2][PT];
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
      for (int pt = 0; pt < PT; ++pt) yacc[t][pt] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
    // Y^T[p][l] = exp(cs_l) sum_n S_in[p][n] C[l][n]   (chunk 0: the initial state, or 0)
    if ((c > 0 || a.init) && active) {
#pragma unroll
      for (int kk = 0; kk < KN; ++kk) {
#pragma unroll
        for (int pt = 0; pt < PT; ++pt) {
          const bf16x8 av =
              as_bf16x8(*reinterpret_cast<const uint4*>(&sS[buf][pt * 16 + r16][kk * 32 + 8 * q4]));
          yacc[0][pt] = mfma_bf16(av, as_bf16x8(cr[0][kk]), yacc[0][pt]);
          yacc[1][pt] = mfma_bf16(av, as_bf16x8(cr[1][kk]), yacc[1][pt]);
        }
      }
#pragma unroll
      for (int t = 0; t < 2; ++t) {
        const float el = fast_exp2(csl[t]);
#pragma unroll
        for (int pt = 0; pt < PT; ++pt) yacc[t][pt] *= el;
      }
    }
    // Y^T[p][l] += sum_s x[s][p] M^T[s][l], M^T[s][l] = G^T[s][l] dt_s
    // exp2(cs_l - cs_s) built pair by pair: slot (q4, half*4 + i) of a pair
    // holds s = 16*(st0 + half) + 4*q4 + i.
    auto pair_mma = [&](const bf16x8& mop, int st0, f32x4 (&acc)[PT]) {
#pragma unroll
      for (int pt = 0; pt < PT; ++pt) {
        // x[16 st0 + 4 q4 + i][16 pt + r16] and x[16 st0 + 16 + 4 q4 + i][...]
        const uint2 lo = lds_col4(&sX[buf][0][0], kRowX, 16 * st0 + 4 * q4, pt * 16);
        const uint2 hi = lds_col4(&sX[buf][0][0], kRowX, 16 * st0 + 16 + 4 * q4, pt * 16);
        acc[pt] = mfma_bf16(as_bf16x8(make_uint4(lo.x, lo.y, hi.x, hi.y)), mop, acc[pt]);
      }
    };
    // Direct form, with the causal mask s <= l when the pair reaches the
    // diagonal.
    auto pair_direct = [&](const bf16x8& g, int st0, int l, float cs_l, bool mask,
                           f32x4 (&acc)[PT]) {
      uint32_t mw[4];  // M^T elements as bf16 pairs
#pragma unroll
      for (int half = 0; half < 2; ++half) {
        const int s0 = (st0 + half) * 16 + 4 * q4;
        const float4 cs4 = *reinterpret_cast<const float4*>(&sCs2[hh][s0 & (kQMax - 1)]);
        const float4 dt4 = *reinterpret_cast<const float4*>(&sDt[hh][s0 & (kQMax - 1)]);
        const float csv[4] = {cs4.x, cs4.y, cs4.z, cs4.w};
        const float dtv[4] = {dt4.x, dt4.y, dt4.z, dt4.w};
        float v[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          v[i] = static_cast<float>(g[half * 4 + i]) * fast_exp2(cs_l - csv[i]) * dtv[i];
          if (mask && s0 + i > l) v[i] = 0.0f;
        }
        mw[2 * half] = pack_bf16x2(v[0], v[1]);
        mw[2 * half + 1] = pack_bf16x2(v[2], v[3]);
      }
      pair_mma(as_bf16x8(make_uint4(mw[0], mw[1], mw[2], mw[3])), st0, acc);
    };
    // Factored form for a pair wholly before the output tile when the decay
    // never grows (cs non-increasing): exp2(cs_l - cs_s) = exp2(cs_l - R)
    // exp2(R - cs_s) with R = cs at the pair's last position, both factors
    // in [0, 1]; dt_s exp2(R - cs_s) is sW.
    auto pair_fact = [&](const bf16x8& g, int st0, float cs_l, f32x4 (&acc)[PT]) {
      const float f = fast_exp2(cs_l - sCs2[hh][(16 * st0 + 31) & (kQMax - 1)]);
      uint32_t mw[4];  // M^T elements as bf16 pairs
#pragma unroll
      for (int half = 0; half < 2; ++half) {
        const int s0 = (st0 + half) * 16 + 4 * q4;
        const float4 w4 = *reinterpret_cast<const float4*>(&sW[hh][s0 & (kQMax - 1)]);
        const float wv4[4] = {w4.x, w4.y, w4.z, w4.w};
        float v[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) v[i] = static_cast<float>(g[half * 4 + i]) * (wv4[i] * f);
        mw[2 * half] = pack_bf16x2(v[0], v[1]);
        mw[2 * half + 1] = pack_bf16x2(v[2], v[3]);
      }
      pair_mma(as_bf16x8(make_uint4(mw[0], mw[1], mw[2], mw[3])), st0, acc);
    };
    if (active) {
      if (fact) {
#pragma unroll
        for (int p = 0; p < NPN; ++p)
          if (p < npA - 1) pair_fact(gpk[p], 2 * p, csl[0], yacc[0]);
#pragma unroll
        for (int j = 0; j < NPN; ++j)
          if (j < npB - 1) pair_fact(gpk[NPN - 1 - j], 2 * j, csl[1], yacc[1]);
      } else {
#pragma unroll
        for (int p = 0; p < NPN; ++p)
          if (p < npA - 1) pair_direct(gpk[p], 2 * p, lcol[0], csl[0], false, yacc[0]);
#pragma unroll
        for (int j = 0; j < NPN; ++j)
          if (j < npB - 1) pair_direct(gpk[NPN - 1 - j], 2 * j, lcol[1], csl[1], false, yacc[1]);
      }
      pair_direct(gdk[0], 2 * (npA - 1), lcol[0], csl[0], true, yacc[0]);
      pair_direct(gdk[1], 2 * (npB - 1), lcol[1], csl[1], true, yacc[1]);
    }
    // y[l][p .. p+3] = Y^T[p .. p+3][l] + D_h x[l][p .. p+3]
    const float Dh = sHead[hh].y;
    uint2 yo[2][PT];
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      const int l = lcol[t] & (kQMax - 1);
#pragma unroll
      for (int pt = 0; pt < PT; ++pt) {
        const int p = pt * 16 + 4 * q4;
        const uint2 xv = *reinterpret_cast<const uint2*>(&sX[buf][l][p]);
        const float xs[4] = {bf16_bits_to_f32(xv.x & 0xffffu), __uint_as_float(xv.x & 0xffff0000u),
                             bf16_bits_to_f32(xv.y & 0xffffu), __uint_as_float(xv.y & 0xffff0000u)};
        float v[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) v[i] = __builtin_fmaf(Dh, xs[i], yacc[t][pt][i]);
        yo[t][pt].x = pack_bf16x2(v[0], v[1]);
        yo[t][pt].y = pack_bf16x2(v[2], v[3]);
      }
    }
    // A lane holds four consecutive p of every 16-wide block of its
    // position's row; swapping with the lane 16 apart (v_permlane16_swap:
    // odd 16-lane rows of the first operand with even rows of the second)
    // gives it runs of eight, so a row is written in 16-byte pieces: for the
    // block pair (2j, 2j+1) the lane ends with p = 32j + 16 (q4 & 1) +
    // 8 (q4 >> 1) .. +7.
    auto store_y = [&]() {
#pragma unroll
      for (int t = 0; t < 2; ++t) {
        uint4 run[PT / 2];
#pragma unroll
        for (int j = 0; j < PT / 2; ++j) {
          const auto lo = __builtin_amdgcn_permlane16_swap(yo[t][2 * j].x, yo[t][2 * j + 1].x,
                                                          false, false);
          const auto hi = __builtin_amdgcn_permlane16_swap(yo[t][2 * j].y, yo[t][2 * j + 1].y,
                                                          false, false);
          run[j] = make_uint4(lo[0], hi[0], lo[1], hi[1]);
        }
        if (!lok[t]) continue;
        uint16_t* yrow = a.y + (((int64_t)b * L + pos0 + lcol[t]) * a.nheads + h) * P +
                         16 * (q4 & 1) + 8 * (q4 >> 1);
#pragma unroll
        for (int j = 0; j < PT / 2; ++j) *reinterpret_cast<uint4*>(yrow + 32 * j) = run[j];
      }
    };
    // Stage the next head before storing this one, and keep stage, stores
    // and the next prefetch on one path: waiting for the staged loads then
    // never waits for these stores.
    if (hh + 1 < nh) {
      if constexpr (W == 8) {
        if (!DB) __syncthreads();  // readers of the single buffer are done
        stage(DB ? ((hh + 1) & 1) : 0);
        store_y();
        if (hh + 2 < nh) prefetch(hh + 2);
      } else {
        prefetch(hh + 1);
        store_y();
        __syncthreads();  // readers of the single buffer are done
        stage(0);
      }
      __syncthreads();
    } else {
      store_y();
    }
  }
}

// Largest divisor of `hpg` (heads per group) that still leaves at least
// `target` workgroups, so that a workgroup's heads share one group.
int heads_per_workgroup(int hpg, int nheads, int64_t base_wgs, int64_t target, int dmax) {
  int best = 1;
  for (int d = 1; d <= hpg && d <= dmax; ++d)
    if (hpg % d == 0 && base_wgs * (nheads / d) >= target) best = d;
  return best;
}

// The four-wave output kernel's LDS (one head buffer, B staged 64 states at
// a time, the decay tables of kHGSmall heads) fits twice in a CU, and its
// registers fit two waves per SIMD without spilling (up to 128 states: the
// C operands of a wave's two output tiles take 2 * N / 8 registers).
template <int P, int N>
constexpr bool out4_fits() {
  if (N > 128) return false;
  constexpr size_t x = (size_t)kQMax * (P + 16) * 2, st = (size_t)P * (N + 8) * 2;
  constexpr size_t bb = (size_t)kQMax * (out_kb<4>(N) + 8) * 2;
  constexpr size_t raw = x + st > bb ? x + st : bb;
  return raw + 3 * kHGSmall * kQMax * 4 + 128 <= 80 * 1024;
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
  a.init = p.initial_state;
  a.states = reinterpret_cast<uint16_t*>(static_cast<char*>(p.workspace) + lay.states_off);
  a.decay = reinterpret_cast<float*>(static_cast<char*>(p.workspace) + lay.decay_off);
  a.dt_softplus = p.dt_softplus;
  a.hshift = p.hshift;
  a.dt_heads = s.nheads >> p.hshift;
  a.batch = s.batch; a.seqlen = s.seqlen; a.nheads = s.nheads; a.headdim = s.headdim;
  a.dstate = s.dstate; a.ngroups = s.ngroups; a.chunk = s.chunk; a.nchunks = s.nchunks;
  const int hpg = s.nheads / s.ngroups;
  a.heads_per_wg_state =
      heads_per_workgroup(hpg, s.nheads, (int64_t)s.nchunks * s.batch, 256, kHGState);
  constexpr bool kOut4 = out4_fits<P, N>();
  a.heads_per_wg_out = heads_per_workgroup(hpg, s.nheads, (int64_t)s.nchunks * s.batch, 256,
                                           kOut4 ? kHGSmall : out_heads_max(P, N));
  a.out_hgroups = (s.nheads + a.heads_per_wg_out - 1) / a.heads_per_wg_out;
  // two four-wave halves when the chunk has more than four output-tile pairs
  a.out_halves = (kOut4 && s.chunk / 32 > 4) ? 2 : 1;

  // state block: B[chunk][NB] and one head's x[chunk][P] share the LDS
  constexpr int NB = N > 128 ? 128 : N;
  dim3 g1(s.nchunks, s.batch, (s.nheads + a.heads_per_wg_state - 1) / a.heads_per_wg_state);
  if (s.chunk == 64)
    hipLaunchKernelGGL((ssd_chunk_state_kernel<P, NB, 64>), g1, dim3(1024), 0, stream, a);
  else if (s.chunk == 128)
    hipLaunchKernelGGL((ssd_chunk_state_kernel<P, NB, 128>), g1, dim3(1024), 0, stream, a);
  else
    hipLaunchKernelGGL((ssd_chunk_state_kernel<P, NB, 256>), g1, dim3(1024), 0, stream, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int64_t PN = (int64_t)P * N;
  dim3 g2((unsigned)(s.batch * s.nheads), (unsigned)((PN / 8 + 255) / 256));
  hipLaunchKernelGGL(ssd_state_pass_kernel, g2, dim3(256), 0, stream, a);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  if constexpr (kOut4) {
    const int64_t pairs = (int64_t)s.nchunks * s.batch * a.out_hgroups;
    const int64_t wgs = a.out_halves == 2 ? (pairs + 7) / 8 * 16 : pairs;
    hipLaunchKernelGGL((ssd_chunk_out_kernel<P, N, 4>), dim3((unsigned)wgs), dim3(256), 0, stream,
                       a);
  } else {
    dim3 g3(s.nchunks, s.batch, a.out_hgroups);
    hipLaunchKernelGGL((ssd_chunk_out_kernel<P, N, 8>), g3, dim3(512), 0, stream, a);
  }
  return hipGetLastError();
}

template <int P>
hipError_t launch_p(const SsdParams& p, hipStream_t stream) {
  switch (p.shape.dstate) {
    case 32: return launch_pn<P, 32>(p, stream);
    case 64: return launch_pn<P, 64>(p, stream);
    case 128: return launch_pn<P, 128>(p, stream);
    case 256:
      if constexpr (P == 32) return launch_pn<32, 256>(p, stream);
      break;
  }
  return hipErrorInvalidValue;
}

// Copy with zero padding or cropping between [outer][ms][ks] (source) and
// [outer][md][kd] (destination): dst[o][m][k] = src[o][m][k] where m < ms
// and k < ks, else 0.  One thread per 8 consecutive destination elements of
// a row; when kd is a multiple of 8 (e.g. a tile size) they are written as
// one 16- or 32-byte store, else one by one.
template <typename T>
__global__ void __launch_bounds__(256) ssd_repack_kernel(const T* __restrict__ src,
                                                       T* __restrict__ dst, int64_t groups,
                                                       int ms, int ks, int md, int kd) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= groups) return;
  const int gpr = (kd + 7) / 8;            // groups per destination row
  const int64_t r = i / gpr;               // destination row: o * md + m
  const int k0 = (int)(i - r * gpr) * 8;
  const int m = (int)(r % md);
  const int64_t o = r / md;
  T v[8];
  const T* s = src + (o * ms + m) * ks;
  if (ks % 8 == 0 && m < ms && k0 + 8 <= ks) {  // whole, aligned source run
    if constexpr (sizeof(T) == 2) {
      const uint4 w = *reinterpret_cast<const uint4*>(s + k0);
      const uint32_t ww[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        v[2 * j] = (T)(ww[j] & 0xffffu);
        v[2 * j + 1] = (T)(ww[j] >> 16);
      }
    } else {
      const float4 lo = reinterpret_cast<const float4*>(s + k0)[0];
      const float4 hi = reinterpret_cast<const float4*>(s + k0)[1];
      v[0] = lo.x; v[1] = lo.y; v[2] = lo.z; v[3] = lo.w;
      v[4] = hi.x; v[5] = hi.y; v[6] = hi.z; v[7] = hi.w;
    }
  } else {
#pragma unroll
    for (int j = 0; j < 8; ++j) v[j] = (m < ms && k0 + j < ks) ? s[k0 + j] : T(0);
  }
  T* d = dst + r * kd + k0;
  if (kd % 8 != 0) {
#pragma unroll
    for (int j = 0; j < 8; ++j)
      if (k0 + j < kd) d[j] = v[j];
    return;
  }
  if constexpr (sizeof(T) == 2) {
    uint32_t w[4];
#pragma unroll
    for (int j = 0; j < 4; ++j)
      w[j] = (uint32_t)v[2 * j] | ((uint32_t)v[2 * j + 1] << 16);
    *reinterpret_cast<uint4*>(d) = make_uint4(w[0], w[1], w[2], w[3]);
  } else {
    reinterpret_cast<float4*>(d)[0] = make_float4(v[0], v[1], v[2], v[3]);
    reinterpret_cast<float4*>(d)[1] = make_float4(v[4], v[5], v[6], v[7]);
  }
}

template <typename T>
hipError_t repack(const void* src, void* dst, int64_t outer, int ms, int ks, int md, int kd,
                  hipStream_t stream) {
  const int64_t groups = outer * md * ((kd + 7) / 8);
  if (groups == 0) return hipSuccess;
  hipLaunchKernelGGL(ssd_repack_kernel<T>, dim3((unsigned)((groups + 255) / 256)), dim3(256), 0,
                     stream, static_cast<const T*>(src), static_cast<T*>(dst), groups, ms, ks, md,
                     kd);
  return hipGetLastError();
}

hipError_t launch_tiles(const SsdParams& p, hipStream_t stream) {
  // Heads wider than the kernels' tile run as 2 or 4 narrower heads: every
  // channel's recurrence is separate, and x, y, the chunk states and the
  // initial and final states of head h, channels vp j .. vp j + vp - 1, are
  // the bytes of head (P / vp) h + j of the vp-channel layout.  The narrower
  // tiles keep the output kernel within its registers (the 128-channel
  // tiles, and 64 channels with 256 states, needed more than 256 VGPRs).
  const int vp = ssd_tile_headdim(p.shape.headdim, p.shape.dstate);
  SsdParams q = p;
  while (q.shape.headdim > vp) {
    q.shape.nheads *= 2;
    q.shape.headdim /= 2;
    q.hshift += 1;
  }
  q.shape.kheaddim = q.shape.headdim;
  switch (q.shape.headdim) {
    case 32: return launch_p<32>(q, stream);
    case 64: return launch_p<64>(q, stream);
  }
  return hipErrorInvalidValue;
}

}  // namespace

hipError_t launch_ssd(const SsdParams& p, hipStream_t stream) {
  const SsdShape& s = p.shape;
  if (!s.padded()) return launch_tiles(p, stream);
  // Headdim or dstate between the tile sizes: run the kernels on
  // zero-padded copies in the workspace (see SsdShape).
  const SsdLayout lay = ssd_layout(s);
  char* ws = static_cast<char*>(p.workspace);
  const int P = s.headdim, N = s.dstate, Pk = s.kheaddim, Nk = s.kdstate;
  const int64_t rows_x = (int64_t)s.batch * s.seqlen * s.nheads;
  const int64_t rows_bc = (int64_t)s.batch * s.seqlen * s.ngroups;
  const int64_t bh = (int64_t)s.batch * s.nheads;
  SsdParams q = p;
  q.x = ws + lay.x_off;
  q.y = ws + lay.y_off;
  q.B = ws + lay.b_off;
  q.C = ws + lay.c_off;
  q.initial_state = p.initial_state ? reinterpret_cast<const float*>(ws + lay.init_off) : nullptr;
  q.final_state = p.final_state ? reinterpret_cast<float*>(ws + lay.final_off) : nullptr;
  q.shape.headdim = Pk;
  q.shape.dstate = Nk;
  hipError_t e = repack<uint16_t>(p.x, ws + lay.x_off, rows_x, 1, P, 1, Pk, stream);
  if (e == hipSuccess) e = repack<uint16_t>(p.B, ws + lay.b_off, rows_bc, 1, N, 1, Nk, stream);
  if (e == hipSuccess) e = repack<uint16_t>(p.C, ws + lay.c_off, rows_bc, 1, N, 1, Nk, stream);
  if (e == hipSuccess && p.initial_state)
    e = repack<float>(p.initial_state, ws + lay.init_off, bh, P, N, Pk, Nk, stream);
  if (e == hipSuccess) e = launch_tiles(q, stream);
  if (e == hipSuccess) e = repack<uint16_t>(ws + lay.y_off, p.y, rows_x, 1, Pk, 1, P, stream);
  if (e == hipSuccess && p.final_state)
    e = repack<float>(ws + lay.final_off, p.final_state, bh, Pk, Nk, P, N, stream);
  return e;
}

}  // namespace ssm
