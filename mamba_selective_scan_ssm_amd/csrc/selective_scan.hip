// selective_scan.hip -- Mamba-1 selective-scan forward kernel for gfx950.
//
// Sources (web pages; cited by title and section/equation):
//   [SPEC]      "ТЕХНИЧЕСКОЕ ЗАДАНИЕ: Реализовать selective scan (Mamba)",
//               Stage 1 items 3-4 (recurrence, softplus, D skip, silu gate).
//   [EXPLAINED] "Mamba CUDA 实现解析", eqs. (4)-(7) (diagonal per-channel
//               recurrence), eqs. (8)-(12) (the associative combine operator
//               and the prefix-scan form), prefix-sum figure.
//   [BLELLOCH]  "从顺序到并行用PyTorch实现Blelloch算法加速Mamba状态空间模型",
//               section 3.2 (chunk long sequences instead of materialising
//               [B, L, ED, N] tensors).
//
// Kernels:
//
// selective_scan_fwd_kernel (whenever there are rows enough to fill the chip):
//   * a channel d of one batch entry b is a row; its dstate axis is split
//     over LPC consecutive lanes (a lane group), NG states per lane, so a
//     wave holds 64/LPC rows and every lane runs the plain recurrence
//     ([EXPLAINED] eq. (7)) for its states over the whole sequence;
//   * B[b,:,t] and C[b,:,t] are the same for every row: each time chunk of
//     them is staged once per workgroup in LDS as float32 (double-buffered,
//     one barrier per chunk);
//   * the per-step work of a row (16-byte loads of u, delta, z; bias,
//     softplus, delta*u, silu(z); skip term, gate and 16-byte stores) is
//     split over the lanes of its group, a contiguous slice of the chunk
//     each; delta and delta*u reach the other lanes of the group by DPP
//     broadcasts folded into the multiplies that consume them, and the
//     group's partial readouts sum_n C h are reduce-scattered back to the
//     owners of the steps with DPP adds.  No per-step value goes through LDS.
//
//   With a workspace it also runs with the sequence cut into segments
//   across workgroups: a first launch stores every segment's aggregate
//   (prod a, v), a DPP scan over the segments turns the aggregates into
//   carry-ins with the combine operator, and a second launch rescans each
//   segment from its carry-in.
//
// selective_scan_chan_kernel / selective_scan_chanw_kernel (B and C read per
// row: groups of channels smaller than a workgroup, down to one channel):
//   one state per lane, a row's states over 16, 32 or 64 lanes, whole
//   128-byte lines of each state's B and C per chunk; the same segments.
//
// selective_scan_slot_kernel (too few rows to give every SIMD a wave, no
// workspace, up to 16 states): the row-parallel lane layout, with the waves
// of a workgroup on the same rows taking consecutive time slots of every
// chunk (slot aggregates and carries through LDS).
//
// selective_scan_split_kernel (too few rows to give every SIMD a wave, no
// workspace, 17..64 states):
//   * lane = row (64 rows per wave); G waves split the dstate axis (NG
//     states each) and share the per-step work through LDS; their partial
//     readouts are added in LDS;
//   * W waves split each time chunk into W slots of T steps.  Slots run the
//     lane-local recurrence from the identity, publish (prod a, v) pairs,
//     and a serial pass over the W slots applies the combine operator of
//     [EXPLAINED] eq. (10) with the running carry to produce every slot's
//     carry-in; the slots then rescan with their carry-in.
//
// All compute exp(delta*A) as exp2(delta*A2) with A2 = A*log2(e) pre-scaled
// once per row (or delta kept in log2 units); the product of a slot's decays is exp2(A2 * sum(delta)), one
// exp per state per slot.  Nothing of size [b, d, L, N] is ever written to
// memory.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <algorithm>

#include "device_math.h"
#include "scan_common.h"
#include "selective_scan_launch.h"

namespace ssm {
namespace {

using namespace scan;

// ---- row-parallel kernel -----------------------------------------------------

// NG: states per lane; LPC: lanes per row (NG*LPC >= dstate); T: steps per
// time chunk.  Block = 256 threads = 4 waves of 64/LPC rows each.
// The workgroup's rows share one group's B and C, staged in LDS (per-row
// B and C: selective_scan_chan_kernel / selective_scan_chanw_kernel).
// With prm.seg_len > 0 the sequence is cut into segments of seg_len steps,
// blockIdx.z selecting one ([EXPLAINED] eq. (11): any regrouping of the
// combine operator gives the same result):
//   AGG = true:  scan the segment from the identity (1, 0) and write its
//                aggregate (prod a, v) per (row, state) to prm.seg_agg;
//   AGG = false: fold the aggregates of the earlier segments onto the
//                initial state (the segment's carry-in), then scan the
//                segment and write its y (and, for the last one, last_state).
template <typename In, int NG, int LPC, int T, bool AGG = false>
__global__ void __launch_bounds__(256) selective_scan_fwd_kernel(ScanParams prm) {
  SSM_POISON_LDS_AT_ENTRY();
  constexpr int NS = NG * LPC;       // states covered per row (>= dstate)
  constexpr int RPW = 64 / LPC;      // rows per wave
  constexpr int RPB = 4 * RPW;       // rows per workgroup
  constexpr int TS = T / LPC;        // steps whose per-step work one lane owns
  constexpr int EPU = Elem<In>::kPer16B;
  static_assert(NG % 4 == 0 && T % EPU == 0 && T % LPC == 0, "tile shape");
  constexpr int UPR = T / EPU;       // 16-byte units per state row of a chunk
  constexpr int UNITS = 2 * NS * UPR;
  constexpr int RBU = (UNITS + 255) / 256;
  // bfloat16 rows with shared B, C keep delta in log2 units: delta' =
  // log2(e) delta (the bias add becomes an fma that scales it, softplus
  // takes its log2 form), so that exp(delta A) = exp2(delta' A) with A as
  // given, and B is staged as ln(2) B so that delta' u B' = delta u B.  Two
  // VALU fewer per (b, d, t) than scaling A; float32 rows keep delta and
  // pre-scale A (the exact form of the float32 parity bound).
  constexpr bool L2U = sizeof(In) == 2;

  __shared__ alignas(16) float sB[2][T][NS];
  __shared__ alignas(16) float sC[2][T][NS];

  const In* __restrict__ u = static_cast<const In*>(prm.u);
  const In* __restrict__ dlt = static_cast<const In*>(prm.delta);
  const In* __restrict__ Bm = static_cast<const In*>(prm.B);
  const In* __restrict__ Cm = static_cast<const In*>(prm.C);
  const In* __restrict__ z = static_cast<const In*>(prm.z);
  In* __restrict__ y = static_cast<In*>(prm.y);

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int slot = lane % LPC;       // position in the row's lane group
  const int b = blockIdx.y;
  const int d = blockIdx.x * RPB + wv * RPW + lane / LPC;
  const bool row_ok = d < prm.dim;
  const bool has_z = !AGG && z != nullptr;
  const int L = prm.seqlen;
  const int N = prm.dstate;
  // time window of this workgroup: segment blockIdx.z, or the whole sequence
  const int seg = blockIdx.z;
  const int t_begin = prm.seg_len ? seg * prm.seg_len : 0;
  const int t_end = prm.seg_len ? min(L, t_begin + prm.seg_len) : L;
  const int64_t nrows = (int64_t)prm.batch * prm.dim;
  const int64_t rowi = (int64_t)b * prm.dim + (row_ok ? d : 0);
  const int64_t row_base = ((int64_t)b * prm.dim + (row_ok ? d : 0)) * (int64_t)L;
  // B, C of group g: [batch, ngroups, dstate, seqlen]; the group of the
  // workgroup's rows (a group covers whole workgroups)
  const int rpg = prm.dim / prm.ngroups;
  const int grp = (int)(blockIdx.x * RPB) / rpg;
  const int64_t bc_base = ((int64_t)b * prm.ngroups + grp) * N * (int64_t)L;

  // Per-row constants for this lane's states n = slot*NG + k.
  float A2[NG];
#pragma unroll
  for (int k = 0; k < NG; ++k) {
    const int n = slot * NG + k;
    A2[k] = (row_ok && n < N) ? prm.A[(int64_t)d * N + n] * (L2U ? 1.0f : kLog2e) : 0.0f;
  }
  const float Dd = (row_ok && prm.D) ? prm.D[d] : 0.0f;
  const float bias = ((row_ok && prm.delta_bias) ? prm.delta_bias[d] : 0.0f) * (L2U ? kLog2e : 1.0f);

  // State: the initial state v_0 of [EXPLAINED] eqs. (8)-(9) when given
  // (a segment's aggregate starts from the identity instead).
  float h[NG];
#pragma unroll
  for (int k = 0; k < NG; ++k) {
    const int n = slot * NG + k;
    h[k] = (!AGG && prm.h0 && row_ok && n < N) ? prm.h0[rowi * N + n] : 0.0f;
  }
  float dsum = 0.0f;  // AGG: sum of delta over the segment (prod a = exp2(A2 dsum))

  // Raw chunk data, loaded one chunk ahead of its use.
  RawSeg<In, TS> ru, rd, rz;
  RawSeg<In, EPU> rbc[RBU];
  auto load_chunk = [&](int c0) {
    const int ts = c0 + slot * TS;
    if (row_ok) {
      load_raw<In, TS>(u, row_base, ts, L, ru);
      load_raw<In, TS>(dlt, row_base, ts, L, rd);
      if (has_z) load_raw<In, TS>(z, row_base, ts, L, rz);
    }
#pragma unroll
    for (int q = 0; q < RBU; ++q) {
      const int e = tid + q * 256;
      const int n = e % NS, rest = e / NS;
      const int seg = rest % UPR, x = rest / UPR;
      if (e < UNITS && n < N) {
        load_raw<In, EPU>(x ? Cm : Bm, bc_base + (int64_t)n * L, c0 + seg * EPU, L, rbc[q]);
      } else {
#pragma unroll
        for (int k = 0; k < RawSeg<In, EPU>::kWords; ++k) rbc[q].w[k] = 0u;
      }
    }
  };

  const int nchunks = (t_end - t_begin + T - 1) / T;
  load_chunk(t_begin);
  if constexpr (!AGG) {
    // carry-in of a later segment, (v_0) (+) agg_0 (+) ... (+) agg_{seg-1}
    // with the combine operator of [EXPLAINED] eq. (10): left in slot seg-1
    // by segment_carry_kernel.
    if (seg > 0 && row_ok) {
      const float* cin = prm.seg_agg + ((int64_t)(seg - 1) * nrows + rowi) * N * 2;
#pragma unroll
      for (int k = 0; k < NG; ++k)
        if (slot * NG + k < N) h[k] = cin[2 * (slot * NG + k) + 1];
    }
  }
  for (int ch = 0; ch < nchunks; ++ch) {
    const int c0 = t_begin + ch * T;
    const int buf = ch & 1;  // its last readers were two chunks ago, before the last barrier

    // -- B and C of this chunk into LDS as float32 [t][n] --------------------
#pragma unroll
    for (int q = 0; q < RBU; ++q) {
      const int e = tid + q * 256;
      if (e < UNITS) {
        const int n = e % NS, rest = e / NS;
        const int seg = rest % UPR, x = rest / UPR;
        float v[EPU];
        decode_raw<In, EPU>(rbc[q], v);
#pragma unroll
        for (int i = 0; i < EPU; ++i) {
          if (x) sC[buf][seg * EPU + i][n] = v[i];
          else sB[buf][seg * EPU + i][n] = L2U ? v[i] * kLn2 : v[i];
        }
      }
    }
    // -- per-step work for this lane's slice of the chunk ---------------------
    const int ts = c0 + slot * TS;
    float uk[TS], gk[TS], dl[TS], du[TS];
    {
      float dr[TS];
      decode_raw<In, TS>(ru, uk);
      decode_raw<In, TS>(rd, dr);
      if (has_z) {
        float zk[TS];
        decode_raw<In, TS>(rz, zk);
#pragma unroll
        for (int j = 0; j < TS; ++j) gk[j] = silu_f(zk[j]);
      } else {
#pragma unroll
        for (int j = 0; j < TS; ++j) gk[j] = 1.0f;
      }
      // (the flag is uniform: one branch around the loop, not a select per
      // step; delta + bias is formed once, before it, or the compiler forms
      // it on both sides)
      if constexpr (L2U) {
#pragma unroll
        for (int j = 0; j < TS; ++j) dl[j] = __builtin_fmaf(dr[j], kLog2e, bias);
        if (prm.delta_softplus) {
#pragma unroll
          for (int j = 0; j < TS; ++j) dl[j] = softplus_log2_short(dl[j]);
        }
      } else {
#pragma unroll
        for (int j = 0; j < TS; ++j) dl[j] = dr[j] + bias;
        if (prm.delta_softplus) {
#pragma unroll
          for (int j = 0; j < TS; ++j) dl[j] = softplus_in<In>(dl[j]);
        }
      }
      // Steps past the end are the identity (delta = 0).  Rows past `dim`
      // compute on zeros and are never stored.
      if (ts + TS > L) {
#pragma unroll
        for (int j = 0; j < TS; ++j)
          if (ts + j >= L) dl[j] = 0.0f;
      }
#pragma unroll
      for (int j = 0; j < TS; ++j) du[j] = dl[j] * uk[j];
    }
    if (ch + 1 < nchunks) load_chunk(c0 + T);
    __syncthreads();

    // -- recurrence over the chunk ([EXPLAINED] eq. (7)) -----------------------
    float yp[T];
    static_for<0, T>([&](auto tc) {
      constexpr int t = decltype(tc)::value;
      float dt, dut;  // delta and delta*u of step t, from the lane that owns it
      if constexpr (LPC > 1) {
        dt = dpp_f<group_bcast<LPC>(t / TS)>(dl[t % TS]);
        dut = dpp_f<group_bcast<LPC>(t / TS)>(du[t % TS]);
      } else {
        dt = dl[t];
        dut = du[t];
      }
      float acc = 0.0f;
      if constexpr (AGG) dsum += dt;
#pragma unroll
      for (int k4 = 0; k4 < NG; k4 += 4) {
        float bv[4], cv[4];
        const float4 bq = *reinterpret_cast<const float4*>(&sB[buf][t][slot * NG + k4]);
        bv[0] = bq.x; bv[1] = bq.y; bv[2] = bq.z; bv[3] = bq.w;
        if constexpr (!AGG) {
          const float4 cq = *reinterpret_cast<const float4*>(&sC[buf][t][slot * NG + k4]);
          cv[0] = cq.x; cv[1] = cq.y; cv[2] = cq.z; cv[3] = cq.w;
        }
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const float a = fast_exp2(dt * A2[k4 + i]);
          h[k4 + i] = __builtin_fmaf(a, h[k4 + i], dut * bv[i]);
          if constexpr (!AGG) acc = __builtin_fmaf(cv[i], h[k4 + i], acc);
        }
      }
      yp[t] = acc;
    });
    if constexpr (AGG) continue;  // an aggregate has no output

    // -- sum the group's partial readouts onto the owners of the steps ---------
    float yo[TS];
    if constexpr (LPC == 4) {
      float s1[T / 2];
      const bool lo = slot < 2;  // lanes 0, 1 keep the first half of the chunk
#pragma unroll
      for (int j = 0; j < T / 2; ++j) {
        const float keep = lo ? yp[j] : yp[T / 2 + j];
        const float send = lo ? yp[T / 2 + j] : yp[j];
        s1[j] = keep + dpp_f<kSwapHalves>(send);
      }
      const bool ev = (slot & 1) == 0;
#pragma unroll
      for (int j = 0; j < TS; ++j) {
        const float keep = ev ? s1[j] : s1[TS + j];
        const float send = ev ? s1[TS + j] : s1[j];
        yo[j] = keep + dpp_f<kSwapPairs>(send);
      }
    } else if constexpr (LPC == 2) {
      const bool ev = slot == 0;
#pragma unroll
      for (int j = 0; j < TS; ++j) {
        const float keep = ev ? yp[j] : yp[TS + j];
        const float send = ev ? yp[TS + j] : yp[j];
        yo[j] = keep + dpp_f<kSwapPairs>(send);
      }
    } else {
#pragma unroll
      for (int j = 0; j < TS; ++j) yo[j] = yp[j];
    }
    // -- skip term, gate, store -------------------------------------------------
#pragma unroll
    for (int j = 0; j < TS; ++j) yo[j] = __builtin_fmaf(Dd, uk[j], yo[j]) * gk[j];
    if (row_ok && y) store_seg<In, TS>(y, row_base, ts, L, yo);
  }

  if constexpr (AGG) {
    // the segment's aggregate (prod a, v) = (exp2(A2 * sum delta), h)
    if (row_ok) {
      float* ag = prm.seg_agg + ((int64_t)seg * nrows + rowi) * N * 2;
#pragma unroll
      for (int k = 0; k < NG; ++k) {
        const int n = slot * NG + k;
        if (n < N) {
          ag[2 * n] = fast_exp2(A2[k] * dsum);
          ag[2 * n + 1] = h[k];
        }
      }
    }
    return;
  }
  // -- final state -------------------------------------------------------------
  if (prm.last_state && row_ok && t_end == L) {
    float* ls = prm.last_state + ((int64_t)b * prm.dim + d) * N;
#pragma unroll
    for (int k = 0; k < NG; ++k)
      if (slot * NG + k < N) ls[slot * NG + k] = h[k];
  }
}

// ---- per-row B, C: one state per lane -------------------------------------------

// For B and C read per row (groups of channels smaller than a row-parallel
// workgroup, e.g. one per channel) with up to 16 states.  B, C are
// [batch, ngroups, dstate, seqlen]: each (row, state) is its own sequence of
// seqlen elements, so a lane that holds several states of a row, reading a
// short piece of each per chunk, touches a 128-byte line four times in four
// chunks, long after the L2 has dropped it (measured: 4x the algorithmic HBM
// bytes).  Here a row's 16 states take the 16 lanes of a DPP row, one state
// per lane, and a chunk is T = 128 bytes of steps (64 bf16, 32 float32), so
// every lane reads whole lines of its state's B and C, loaded one chunk
// ahead into registers.  Step t of a chunk belongs to lane t % 16 of the
// row (its delta, softplus, delta*u, gate, skip term and y); its delta and
// delta*u reach the row's lanes through a DPP row broadcast folded into the
// multiplies.  Each lane's partial readout C h of a step goes to LDS; after
// every 16 steps each lane adds the 16 partials of its step of the block
// ([EXPLAINED] eq. (7) per state; the readout sum of [SPEC] Stage 1 item 3).
// Block = 256 threads = 4 waves of 4 rows.
// LOAD: how B and C of the next chunk are loaded.  Rows a whole number of
// 16-byte units long: 16-byte loads after the chunk (kChanLoadAfter), or
// each unit reloaded with the next chunk's as soon as its last step has been
// used (kChanLoadSpread: the loads spread over the chunk, no second set of
// registers; float32 3.0 against 4.1 ms at 4096 channels of 2048 steps,
// bfloat16 1.5 against 1.1 ms, so bfloat16 loads after the chunk).  Other
// rows: element loads after the chunk (kChanLoadElem).
constexpr int kChanLoadElem = 0, kChanLoadAfter = 1, kChanLoadSpread = 2;
// With prm.seg_len > 0, blockIdx.z selects a time segment as in the
// row-parallel kernel: AGG = true scans it from the identity and writes its
// aggregate (prod a, v) per (row, state); AGG = false starts from the
// carry-in the combine scan left for it.
template <typename In, int LOAD, bool AGG = false>
__global__ void __launch_bounds__(256) selective_scan_chan_kernel(ScanParams prm) {
  SSM_POISON_LDS_AT_ENTRY();
  constexpr bool VEC = LOAD != kChanLoadElem;
  constexpr int EPU = Elem<In>::kPer16B;
  constexpr int T = 128 / (int)sizeof(In);  // steps per chunk: one 128-byte line per state
  constexpr int NB = T / 16;                // 16-step blocks per chunk
  constexpr int kRowP = 16 * 20 + 16;       // LDS floats per row of partials
  // partials of step tt of the block from state n at [rw][tt][n], rows of 20
  // floats and row groups 16 floats apart modulo 64 banks: the stores of a
  // step (16 consecutive floats per row) and each lane's four 16-byte reads
  // of its step (16 lanes 80 bytes apart) meet no bank twice
  __shared__ alignas(16) float sP[4][4 * kRowP];

  const In* __restrict__ u = static_cast<const In*>(prm.u);
  const In* __restrict__ dlt = static_cast<const In*>(prm.delta);
  const In* __restrict__ Bm = static_cast<const In*>(prm.B);
  const In* __restrict__ Cm = static_cast<const In*>(prm.C);
  const In* __restrict__ z = static_cast<const In*>(prm.z);
  In* __restrict__ y = static_cast<In*>(prm.y);

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int rw = lane >> 4;   // row within the wave
  const int l = lane & 15;    // state n of this lane, and the owner index of steps
  const int b = blockIdx.y;
  const int d = blockIdx.x * 16 + wv * 4 + rw;
  const bool row_ok = d < prm.dim;
  const int L = prm.seqlen;
  const int N = prm.dstate;
  const bool st_ok = row_ok && l < N;
  const bool has_z = z != nullptr;
  const int64_t rowi = (int64_t)b * prm.dim + (row_ok ? d : 0);
  const int64_t row_base = rowi * (int64_t)L;
  const int rpg = prm.dim / prm.ngroups;
  const int64_t bc_row = (((int64_t)b * prm.ngroups + (row_ok ? d : 0) / rpg) * N +
                          (st_ok ? l : 0)) * (int64_t)L;

  const float A2 = st_ok ? prm.A[(int64_t)d * N + l] * kLog2e : 0.0f;
  const float Dd = (row_ok && prm.D) ? prm.D[d] : 0.0f;
  const float bias = (row_ok && prm.delta_bias) ? prm.delta_bias[d] : 0.0f;
  // time window: segment blockIdx.z, or the whole sequence
  const int seg = blockIdx.z;
  const int t_begin = prm.seg_len ? seg * prm.seg_len : 0;
  const int t_end = prm.seg_len ? min(L, t_begin + prm.seg_len) : L;
  const int64_t nrows = (int64_t)prm.batch * prm.dim;
  float h = (!AGG && st_ok && prm.h0) ? prm.h0[rowi * N + l] : 0.0f;
  if (!AGG && seg > 0 && st_ok)  // carry-in left in slot seg - 1 by segment_carry_kernel
    h = prm.seg_agg[(((int64_t)(seg - 1) * nrows + rowi) * N + l) * 2 + 1];
  float dsum = 0.0f;  // AGG: sum of delta over the segment (prod a = exp2(A2 dsum))

  // B, C of this lane's state for the steps c0 .. c0 + T - 1.  Steps past
  // the end read the row's last elements instead (finite values that meet
  // delta = 0 there: the state does not move and their readout is not
  // stored), so every load is unconditional (lanes of states past dstate
  // read state 0 and use zeros).
  RawSeg<In, T> rB, rC;
  auto load_unit = [&](const In* __restrict__ p, int c0, int k, RawSeg<In, T>& r) {
    const uint4 v = *reinterpret_cast<const uint4*>(p + bc_row + min(c0 + EPU * k, L - EPU));
    r.w[4 * k] = st_ok ? v.x : 0u;
    r.w[4 * k + 1] = st_ok ? v.y : 0u;
    r.w[4 * k + 2] = st_ok ? v.z : 0u;
    r.w[4 * k + 3] = st_ok ? v.w : 0u;
  };
  auto load_line = [&](const In* __restrict__ p, int c0, RawSeg<In, T>& r) {
    if constexpr (VEC) {
#pragma unroll
      for (int k = 0; k < T / EPU; ++k) load_unit(p, c0, k, r);
    } else if constexpr (sizeof(In) == 4) {
#pragma unroll
      for (int k = 0; k < T; ++k)
        r.w[k] = reinterpret_cast<const uint32_t*>(p)[bc_row + min(c0 + k, L - 1)];
    } else {
#pragma unroll
      for (int k = 0; k < T / 2; ++k)
        r.w[k] = (uint32_t)p[bc_row + min(c0 + 2 * k, L - 1)] |
                 ((uint32_t)p[bc_row + min(c0 + 2 * k + 1, L - 1)] << 16);
    }
  };
  auto load_bc = [&](int c0, RawSeg<In, T>& rb, RawSeg<In, T>& rc) {
    load_line(Bm, c0, rb);
    load_line(Cm, c0, rc);
    if (!VEC && !st_ok) {
#pragma unroll
      for (int w = 0; w < RawSeg<In, T>::kWords; ++w) rb.w[w] = rc.w[w] = 0u;
    }
  };
  float* const prow = &sP[wv][rw * kRowP];

  auto to_f32 = [](In v) {
    if constexpr (sizeof(In) == 4) return (float)v;
    else return __uint_as_float((uint32_t)v << 16);
  };
  // this lane's steps c0 + 16 j + l of u, delta, z, loaded one chunk ahead
  // (B and C are loaded after their last use in the previous chunk: the
  // registers of one chunk, not two, leave room for four waves per SIMD)
  In ru[NB], rd[NB], rz[NB];
  auto load_own = [&](int c0) {
#pragma unroll
    for (int j = 0; j < NB; ++j) {
      const int t = min(c0 + 16 * j + l, L - 1);
      ru[j] = u[row_base + t];
      rd[j] = dlt[row_base + t];
      rz[j] = has_z ? z[row_base + t] : In(0);
    }
  };
  const int nchunks = (t_end - t_begin + T - 1) / T;
  load_bc(t_begin, rB, rC);
  load_own(t_begin);
  for (int ch = 0; ch < nchunks; ++ch) {
    const int c0 = t_begin + ch * T;
    // -- this lane's steps c0 + 16 j + l: delta, softplus, delta*u, gate --------
    float dl[NB], du[NB], uk[NB], gk[NB];
#pragma unroll
    for (int j = 0; j < NB; ++j) {
      const bool in = row_ok && c0 + 16 * j + l < t_end;
      uk[j] = in ? to_f32(ru[j]) : 0.0f;
      const float dr = in ? to_f32(rd[j]) : 0.0f;
      const float zz = (in && has_z) ? to_f32(rz[j]) : 0.0f;
      float dd = dr + bias;
      if (prm.delta_softplus) dd = softplus_in<In>(dd);
      dl[j] = in ? dd : 0.0f;  // steps past the end are the identity
      du[j] = dl[j] * uk[j];
      gk[j] = has_z ? silu_f(zz) : 1.0f;
    }
    if (ch + 1 < nchunks) load_own(c0 + T);

    float yo[NB] = {};
    static_for<0, T>([&](auto tc) {
      constexpr int t = decltype(tc)::value;
      constexpr int own = t % 16, j = t / 16;
      const float dt = dpp_f<0x150 + own>(dl[j]);    // row broadcast of lane `own`
      const float dut = dpp_f<0x150 + own>(du[j]);
      const float a = fast_exp2(dt * A2);
      h = __builtin_fmaf(a, h, dut * raw_elem<In, T, t>(rB));
      if constexpr (AGG) dsum += dt;
      else prow[own * 20 + l] = raw_elem<In, T, t>(rC) * h;
      if constexpr (LOAD == kChanLoadSpread && (t + 1) % EPU == 0) {  // unit used up: the next chunk's
        load_unit(Bm, c0 + T, t / EPU, rB);
        load_unit(Cm, c0 + T, t / EPU, rC);
      }
      if constexpr (!AGG && own == 15) {
        // the 16 partials of this lane's step of the block, in a fixed order
        // (the lanes of a row share a wave, whose LDS accesses complete in
        // program order: no barrier)
        __builtin_amdgcn_wave_barrier();
        const float4 q0 = *reinterpret_cast<const float4*>(prow + l * 20);
        const float4 q1 = *reinterpret_cast<const float4*>(prow + l * 20 + 4);
        const float4 q2 = *reinterpret_cast<const float4*>(prow + l * 20 + 8);
        const float4 q3 = *reinterpret_cast<const float4*>(prow + l * 20 + 12);
        __builtin_amdgcn_wave_barrier();
        yo[j] = (((q0.x + q0.y) + (q0.z + q0.w)) + ((q1.x + q1.y) + (q1.z + q1.w))) +
                (((q2.x + q2.y) + (q2.z + q2.w)) + ((q3.x + q3.y) + (q3.z + q3.w)));
      }
    });
    // -- skip term, gate ([SPEC] Stage 1 item 4), store -------------------------------
    if (!AGG && row_ok && y) {
#pragma unroll
      for (int j = 0; j < NB; ++j) {
        const int t = c0 + 16 * j + l;
        if (t < t_end) Elem<In>::store(y, row_base + t, __builtin_fmaf(Dd, uk[j], yo[j]) * gk[j]);
      }
    }
    if (LOAD != kChanLoadSpread && ch + 1 < nchunks) load_bc(c0 + T, rB, rC);
  }
  if constexpr (AGG) {
    if (st_ok) {
      float* ag = prm.seg_agg + (((int64_t)seg * nrows + rowi) * N + l) * 2;
      ag[0] = fast_exp2(A2 * dsum);
      ag[1] = h;
    }
  } else if (prm.last_state && st_ok && t_end == L) {
    prm.last_state[rowi * N + l] = h;
  }
}

// Per-row B, C with 17..64 states: the same one-state-per-lane layout with
// S = 32 or 64 lanes per row (two rows or one per wave; lanes past dstate
// idle).  A row now spans more than one DPP row, so the delta and delta*u of
// step t come from its owner lane (t mod S of the row) with v_readlane into
// a scalar register, one per row of the wave (a select between the two rows
// when S = 32): a few instructions per step of the wave, not per state.
// Partial readouts go to LDS ([row][step][state], rows of S + 4 floats) and
// after the chunk the owner of each step adds its S partials.
template <typename In, int S, int LOAD, bool AGG = false>
__global__ void __launch_bounds__(256) selective_scan_chanw_kernel(ScanParams prm) {
  SSM_POISON_LDS_AT_ENTRY();
  constexpr bool VEC = LOAD != kChanLoadElem;
  constexpr int EPU = Elem<In>::kPer16B;
  constexpr int T = 128 / (int)sizeof(In);  // steps per chunk: one 128-byte line per state
  constexpr int RPW = 64 / S;               // rows per wave
  constexpr int NOWN = (T + S - 1) / S;     // steps of a chunk owned per lane (some lanes
                                            // own none when T < S)
  constexpr int kRowT = S + 4;              // LDS floats per step of a row
  // the two rows of a wave (S = 32) 32 floats apart modulo 64 banks, so the
  // 64 lanes' stores of a step meet no bank twice
  constexpr int kRowR = T * kRowT + 32;
  static_assert(S == 32 || S == 64, "lanes per row");
  __shared__ alignas(16) float sP[4][RPW * kRowR];

  const In* __restrict__ u = static_cast<const In*>(prm.u);
  const In* __restrict__ dlt = static_cast<const In*>(prm.delta);
  const In* __restrict__ Bm = static_cast<const In*>(prm.B);
  const In* __restrict__ Cm = static_cast<const In*>(prm.C);
  const In* __restrict__ z = static_cast<const In*>(prm.z);
  In* __restrict__ y = static_cast<In*>(prm.y);

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int rw = lane / S;   // row within the wave
  const int l = lane % S;    // state n of this lane, and the owner index of steps
  const int b = blockIdx.y;
  const int d = blockIdx.x * (4 * RPW) + wv * RPW + rw;
  const bool row_ok = d < prm.dim;
  const int L = prm.seqlen;
  const int N = prm.dstate;
  const bool st_ok = row_ok && l < N;
  const bool has_z = z != nullptr;
  const int64_t rowi = (int64_t)b * prm.dim + (row_ok ? d : 0);
  const int64_t row_base = rowi * (int64_t)L;
  const int rpg = prm.dim / prm.ngroups;
  const int64_t bc_row = (((int64_t)b * prm.ngroups + (row_ok ? d : 0) / rpg) * N +
                          (st_ok ? l : 0)) * (int64_t)L;

  const float A2 = st_ok ? prm.A[(int64_t)d * N + l] * kLog2e : 0.0f;
  const float Dd = (row_ok && prm.D) ? prm.D[d] : 0.0f;
  const float bias = (row_ok && prm.delta_bias) ? prm.delta_bias[d] : 0.0f;
  // time window: segment blockIdx.z, or the whole sequence
  const int seg = blockIdx.z;
  const int t_begin = prm.seg_len ? seg * prm.seg_len : 0;
  const int t_end = prm.seg_len ? min(L, t_begin + prm.seg_len) : L;
  const int64_t nrows = (int64_t)prm.batch * prm.dim;
  float h = (!AGG && st_ok && prm.h0) ? prm.h0[rowi * N + l] : 0.0f;
  if (!AGG && seg > 0 && st_ok)  // carry-in left in slot seg - 1 by segment_carry_kernel
    h = prm.seg_agg[(((int64_t)(seg - 1) * nrows + rowi) * N + l) * 2 + 1];
  float dsum = 0.0f;  // AGG: sum of delta over the segment (prod a = exp2(A2 dsum))

  // B, C of this lane's state, steps past the end reading the row's last
  // elements (as in selective_scan_chan_kernel)
  RawSeg<In, T> rB, rC;
  auto load_unit = [&](const In* __restrict__ p, int c0, int k, RawSeg<In, T>& r) {
    const uint4 v = *reinterpret_cast<const uint4*>(p + bc_row + min(c0 + EPU * k, L - EPU));
    r.w[4 * k] = st_ok ? v.x : 0u;
    r.w[4 * k + 1] = st_ok ? v.y : 0u;
    r.w[4 * k + 2] = st_ok ? v.z : 0u;
    r.w[4 * k + 3] = st_ok ? v.w : 0u;
  };
  auto load_line = [&](const In* __restrict__ p, int c0, RawSeg<In, T>& r) {
    if constexpr (VEC) {
#pragma unroll
      for (int k = 0; k < T / EPU; ++k) load_unit(p, c0, k, r);
    } else if constexpr (sizeof(In) == 4) {
#pragma unroll
      for (int k = 0; k < T; ++k)
        r.w[k] = reinterpret_cast<const uint32_t*>(p)[bc_row + min(c0 + k, L - 1)];
    } else {
#pragma unroll
      for (int k = 0; k < T / 2; ++k)
        r.w[k] = (uint32_t)p[bc_row + min(c0 + 2 * k, L - 1)] |
                 ((uint32_t)p[bc_row + min(c0 + 2 * k + 1, L - 1)] << 16);
    }
  };
  auto load_bc = [&](int c0) {
    load_line(Bm, c0, rB);
    load_line(Cm, c0, rC);
    if (!VEC && !st_ok) {
#pragma unroll
      for (int w = 0; w < RawSeg<In, T>::kWords; ++w) rB.w[w] = rC.w[w] = 0u;
    }
  };
  auto to_f32 = [](In v) {
    if constexpr (sizeof(In) == 4) return (float)v;
    else return __uint_as_float((uint32_t)v << 16);
  };
  // this lane's steps c0 + S j + l of u, delta, z, loaded one chunk ahead
  In ru[NOWN], rd[NOWN], rz[NOWN];
  auto load_own = [&](int c0) {
#pragma unroll
    for (int j = 0; j < NOWN; ++j) {
      const int t = min(c0 + S * j + l, L - 1);
      ru[j] = u[row_base + t];
      rd[j] = dlt[row_base + t];
      rz[j] = has_z ? z[row_base + t] : In(0);
    }
  };
  float* const prow = &sP[wv][rw * kRowR];
  // the value of lane `own` of each row of the wave, for this lane's row
  auto from_owner = [&](float v, auto ownc) {
    constexpr int own = decltype(ownc)::value;
    const float s0 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), own));
    if constexpr (RPW == 1) {
      return s0;
    } else {
      const float s1 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), S + own));
      return rw == 0 ? s0 : s1;
    }
  };

  const int nchunks = (t_end - t_begin + T - 1) / T;
  load_bc(t_begin);
  load_own(t_begin);
  for (int ch = 0; ch < nchunks; ++ch) {
    const int c0 = t_begin + ch * T;
    float dl[NOWN], du[NOWN], uk[NOWN], gk[NOWN];
#pragma unroll
    for (int j = 0; j < NOWN; ++j) {
      const bool in = row_ok && S * j + l < T && c0 + S * j + l < t_end;
      uk[j] = in ? to_f32(ru[j]) : 0.0f;
      const float dr = in ? to_f32(rd[j]) : 0.0f;
      const float zz = (in && has_z) ? to_f32(rz[j]) : 0.0f;
      float dd = dr + bias;
      if (prm.delta_softplus) dd = softplus_in<In>(dd);
      dl[j] = in ? dd : 0.0f;  // steps past the end are the identity
      du[j] = dl[j] * uk[j];
      gk[j] = has_z ? silu_f(zz) : 1.0f;
    }
    if (ch + 1 < nchunks) load_own(c0 + T);

    static_for<0, T>([&](auto tc) {
      constexpr int t = decltype(tc)::value;
      constexpr int own = t % S, j = t / S;
      const float dt = from_owner(dl[j], std::integral_constant<int, own>{});
      const float dut = from_owner(du[j], std::integral_constant<int, own>{});
      const float a = fast_exp2(dt * A2);
      h = __builtin_fmaf(a, h, dut * raw_elem<In, T, t>(rB));
      if constexpr (AGG) dsum += dt;
      else prow[t * kRowT + l] = raw_elem<In, T, t>(rC) * h;
      if constexpr (LOAD == kChanLoadSpread && (t + 1) % EPU == 0) {
        load_unit(Bm, c0 + T, t / EPU, rB);
        load_unit(Cm, c0 + T, t / EPU, rC);
      }
    });
    // -- each owner adds the S partials of its steps, skip term, gate, store --
    // (the lanes of a row share a wave, whose LDS accesses complete in
    // program order: no barrier)
    __builtin_amdgcn_wave_barrier();
    float yo[NOWN];
#pragma unroll
    for (int j = 0; j < NOWN; ++j) {
      if constexpr (AGG) { yo[j] = 0.0f; continue; }
      const int t = (S * j + l) < T ? S * j + l : T - 1;
      const float* q = prow + t * kRowT;
      float acc[4] = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
      for (int k = 0; k < S / 4; ++k) {
        const float4 v = *reinterpret_cast<const float4*>(q + 4 * k);
        acc[k & 3] += (v.x + v.y) + (v.z + v.w);
      }
      yo[j] = (acc[0] + acc[1]) + (acc[2] + acc[3]);
    }
    __builtin_amdgcn_wave_barrier();
    if (!AGG && row_ok && y) {
#pragma unroll
      for (int j = 0; j < NOWN; ++j) {
        const int t = c0 + S * j + l;
        if (S * j + l < T && t < t_end)
          Elem<In>::store(y, row_base + t, __builtin_fmaf(Dd, uk[j], yo[j]) * gk[j]);
      }
    }
    if (LOAD != kChanLoadSpread && ch + 1 < nchunks) load_bc(c0 + T);
  }
  if constexpr (AGG) {
    if (st_ok) {
      float* ag = prm.seg_agg + (((int64_t)seg * nrows + rowi) * N + l) * 2;
      ag[0] = fast_exp2(A2 * dsum);
      ag[1] = h;
    }
  } else if (prm.last_state && st_ok && t_end == L) {
    prm.last_state[rowi * N + l] = h;
  }
}

// ---- time-sliced row kernel --------------------------------------------------

// NG: states per lane; LPC: lanes per row (NG*LPC >= dstate); T: steps per
// time slot; W: time slots per chunk = waves per workgroup.  Block = 64*W
// threads, all W waves on the same 64/LPC rows (the row kernel's lane
// layout: a row's states over a group of LPC lanes, its per-step work over
// their slices of the slot), wave w taking the steps [c0 + w T, c0 + (w+1) T)
// of every chunk of W T steps.  Per chunk, each wave
//   1. scans its slot from the identity, keeping the slot's decays
//      a_t = exp2(delta_t A2) in registers, and publishes the slot's
//      aggregate (prod a, v) = (exp2(A2 sum delta), h) per (row, state);
//   2. folds the aggregates of the earlier slots onto the running carry of
//      the chunks before ([EXPLAINED] eqs. (10)-(11)) -- its carry-in -- and
//      all W of them into the next chunk's carry;
//   3. rescans the slot from its carry-in with the cached decays, reads out
//      y, reduce-scatters the partial readouts over the row's lanes, adds
//      the skip term, gates and stores.
// For shapes whose rows alone give too few waves, without any workspace:
// the rows of a wave are spread over W times as many waves (the rescan
// costs about three issue slots per state update on top of the scan).
template <typename In, int NG, int LPC, int T, int W>
__global__ void __launch_bounds__(64 * W) selective_scan_slot_kernel(ScanParams prm) {
  SSM_POISON_LDS_AT_ENTRY();
  constexpr int NS = NG * LPC;       // states covered per row (>= dstate)
  constexpr int RPB = 64 / LPC;      // rows per workgroup (shared by its waves)
  constexpr int TS = T / LPC;        // steps of the slot whose per-step work one lane owns
  constexpr int TC = W * T;          // steps per chunk
  constexpr int NTHR = 64 * W;
  constexpr int EPU = Elem<In>::kPer16B;
  static_assert(NG % 4 == 0 && T % LPC == 0 && TC % EPU == 0, "tile shape");
  constexpr int UPR = TC / EPU;      // 16-byte units per state row of a chunk
  constexpr int UNITS = 2 * NS * UPR;
  constexpr int RBU = (UNITS + NTHR - 1) / NTHR;

  __shared__ alignas(16) float sB[2][TC][NS];
  __shared__ alignas(16) float sC[2][TC][NS];
  __shared__ alignas(16) float2 sAgg[W][RPB][NS];  // slot aggregates per (row, state)

  const In* __restrict__ u = static_cast<const In*>(prm.u);
  const In* __restrict__ dlt = static_cast<const In*>(prm.delta);
  const In* __restrict__ Bm = static_cast<const In*>(prm.B);
  const In* __restrict__ Cm = static_cast<const In*>(prm.C);
  const In* __restrict__ z = static_cast<const In*>(prm.z);
  In* __restrict__ y = static_cast<In*>(prm.y);

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);  // time slot of this wave
  const int slot = lane % LPC;       // position in the row's lane group
  const int r = lane / LPC;          // row within the workgroup
  const int b = blockIdx.y;
  const int d = blockIdx.x * RPB + r;
  const bool row_ok = d < prm.dim;
  const bool has_z = z != nullptr;
  const int L = prm.seqlen;
  const int N = prm.dstate;
  const int64_t rowi = (int64_t)b * prm.dim + (row_ok ? d : 0);
  const int64_t row_base = rowi * (int64_t)L;
  // B, C of the group of the workgroup's rows: [batch, ngroups, dstate, seqlen]
  const int grp = (int)(blockIdx.x * RPB) / (prm.dim / prm.ngroups);
  const int64_t bc_base = ((int64_t)b * prm.ngroups + grp) * N * (int64_t)L;

  float A2[NG];
#pragma unroll
  for (int k = 0; k < NG; ++k) {
    const int n = slot * NG + k;
    A2[k] = (row_ok && n < N) ? prm.A[(int64_t)d * N + n] * kLog2e : 0.0f;
  }
  const float Dd = (row_ok && prm.D) ? prm.D[d] : 0.0f;
  const float bias = (row_ok && prm.delta_bias) ? prm.delta_bias[d] : 0.0f;
  // running carry: the state entering the chunk (v_0 of [EXPLAINED] eqs.
  // (8)-(9) when an initial state is given)
  float carry[NG];
#pragma unroll
  for (int k = 0; k < NG; ++k) {
    const int n = slot * NG + k;
    carry[k] = (prm.h0 && row_ok && n < N) ? prm.h0[rowi * N + n] : 0.0f;
  }

  RawSeg<In, TS> ru, rd, rz;
  RawSeg<In, EPU> rbc[RBU];
  auto load_chunk = [&](int c0) {
    const int ts = c0 + w * T + slot * TS;
    if (row_ok) {
      load_raw<In, TS>(u, row_base, ts, L, ru);
      load_raw<In, TS>(dlt, row_base, ts, L, rd);
      if (has_z) load_raw<In, TS>(z, row_base, ts, L, rz);
    }
#pragma unroll
    for (int q = 0; q < RBU; ++q) {
      const int e = tid + q * NTHR;
      const int n = e % NS, rest = e / NS;
      const int sg = rest % UPR, x = rest / UPR;
      if (e < UNITS && n < N) {
        load_raw<In, EPU>(x ? Cm : Bm, bc_base + (int64_t)n * L, c0 + sg * EPU, L, rbc[q]);
      } else {
#pragma unroll
        for (int k = 0; k < RawSeg<In, EPU>::kWords; ++k) rbc[q].w[k] = 0u;
      }
    }
  };

  const int nchunks = (L + TC - 1) / TC;
  load_chunk(0);
  for (int ch = 0; ch < nchunks; ++ch) {
    const int c0 = ch * TC;
    const int buf = ch & 1;  // its last readers were two chunks ago, before the last barrier
    // -- B and C of this chunk into LDS as float32 [t][n] ----------------------
#pragma unroll
    for (int q = 0; q < RBU; ++q) {
      const int e = tid + q * NTHR;
      if (e < UNITS) {
        const int n = e % NS, rest = e / NS;
        const int sg = rest % UPR, x = rest / UPR;
        float v[EPU];
        decode_raw<In, EPU>(rbc[q], v);
#pragma unroll
        for (int i = 0; i < EPU; ++i) {
          if (x) sC[buf][sg * EPU + i][n] = v[i];
          else sB[buf][sg * EPU + i][n] = v[i];
        }
      }
    }
    // -- per-step work for this lane's slice of the slot ------------------------
    const int ts = c0 + w * T + slot * TS;
    float uk[TS], gk[TS], dl[TS], du[TS];
    {
      float dr[TS];
      decode_raw<In, TS>(ru, uk);
      decode_raw<In, TS>(rd, dr);
      if (has_z) {
        float zk[TS];
        decode_raw<In, TS>(rz, zk);
#pragma unroll
        for (int j = 0; j < TS; ++j) gk[j] = silu_f(zk[j]);
      } else {
#pragma unroll
        for (int j = 0; j < TS; ++j) gk[j] = 1.0f;
      }
#pragma unroll
      for (int j = 0; j < TS; ++j) dl[j] = dr[j] + bias;  // (formed once, outside the branch)
      if (prm.delta_softplus) {
#pragma unroll
        for (int j = 0; j < TS; ++j) dl[j] = softplus_in<In>(dl[j]);
      }
      // steps past the end are the identity (delta = 0)
      if (ts + TS > L) {
#pragma unroll
        for (int j = 0; j < TS; ++j)
          if (ts + j >= L) dl[j] = 0.0f;
      }
#pragma unroll
      for (int j = 0; j < TS; ++j) du[j] = dl[j] * uk[j];
    }
    if (ch + 1 < nchunks) load_chunk(c0 + TC);
    __syncthreads();  // B, C of this chunk staged; last chunk's aggregates read

    // -- 1. the slot from the identity: decays and aggregate ---------------------
    float acache[T][NG], v[NG];
#pragma unroll
    for (int k = 0; k < NG; ++k) v[k] = 0.0f;
    float dsum = 0.0f;
    static_for<0, T>([&](auto tc) {
      constexpr int t = decltype(tc)::value;
      float dt, dut;
      if constexpr (LPC > 1) {
        dt = dpp_f<group_bcast<LPC>(t / TS)>(dl[t % TS]);
        dut = dpp_f<group_bcast<LPC>(t / TS)>(du[t % TS]);
      } else {
        dt = dl[t];
        dut = du[t];
      }
      dsum += dt;
#pragma unroll
      for (int k4 = 0; k4 < NG; k4 += 4) {
        const float4 bq = *reinterpret_cast<const float4*>(&sB[buf][w * T + t][slot * NG + k4]);
        const float bv[4] = {bq.x, bq.y, bq.z, bq.w};
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const float a = fast_exp2(dt * A2[k4 + i]);
          acache[t][k4 + i] = a;
          v[k4 + i] = __builtin_fmaf(a, v[k4 + i], dut * bv[i]);
        }
      }
    });
#pragma unroll
    for (int k = 0; k < NG; ++k)
      sAgg[w][r][slot * NG + k] = make_float2(fast_exp2(A2[k] * dsum), v[k]);
    __syncthreads();  // every slot's aggregate published

    // -- 2. carry-in of this slot and the next chunk's carry ---------------------
    float h[NG];
    for (int s2 = 0; s2 < W; ++s2) {  // (uniform per wave)
      if (s2 == w) {
#pragma unroll
        for (int k = 0; k < NG; ++k) h[k] = carry[k];
      }
#pragma unroll
      for (int k = 0; k < NG; ++k) {
        const float2 g = sAgg[s2][r][slot * NG + k];
        carry[k] = __builtin_fmaf(g.x, carry[k], g.y);
      }
    }

    // -- 3. rescan with the cached decays, read out ------------------------------
    float yp[T];
    static_for<0, T>([&](auto tc) {
      constexpr int t = decltype(tc)::value;
      float dut;
      if constexpr (LPC > 1) dut = dpp_f<group_bcast<LPC>(t / TS)>(du[t % TS]);
      else dut = du[t];
      float acc = 0.0f;
#pragma unroll
      for (int k4 = 0; k4 < NG; k4 += 4) {
        const float4 bq = *reinterpret_cast<const float4*>(&sB[buf][w * T + t][slot * NG + k4]);
        const float4 cq = *reinterpret_cast<const float4*>(&sC[buf][w * T + t][slot * NG + k4]);
        const float bv[4] = {bq.x, bq.y, bq.z, bq.w};
        const float cv[4] = {cq.x, cq.y, cq.z, cq.w};
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          h[k4 + i] = __builtin_fmaf(acache[t][k4 + i], h[k4 + i], dut * bv[i]);
          acc = __builtin_fmaf(cv[i], h[k4 + i], acc);
        }
      }
      yp[t] = acc;
    });

    // -- sum the group's partial readouts onto the owners of the steps ---------
    float yo[TS];
    if constexpr (LPC == 4) {
      float s1[T / 2];
      const bool lo = slot < 2;
#pragma unroll
      for (int j = 0; j < T / 2; ++j) {
        const float keep = lo ? yp[j] : yp[T / 2 + j];
        const float send = lo ? yp[T / 2 + j] : yp[j];
        s1[j] = keep + dpp_f<kSwapHalves>(send);
      }
      const bool ev = (slot & 1) == 0;
#pragma unroll
      for (int j = 0; j < TS; ++j) {
        const float keep = ev ? s1[j] : s1[TS + j];
        const float send = ev ? s1[TS + j] : s1[j];
        yo[j] = keep + dpp_f<kSwapPairs>(send);
      }
    } else if constexpr (LPC == 2) {
      const bool ev = slot == 0;
#pragma unroll
      for (int j = 0; j < TS; ++j) {
        const float keep = ev ? yp[j] : yp[TS + j];
        const float send = ev ? yp[TS + j] : yp[j];
        yo[j] = keep + dpp_f<kSwapPairs>(send);
      }
    } else {
#pragma unroll
      for (int j = 0; j < TS; ++j) yo[j] = yp[j];
    }
#pragma unroll
    for (int j = 0; j < TS; ++j) yo[j] = __builtin_fmaf(Dd, uk[j], yo[j]) * gk[j];
    if (row_ok && y) store_seg<In, TS>(y, row_base, ts, L, yo);
  }
  // -- final state: the carry after the last chunk (steps past the end are
  //    identity steps) -----------------------------------------------------------
  if (prm.last_state && row_ok && w == 0) {
    float* ls = prm.last_state + rowi * N;
#pragma unroll
    for (int k = 0; k < NG; ++k)
      if (slot * NG + k < N) ls[slot * NG + k] = carry[k];
  }
}

// ---- carry-ins of the time segments --------------------------------------------

// One step of the inclusive scan below: combine this lane's (a, v) with the
// pair of the lane CTRL selects (the earlier one, on the left of the combine
// operator of [EXPLAINED] eq. (10)); lanes without a source, or outside
// ROW_MASK, take the identity (1, 0).
template <int CTRL, int ROW_MASK, int K>
__device__ __forceinline__ void scan_step(float (&a)[K], float (&v)[K]) {
#pragma unroll
  for (int k = 0; k < K; ++k) {
    const float ap = __int_as_float(__builtin_amdgcn_update_dpp(
        __float_as_int(1.0f), __float_as_int(a[k]), CTRL, ROW_MASK, 0xF, false));
    const float vp = __int_as_float(__builtin_amdgcn_update_dpp(
        0, __float_as_int(v[k]), CTRL, ROW_MASK, 0xF, false));
    v[k] = __builtin_fmaf(a[k], vp, v[k]);  // (ap, vp) (+) (a, v) = (a ap, a vp + v)
    a[k] *= ap;
  }
}

// Inclusive scans of K independent sequences of (a, v) pairs, each over
// 16 RPP consecutive lanes (RPP = 1, 2 or 4 16-lane rows), lane order =
// sequence order ([EXPLAINED] eqs. (10)-(12) and the doubling prefix-sum
// figure): four doubling steps inside each 16-lane row (DPP row_shr by 1,
// 2, 4, 8); for RPP >= 2 the totals of rows 0 and 2 are combined into rows
// 1 and 3 (row_bcast:15), and for RPP = 4 the total of rows 0-1 into rows
// 2-3 (row_bcast:31).  So a wave holds 4 / RPP sequences side by side, and
// the K scans are interleaved so that their dependent chains overlap.
template <int RPP, int K>
__device__ __forceinline__ void wave_inclusive_scan(float (&a)[K], float (&v)[K]) {
  scan_step<0x111, 0xF>(a, v);
  scan_step<0x112, 0xF>(a, v);
  scan_step<0x114, 0xF>(a, v);
  scan_step<0x118, 0xF>(a, v);
  if constexpr (RPP >= 2) scan_step<0x142, 0xA>(a, v);
  if constexpr (RPP == 4) scan_step<0x143, 0xC>(a, v);
}

// Carry-ins of the time segments from their aggregates.  slots[s][pair]
// holds (prod a, v) of one segment per (row, state) pair, nslots <= 64 of
// them; on return its v part holds the state entering the neighbouring
// segment: the exclusive combine-scan of the aggregates, started from
// init[pair] (or zero).
//   REV = false (forward scan): slot s holds segment s's aggregate and gets
//     the carry-in of segment s + 1 = init (+) agg_0 (+) ... (+) agg_s.
//   REV = true (adjoint, scanned from the right): slot s holds the
//     aggregate of segment s + 1 and gets the adjoint entering segment s
//     from the right = init (+) agg_{nslots} (+) ... (+) agg_{s+1}.
// With nslots <= 16 RPP, a pair's slots take 16 RPP lanes (lane = slot), so
// one wave scan covers 4 / RPP pairs, and a workgroup takes PB = 16 pairs
// per wave scan width (16, 32 or 64 pairs): it stages their slots in LDS
// with loads of PB * 8 contiguous bytes per segment (all issued before any
// is used), each wave runs 4 interleaved scans, and the carries go back
// with stores of the same shape.  (Small workgroups: the pass is a few
// microseconds of latency, and more workgroups overlap more of it.)
template <bool REV, int RPP>
__global__ void __launch_bounds__(256) segment_carry_kernel(float2* __restrict__ slots, int nslots,
                                                          int64_t npairs,
                                                          const float* __restrict__ init) {
  SSM_POISON_LDS_AT_ENTRY();
  constexpr int SL = 16 * RPP;         // lanes (slots) per pair
  constexpr int PPS = 4 / RPP;         // pairs per wave scan
  constexpr int ILP = 4;               // interleaved scans per wave
  constexpr int PB = 4 * PPS * ILP;    // pairs per workgroup
  constexpr int PER = SL * PB / 256;   // staged entries per thread
  __shared__ float2 tile[SL][PB + 1];
  __shared__ float sInit[PB];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int64_t p0 = (int64_t)blockIdx.x * PB;
  const int np = (int)min<int64_t>(PB, npairs - p0);
  float2 ld[PER];
#pragma unroll
  for (int i = 0; i < PER; ++i) {  // clamped indices, no condition on the loads
    const int e = tid + 256 * i;
    const int s = min(e / PB, nslots - 1), p = min(e % PB, np - 1);
    ld[i] = slots[(int64_t)s * npairs + p0 + p];
  }
  if (tid < PB) sInit[tid] = init ? init[p0 + min(tid, np - 1)] : 0.0f;
#pragma unroll
  for (int i = 0; i < PER; ++i) {
    const int e = tid + 256 * i;
    if (e / PB < nslots) tile[e / PB][e % PB] = ld[i];
  }
  __syncthreads();
  const int sub = lane / SL;                      // pair of the scan this lane is in
  const int sl = lane % SL;
  const int s = REV ? nslots - 1 - sl : sl;       // this lane's slot
  const bool on = sl < nslots;
  float a[ILP], v[ILP];
#pragma unroll
  for (int k = 0; k < ILP; ++k) {
    const int p = (wv * ILP + k) * PPS + sub;     // pairs past np compute on stale entries, unused
    const float2 g = tile[on ? s : 0][p];
    a[k] = on ? g.x : 1.0f;
    v[k] = on ? g.y : 0.0f;
  }
  wave_inclusive_scan<RPP>(a, v);
#pragma unroll
  for (int k = 0; k < ILP; ++k) {
    const int p = (wv * ILP + k) * PPS + sub;
    if (on && p < np) tile[s][p].y = __builtin_fmaf(a[k], sInit[p], v[k]);
  }
  __syncthreads();
  for (int e = tid; e < nslots * PB; e += 256) {
    const int s2 = e / PB, p = e % PB;
    if (p < np) slots[(int64_t)s2 * npairs + p0 + p] = tile[s2][p];
  }
}

// ---- time-split kernel -------------------------------------------------------

// NG: states per wave; G: waves splitting the states; W (> 1): time slots
// per chunk; T: steps per slot.  Block = 64 * G * W threads.
template <typename In, int NG, int G, int W, int T>
__global__ void __launch_bounds__(64 * G * W)
selective_scan_split_kernel(ScanParams prm) {
  SSM_POISON_LDS_AT_ENTRY();
  static_assert(W > 1, "the row-parallel kernel covers W = 1");
  constexpr int NT = NG * G;       // states covered by one workgroup (>= dstate)
  constexpr int TC = W * T;        // steps per chunk
  constexpr int TG = T / G;        // steps of a slot whose per-step work one wave owns
  constexpr int NTHR = 64 * G * W;
  static_assert(T % G == 0, "T must be a multiple of G");
  constexpr int PAIRS = (NT + G * W - 1) / (G * W);  // scan pairs per thread (W > 1)
  // B/C staging: 16-byte units, NT rows x UPR units per tensor and chunk.
  constexpr int EPU = Elem<In>::kPer16B;             // elements per unit
  static_assert(TC % EPU == 0, "chunk must hold whole 16-byte units");
  constexpr int UPR = TC / EPU;
  constexpr int UNITS = 2 * NT * UPR;
  constexpr int RB = (UNITS + NTHR - 1) / NTHR;      // units per thread

  __shared__ alignas(16) float sB[TC][NT];
  __shared__ alignas(16) float sC[TC][NT];
  __shared__ float2 sDD[W][T][64];                  // (delta, delta*u) per step and row
  __shared__ float sP[W > 1 ? W : 1][W > 1 ? NT : 1][64];   // slot decay products
  __shared__ float sV[W > 1 ? W : 1][W > 1 ? NT : 1][64];   // slot values / carry-ins
  __shared__ float sY[G > 1 ? G : 1][G > 1 ? W : 1][G > 1 ? T : 1][64];  // partial readouts

  const In* __restrict__ u = static_cast<const In*>(prm.u);
  const In* __restrict__ dlt = static_cast<const In*>(prm.delta);
  const In* __restrict__ Bm = static_cast<const In*>(prm.B);
  const In* __restrict__ Cm = static_cast<const In*>(prm.C);
  const In* __restrict__ z = static_cast<const In*>(prm.z);
  In* __restrict__ y = static_cast<In*>(prm.y);

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int g = wv % G;
  const int w = wv / G;
  const int b = blockIdx.y;
  const int d = blockIdx.x * 64 + lane;
  const bool row_ok = d < prm.dim;
  const bool has_z = z != nullptr;
  const int L = prm.seqlen;
  const int N = prm.dstate;
  const int64_t row_base = ((int64_t)b * prm.dim + (row_ok ? d : 0)) * (int64_t)L;
  // B, C of the group of the workgroup's rows: [batch, ngroups, dstate, seqlen]
  const int grp = (int)(blockIdx.x * 64) / (prm.dim / prm.ngroups);
  const int64_t bc_base = ((int64_t)b * prm.ngroups + grp) * N * (int64_t)L;

  // Per-row constants for this wave's states.
  float A2[NG];
#pragma unroll
  for (int k = 0; k < NG; ++k) {
    const int n = g * NG + k;
    A2[k] = (row_ok && n < N) ? prm.A[(int64_t)d * N + n] * kLog2e : 0.0f;
  }
  const float Dd = (row_ok && prm.D) ? prm.D[d] : 0.0f;
  const float bias = (row_ok && prm.delta_bias) ? prm.delta_bias[d] : 0.0f;

  float h[NG];
#pragma unroll
  for (int k = 0; k < NG; ++k) h[k] = 0.0f;
  // Running carry per (state, row) pair this thread folds: starts at the
  // initial state v_0 of [EXPLAINED] eqs. (8)-(9) when given.
  float carry[PAIRS];
#pragma unroll
  for (int q = 0; q < PAIRS; ++q) {
    const int n = wv + q * (G * W);
    carry[q] = (prm.h0 && row_ok && n < N) ? prm.h0[((int64_t)b * prm.dim + d) * N + n] : 0.0f;
  }

  // Raw chunk data, loaded one chunk ahead of its use.
  RawSeg<In, TG> ru, rd, rz;
  RawSeg<In, EPU> rbc[RB];
  auto load_chunk = [&](int c0) {
    const int ts = c0 + w * T + g * TG;
    if (row_ok) {
      load_raw<In, TG>(u, row_base, ts, L, ru);
      load_raw<In, TG>(dlt, row_base, ts, L, rd);
      if (has_z) load_raw<In, TG>(z, row_base, ts, L, rz);
    }
#pragma unroll
    for (int q = 0; q < RB; ++q) {
      const int e = tid + q * NTHR;
      const int n = e % NT, rest = e / NT;
      const int seg = rest % UPR, x = rest / UPR;
      if (e < UNITS && n < N) {
        const In* src = x ? Cm : Bm;
        load_raw<In, EPU>(src, bc_base + (int64_t)n * L, c0 + seg * EPU, L, rbc[q]);
      } else {
#pragma unroll
        for (int k = 0; k < RawSeg<In, EPU>::kWords; ++k) rbc[q].w[k] = 0u;
      }
    }
  };

  const int nchunks = (L + TC - 1) / TC;
  load_chunk(0);
  for (int ch = 0; ch < nchunks; ++ch) {
    const int c0 = ch * TC;
    if (G == 1) __syncthreads();  // previous chunk's LDS readers are done

    // -- decode: B and C into LDS as float32 [t][n] --------------------------
#pragma unroll
    for (int q = 0; q < RB; ++q) {
      const int e = tid + q * NTHR;
      if (e < UNITS) {
        const int n = e % NT, rest = e / NT;
        const int seg = rest % UPR, x = rest / UPR;
        float v[EPU];
        decode_raw<In, EPU>(rbc[q], v);
#pragma unroll
        for (int i = 0; i < EPU; ++i) {
          if (x) sC[seg * EPU + i][n] = v[i];
          else sB[seg * EPU + i][n] = v[i];
        }
      }
    }
    // -- decode: per-step work for this wave's share of its slot ------------
    const int ts = c0 + w * T + g * TG;  // first step owned by this wave
    float uk[TG], gk[TG];
    {
      float dr[TG];
      decode_raw<In, TG>(ru, uk);
      decode_raw<In, TG>(rd, dr);
      if (has_z) {
        float zk[TG];
        decode_raw<In, TG>(rz, zk);
#pragma unroll
        for (int j = 0; j < TG; ++j) gk[j] = silu_f(zk[j]);
      } else {
#pragma unroll
        for (int j = 0; j < TG; ++j) gk[j] = 1.0f;
      }
      // Steps past the end are the identity (delta = 0).  Rows past `dim`
      // compute on zeros and are never stored, so they need no mask.
      const bool tail = ts + TG > L;
#pragma unroll
      for (int j = 0; j < TG; ++j) {
        float dl = dr[j] + bias;
        if (prm.delta_softplus) dl = softplus_f(dl);
        if (tail && ts + j >= L) dl = 0.0f;
        sDD[w][g * TG + j][lane] = make_float2(dl, dl * uk[j]);
      }
    }
    if (ch + 1 < nchunks) load_chunk(c0 + TC);
    __syncthreads();

    // -- recurrence over this wave's slot and states --------------------------
    float yp[T];
#pragma unroll
    for (int j = 0; j < T; ++j) yp[j] = 0.0f;

    {
      // Pass 1: slot aggregate from the identity (1, 0).
      float acache[T][NG];
      float v[NG];
#pragma unroll
      for (int k = 0; k < NG; ++k) v[k] = 0.0f;
      float dsum = 0.0f;
#pragma unroll
      for (int j = 0; j < T; ++j) {
        const float2 dd = sDD[w][j][lane];
        dsum += dd.x;
#pragma unroll
        for (int k = 0; k < NG; ++k) {
          const float a = fast_exp2(dd.x * A2[k]);
          acache[j][k] = a;
          v[k] = __builtin_fmaf(a, v[k], dd.y * sB[w * T + j][g * NG + k]);
        }
      }
#pragma unroll
      for (int k = 0; k < NG; ++k) {
        sP[w][g * NG + k][lane] = fast_exp2(A2[k] * dsum);
        sV[w][g * NG + k][lane] = v[k];
      }
      __syncthreads();
      // Serial combine over the W slots for the (state, row) pairs this
      // thread owns: carry-in of slot s = carry (+) slot_0 (+) ... (+) slot_{s-1}.
#pragma unroll
      for (int q = 0; q < PAIRS; ++q) {
        const int n = wv + q * (G * W);
        if (n < NT) {
          float c = carry[q];
#pragma unroll
          for (int s = 0; s < W; ++s) {
            const float p = sP[s][n][lane];
            const float vv = sV[s][n][lane];
            sV[s][n][lane] = c;
            c = __builtin_fmaf(p, c, vv);
          }
          carry[q] = c;
        }
      }
      __syncthreads();
      // Pass 2: rescan the slot from its carry-in and read out y.
#pragma unroll
      for (int k = 0; k < NG; ++k) h[k] = sV[w][g * NG + k][lane];
#pragma unroll
      for (int j = 0; j < T; ++j) {
        const float2 dd = sDD[w][j][lane];
#pragma unroll
        for (int k = 0; k < NG; ++k) {
          h[k] = __builtin_fmaf(acache[j][k], h[k], dd.y * sB[w * T + j][g * NG + k]);
          yp[j] = __builtin_fmaf(sC[w * T + j][g * NG + k], h[k], yp[j]);
        }
      }
    }

    // -- combine the state groups' readouts, skip term, gate, store ----------
    float yo[TG];
    if constexpr (G > 1) {
#pragma unroll
      for (int j = 0; j < T; ++j) sY[g][w][j][lane] = yp[j];
      __syncthreads();
#pragma unroll
      for (int j = 0; j < TG; ++j) {
        float acc = 0.0f;
#pragma unroll
        for (int gg = 0; gg < G; ++gg) acc += sY[gg][w][g * TG + j][lane];
        yo[j] = acc;
      }
    } else {
#pragma unroll
      for (int j = 0; j < TG; ++j) yo[j] = yp[j];
    }
#pragma unroll
    for (int j = 0; j < TG; ++j) yo[j] = __builtin_fmaf(Dd, uk[j], yo[j]) * gk[j];
    if (row_ok) store_seg<In, TG>(y, row_base, ts, L, yo);
  }

  // -- final state -----------------------------------------------------------
  if (prm.last_state && row_ok) {
    float* ls = prm.last_state + ((int64_t)b * prm.dim + d) * N;
#pragma unroll
    for (int q = 0; q < PAIRS; ++q) {
      const int n = wv + q * (G * W);
      if (n < N) ls[n] = carry[q];
    }
  }
}

// Time chunk of the row-parallel kernel for 9..16 states over whole rows:
// the four lanes of a row then read whole 128-byte lines of u, delta, z and
// write whole lines of y per chunk (64 bf16 or 32 float32 steps), and
// float32 rows stay at 140 VGPRs (three waves per SIMD; 1.4B shape in
// float32: 403 -> 362 us against 64-step chunks).
template <typename In>
constexpr int t16_rows() { return sizeof(In) == 4 ? 32 : 64; }

// Time chunk of the row-parallel kernel for 9..16 states when the sequence
// is cut into segments: segments are a few chunks long, and 32-step chunks
// keep the kernel at 140 (float32) / 128 (bf16) VGPRs, so three or four
// waves fit per SIMD (64-step chunks: 228 / 196, two waves).
constexpr int kTSeg16 = 32;

template <typename In, int NG, int LPC, int T, bool AGG = false>
hipError_t launch_rows(const ScanParams& p, hipStream_t stream, int nz = 1) {
  constexpr int RPB = 4 * (64 / LPC);
  dim3 grid((unsigned)((p.dim + RPB - 1) / RPB), (unsigned)p.batch, (unsigned)nz);
  hipLaunchKernelGGL((selective_scan_fwd_kernel<In, NG, LPC, T, AGG>), grid, dim3(256), 0,
                     stream, p);
  return hipGetLastError();
}

template <typename In, int NG, int G, int W, int T>
hipError_t launch_cfg(const ScanParams& p, hipStream_t stream) {
  dim3 grid((unsigned)((p.dim + 63) / 64), (unsigned)p.batch);
  dim3 block(64 * G * W);
  hipLaunchKernelGGL((selective_scan_split_kernel<In, NG, G, W, T>), grid, block, 0, stream, p);
  return hipGetLastError();
}

template <typename In, int NG, int LPC, int T, int W>
hipError_t launch_slot(const ScanParams& p, hipStream_t stream) {
  constexpr int RPB = 64 / LPC;
  dim3 grid((unsigned)((p.dim + RPB - 1) / RPB), (unsigned)p.batch);
  hipLaunchKernelGGL((selective_scan_slot_kernel<In, NG, LPC, T, W>), grid, dim3(64 * W), 0,
                     stream, p);
  return hipGetLastError();
}

template <typename In>
hipError_t launch_typed(const ScanParams& p, const ScanTile& t, hipStream_t s) {
  switch (t.id) {
    case ScanTileId::kN4_Seq: return launch_rows<In, 4, 1, 16>(p, s);
    case ScanTileId::kN8_Seq: return launch_rows<In, 4, 2, 32>(p, s);
    case ScanTileId::kN16_Seq: return launch_rows<In, 4, 4, t16_rows<In>()>(p, s);
    case ScanTileId::kN64_Seq: return launch_rows<In, 16, 4, 32>(p, s);
    case ScanTileId::kN4_Split: return launch_cfg<In, 4, 1, 8, 8>(p, s);
    case ScanTileId::kN8_Split: return launch_cfg<In, 4, 2, 4, 16>(p, s);
    case ScanTileId::kN16_Split: return launch_cfg<In, 4, 4, 2, 32>(p, s);
    case ScanTileId::kN64_Split: return launch_cfg<In, 16, 4, 2, 4>(p, s);
    case ScanTileId::kN4_Slot: return launch_slot<In, 4, 1, 16, 8>(p, s);
    case ScanTileId::kN8_Slot: return launch_slot<In, 4, 2, 16, 8>(p, s);
    case ScanTileId::kN16_Slot: return launch_slot<In, 4, 4, 16, 8>(p, s);
  }
  return hipErrorInvalidValue;
}

// Scratch of the no-allocation entry point (the time-split aggregates).
// Every GPU the library runs on holds its own copy until the process ends.
// Host code must not pass this name to a kernel: it is a host-side stand-in
// for the symbol; the device address comes from scan_scratch_address().
__device__ __align__(256) unsigned char scratch[kNoAllocScratchBytes];

}  // namespace

hipError_t scan_scratch_address(void** out) {
  return hipGetSymbolAddress(out, HIP_SYMBOL(scratch));
}

// Row-parallel shape per dstate tier: (NG, LPC, T) = (4,1,16) / (4,2,32) /
// (4,4,64) / (16,4,32) for dstate <= 4 / 8 / 16 / 64.
template <typename In, bool AGG>
hipError_t launch_rows_tier(const ScanParams& p, hipStream_t s, int nz) {
  if (p.dstate <= 4) return launch_rows<In, 4, 1, 16, AGG>(p, s, nz);
  if (p.dstate <= 8) return launch_rows<In, 4, 2, 32, AGG>(p, s, nz);
  if (p.dstate <= 16) return launch_rows<In, 4, 4, kTSeg16, AGG>(p, s, nz);
  return launch_rows<In, 16, 4, 32, AGG>(p, s, nz);
}

template <bool REV, int RPP>
void launch_carry_rpp(float2* slots, int nslots, int64_t npairs, const float* init,
                      hipStream_t stream) {
  constexpr int PB = 64 / RPP;  // pairs per workgroup (as in the kernel)
  hipLaunchKernelGGL((segment_carry_kernel<REV, RPP>), dim3((unsigned)((npairs + PB - 1) / PB)),
                     dim3(256), 0, stream, slots, nslots, npairs, init);
}

template <bool REV>
void launch_carry(float2* slots, int nslots, int64_t npairs, const float* init,
                  hipStream_t stream) {
  if (nslots <= 16) launch_carry_rpp<REV, 1>(slots, nslots, npairs, init, stream);
  else if (nslots <= 32) launch_carry_rpp<REV, 2>(slots, nslots, npairs, init, stream);
  else launch_carry_rpp<REV, 4>(slots, nslots, npairs, init, stream);
}

hipError_t launch_segment_carry(float* slots, int nslots, int64_t npairs, const float* init,
                                bool reverse, hipStream_t stream) {
  if (nslots < 1 || nslots > 64) return hipErrorInvalidValue;
  float2* s2 = reinterpret_cast<float2*>(slots);
  if (reverse) launch_carry<true>(s2, nslots, npairs, init, stream);
  else launch_carry<false>(s2, nslots, npairs, init, stream);
  return hipGetLastError();
}

hipError_t launch_selective_scan_carries(const ScanParams& p, bool bf16, hipStream_t stream) {
  // every segment but the last scanned from the identity (its aggregate into
  // p.seg_agg), then the combine scan of the aggregates in place
  const int nz = (p.seqlen + p.seg_len - 1) / p.seg_len;
  if (nz <= 1) return hipSuccess;
  hipError_t e = bf16 ? launch_rows_tier<uint16_t, true>(p, stream, nz - 1)
                      : launch_rows_tier<float, true>(p, stream, nz - 1);
  if (e != hipSuccess) return e;
  return launch_segment_carry(p.seg_agg, nz - 1, (int64_t)p.batch * p.dim * p.dstate, p.h0, false,
                              stream);
}

hipError_t launch_selective_scan(const ScanParams& p, const ScanTile& tile, bool bf16,
                                 hipStream_t stream) {
  return bf16 ? launch_typed<uint16_t>(p, tile, stream) : launch_typed<float>(p, tile, stream);
}

ScanSegments plan_scan_segments(int64_t batch, int64_t dim, int64_t dstate, int64_t seqlen,
                                int num_cus) {
  const int lpc = dstate <= 4 ? 1 : dstate <= 8 ? 2 : 4;
  const int T = dstate <= 4 ? 16 : dstate <= 8 ? 32 : dstate <= 16 ? kTSeg16 : 32;
  const int rpb = 256 / lpc;
  ScanSegments sg{1, 0, rpb, 0};
  // Split only when the rows leave SIMDs without a wave (the aggregate pass
  // costs about half a scan of the segments it covers) and the sequence has
  // at least 8 chunks; aim at three waves per SIMD, the most that stay
  // resident together (measured at the 130M shape, float32: 67.5 / 66.3 /
  // 69.3 us for two, three, four; 75.2 us with 64-step chunks at four).
  const int64_t cus = num_cus > 0 ? num_cus : 256;
  const int64_t waves = batch * ((dim + rpb - 1) / rpb) * 4;
  const int64_t target = 12 * cus;
  const int64_t chunks = (seqlen + T - 1) / T;
  if (waves >= 4 * cus || chunks < 8) return sg;
  const int64_t want = std::min<int64_t>({(target + waves - 1) / waves, chunks, 64});
  if (want <= 1) return sg;
  const int64_t seg_len = ((seqlen + want - 1) / want + T - 1) / T * T;
  const int64_t nseg = (seqlen + seg_len - 1) / seg_len;
  if (nseg <= 1) return sg;
  sg.nseg = (int)nseg;
  sg.seg_len = (int)seg_len;
  sg.bytes = (size_t)(nseg - 1) * (size_t)batch * (size_t)dim * (size_t)dstate * 2 * sizeof(float);
  return sg;
}

hipError_t launch_selective_scan_segmented(const ScanParams& p0, const ScanSegments& sg, bool bf16,
                                           hipStream_t stream) {
  ScanParams p = p0;
  p.seg_len = sg.seg_len;
  hipError_t e = bf16 ? launch_rows_tier<uint16_t, true>(p, stream, sg.nseg - 1)
                      : launch_rows_tier<float, true>(p, stream, sg.nseg - 1);
  if (e != hipSuccess) return e;
  e = launch_segment_carry(p.seg_agg, sg.nseg - 1, (int64_t)p.batch * p.dim * p.dstate, p.h0,
                           false, stream);
  if (e != hipSuccess) return e;
  return bf16 ? launch_rows_tier<uint16_t, false>(p, stream, sg.nseg)
              : launch_rows_tier<float, false>(p, stream, sg.nseg);
}

int scan_tile_rows(const ScanTile& tile) {
  switch (tile.id) {
    case ScanTileId::kN4_Seq: return 256;
    case ScanTileId::kN8_Seq: return 128;
    case ScanTileId::kN16_Seq: case ScanTileId::kN64_Seq: return 64;
    case ScanTileId::kN4_Slot: return 64;
    case ScanTileId::kN8_Slot: return 32;
    case ScanTileId::kN16_Slot: return 16;
    default: return 64;  // time-split kernels: 64 rows per workgroup
  }
}

// Per-row B and C, one state per lane: 16 lanes per row up to 16 states
// (selective_scan_chan_kernel), else S = 32 or 64 lanes per row
// (selective_scan_chanw_kernel).  nz > 1: one z slice per time segment.
template <typename In, bool AGG = false>
hipError_t launch_chan(const ScanParams& p, hipStream_t stream, int nz = 1) {
  dim3 grid((unsigned)((p.dim + 15) / 16), (unsigned)p.batch, (unsigned)nz);
  constexpr int kVec = sizeof(In) == 4 ? kChanLoadSpread : kChanLoadAfter;
  if (p.seqlen % Elem<In>::kPer16B == 0)
    hipLaunchKernelGGL((selective_scan_chan_kernel<In, kVec, AGG>), grid, dim3(256), 0, stream, p);
  else
    hipLaunchKernelGGL((selective_scan_chan_kernel<In, kChanLoadElem, AGG>), grid, dim3(256), 0,
                       stream, p);
  return hipGetLastError();
}

template <typename In, int S, bool AGG = false>
hipError_t launch_chanw(const ScanParams& p, hipStream_t stream, int nz = 1) {
  dim3 grid((unsigned)((p.dim + 4 * (64 / S) - 1) / (4 * (64 / S))), (unsigned)p.batch,
            (unsigned)nz);
  constexpr int kVec = sizeof(In) == 4 ? kChanLoadSpread : kChanLoadAfter;
  if (p.seqlen % Elem<In>::kPer16B == 0)
    hipLaunchKernelGGL((selective_scan_chanw_kernel<In, S, kVec, AGG>), grid, dim3(256), 0, stream,
                       p);
  else
    hipLaunchKernelGGL((selective_scan_chanw_kernel<In, S, kChanLoadElem, AGG>), grid, dim3(256),
                       0, stream, p);
  return hipGetLastError();
}

// Per-row B, C kernel by dstate: one state per lane, 16 / 32 / 64 lanes per row.
template <typename In, bool AGG>
hipError_t launch_rowbc_typed(const ScanParams& p, hipStream_t stream, int nz) {
  if (p.dstate <= 16) return launch_chan<In, AGG>(p, stream, nz);
  if (p.dstate <= 32) return launch_chanw<In, 32, AGG>(p, stream, nz);
  return launch_chanw<In, 64, AGG>(p, stream, nz);
}

hipError_t launch_selective_scan_rowbc(const ScanParams& p, bool bf16, hipStream_t stream) {
  // up to 16 states: one state per lane, whole 128-byte lines of B and C
  // (per channel at the 1.4B shape, bf16 / f32: 16 states 2.50 / 5.21 ->
  // 1.2 / 2.9 ms against four states per lane and 32-byte pieces; 4 states
  // 0.95 / 2.13 -> 0.59 / 0.80 ms; 1 state 0.48 / 1.27 -> 0.52 / 0.56 ms)
  return bf16 ? launch_rowbc_typed<uint16_t, false>(p, stream, 1)
              : launch_rowbc_typed<float, false>(p, stream, 1);
}

ScanSegments plan_scan_segments_rowbc(int64_t batch, int64_t dim, int64_t dstate, int64_t seqlen,
                                      int num_cus) {
  // rows per wave of the per-row kernels; segments are whole 64-step chunks
  // (a multiple of both chunk lengths, 64 bf16 and 32 float32 steps).
  // Split only below one wave per CU: the aggregate pass reads B a second
  // time, which these kernels feel (per channel, float32: batch 1, dim 256,
  // 64 waves 177 -> 41 us split; batch 2, dim 1536, 768 waves 267 -> 426 us).
  const int rpw = dstate <= 16 ? 4 : dstate <= 32 ? 2 : 1;
  constexpr int kSegUnit = 64;
  ScanSegments sg{1, 0, 4 * rpw, 0};
  const int64_t cus = num_cus > 0 ? num_cus : 256;
  const int64_t waves = batch * ((dim + rpw - 1) / rpw);
  const int64_t target = 12 * cus;
  const int64_t units = (seqlen + kSegUnit - 1) / kSegUnit;
  if (waves > cus || units < 8) return sg;
  const int64_t want = std::min<int64_t>({(target + waves - 1) / waves, units, 64});
  if (want <= 1) return sg;
  const int64_t seg_len = ((seqlen + want - 1) / want + kSegUnit - 1) / kSegUnit * kSegUnit;
  const int64_t nseg = (seqlen + seg_len - 1) / seg_len;
  if (nseg <= 1) return sg;
  sg.nseg = (int)nseg;
  sg.seg_len = (int)seg_len;
  sg.bytes = (size_t)(nseg - 1) * (size_t)batch * (size_t)dim * (size_t)dstate * 2 * sizeof(float);
  return sg;
}

hipError_t launch_selective_scan_rowbc_carries(const ScanParams& p, bool bf16, hipStream_t stream) {
  // every segment but the last scanned from the identity by the per-row
  // kernels (aggregates into p.seg_agg), then the combine scan in place
  const int nz = (p.seqlen + p.seg_len - 1) / p.seg_len;
  if (nz <= 1) return hipSuccess;
  hipError_t e = bf16 ? launch_rowbc_typed<uint16_t, true>(p, stream, nz - 1)
                      : launch_rowbc_typed<float, true>(p, stream, nz - 1);
  if (e != hipSuccess) return e;
  return launch_segment_carry(p.seg_agg, nz - 1, (int64_t)p.batch * p.dim * p.dstate, p.h0, false,
                              stream);
}

hipError_t launch_selective_scan_rowbc_segmented(const ScanParams& p0, const ScanSegments& sg,
                                                 bool bf16, hipStream_t stream) {
  ScanParams p = p0;
  p.seg_len = sg.seg_len;
  hipError_t e = bf16 ? launch_rowbc_typed<uint16_t, true>(p, stream, sg.nseg - 1)
                      : launch_rowbc_typed<float, true>(p, stream, sg.nseg - 1);
  if (e != hipSuccess) return e;
  e = launch_segment_carry(p.seg_agg, sg.nseg - 1, (int64_t)p.batch * p.dim * p.dstate, p.h0,
                           false, stream);
  if (e != hipSuccess) return e;
  return bf16 ? launch_rowbc_typed<uint16_t, false>(p, stream, sg.nseg)
              : launch_rowbc_typed<float, false>(p, stream, sg.nseg);
}

}  // namespace ssm
