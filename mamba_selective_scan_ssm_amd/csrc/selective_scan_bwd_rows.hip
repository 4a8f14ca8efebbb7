// selective_scan_bwd_rows.hip -- Mamba-1 backward pass with B and C read per
// row (groups of channels smaller than a workgroup of the shared-B/C
// backward kernels, down to one channel per group), for gfx950.
//
// Sources (web pages; cited by title and section/equation):
//   [SPEC]      "ТЕХНИЧЕСКОЕ ЗАДАНИЕ: Реализовать selective scan (Mamba)",
//               Stage 1 items 3-4 (forward: softplus, D skip, silu gate), its
//               backward-pass stage, and its reference kernel's per-channel
//               B and C.
//   [EXPLAINED] "Mamba CUDA 实现解析", eqs. (5)-(7) (the recurrence being
//               differentiated).
//
// The same reverse-mode rules as the shared-B/C backward (per row, per
// state n, t descending; lam = dL/dh_t):
//   dyh_t = dy_t silu(z_t);  dz_t = dy_t yh_t silu'(z_t);  dD += dyh_t u_t
//   lam  = C_t dyh_t + a_{t+1} lam;  dC_t = dyh_t h_t;  dB_t = lam delta_t u_t
//   du_t = dyh_t D + delta_t sum_n lam B_t;  dA += lam delta_t a_t h_{t-1}
//   ddelta_t = (sum_n lam A a_t h_{t-1} + u_t sum_n lam B_t) softplus'
//   dh0 = a_0 lam_0.
// Layout: one state per lane, a row's states over S = 16, 32 or 64 lanes of
// one wave (64 / S rows per wave; a workgroup is one wave, so there is no
// cross-wave barrier), B and C of each lane's own state read as whole
// pieces of its row per chunk.  Per-step values of a row (delta, delta*u,
// dyh, softplus') are formed by the lane that owns the step and shared
// through LDS; per-step sums over the row's states go through LDS to the
// owner.  One kernel runs the forward sweep (saving the state entering every
// chunk, dz, dD and dC) and then the reverse sweep over the chunks (the
// chunk's a_t h_{t-1} recomputed from its saved entry state; du, ddelta, dA,
// dB, dinitial_state).  dA, dD and ddelta_bias are summed over the batch by
// a second kernel in a fixed order; with groups of more than one channel,
// dB and dC are written per row and a third kernel adds each group's rows.
// Rows too few to fill the device cut the sequence into time segments
// ([EXPLAINED] eqs. (10)-(11)): the forward's carry-ins come from the
// per-row forward kernels' aggregate pass and the combine scan, the
// adjoint's from bwd_rows_lam_agg_kernel and the same scan run from the
// right, and every segment is then a workgroup of its own.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <algorithm>

#include "device_math.h"
#include "scan_common.h"
#include "selective_scan_launch.h"

namespace ssm {
namespace {

using namespace scan;

constexpr int kRowsBwdT = 32;  // steps per chunk

size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

// Workspace: [rows][dstate][chunks] saved states; [segments][batch][dim]
// [dstate] dA partials; [segments][2][batch][dim] dD and ddelta_bias
// partials; with more than one channel per group, [2][rows][dstate][seqlen]
// per-row dB and dC; with a time split, the forward's and the adjoint's
// segment aggregates, [segments - 1][rows][dstate][2] each.
struct RowsBwdLayout {
  size_t ck_off, pa_off, pd_off, rb_off, fwd_agg_off, lam_agg_off, total;
  int nck, nseg, seg_len;
};

RowsBwdLayout rows_bwd_layout(int batch, int dim, int dstate, int seqlen, int ngroups,
                              int num_cus) {
  RowsBwdLayout l;
  l.nck = (seqlen + kRowsBwdT - 1) / kRowsBwdT;
  // Time segments (whole 64-step units: the forward kernels' chunks) when
  // the one-wave workgroups number at most one per CU and the sequence has
  // at least 8 units; aim at eight waves per CU, two per SIMD, the kernel's
  // occupancy.  (Per channel, float32, dim 256, 2048 steps: 0.43 -> 0.13 ms
  // split; batch 2, dim 1536, three waves per CU: 0.79 ms unsplit against
  // 1.04 ms split in three.)
  const int rpw = dstate <= 16 ? 4 : dstate <= 32 ? 2 : 1;
  const int64_t cus = num_cus > 0 ? num_cus : 256;
  const int64_t waves = (int64_t)batch * ((dim + rpw - 1) / rpw);
  const int64_t units = (seqlen + 63) / 64;
  l.nseg = 1;
  l.seg_len = 0;
  if (waves <= cus && units >= 8) {
    const int64_t want = std::min<int64_t>({(8 * cus + waves - 1) / waves, units, 64});
    const int64_t seg_len = ((seqlen + want - 1) / want + 63) / 64 * 64;
    const int64_t nseg = (seqlen + seg_len - 1) / seg_len;
    if (nseg > 1) {
      l.nseg = (int)nseg;
      l.seg_len = (int)seg_len;
    }
  }
  const size_t rows = (size_t)batch * dim;
  const size_t aggs = (size_t)(l.nseg - 1) * rows * dstate * 2 * sizeof(float);
  size_t o = 0;
  l.ck_off = o; o = align256(o + rows * dstate * l.nck * sizeof(float));
  l.pa_off = o; o = align256(o + (size_t)l.nseg * rows * dstate * sizeof(float));
  l.pd_off = o; o = align256(o + (size_t)l.nseg * 2 * rows * sizeof(float));
  l.rb_off = o;
  if (dim / ngroups > 1) o = align256(o + 2 * rows * dstate * (size_t)seqlen * sizeof(float));
  l.fwd_agg_off = o; o = align256(o + aggs);
  l.lam_agg_off = o; o = align256(o + aggs);
  l.total = o;
  return l;
}

template <typename In, int S>
__global__ void __launch_bounds__(64) bwd_rows_kernel(BwdParams P, RowsBwdLayout lay) {
  SSM_POISON_LDS_AT_ENTRY();
  constexpr int T = kRowsBwdT;
  constexpr int RPW = 64 / S;                 // rows per wave (= workgroup)
  constexpr int NOWN = (T + S - 1) / S;       // steps of a chunk a lane may own
  constexpr int kRowP = S + 4;                // LDS stride (floats) of a step's partials
  __shared__ alignas(16) float4 sStep[RPW][T];          // delta, delta*u, dyh, softplus'
  __shared__ alignas(16) float sP[2][RPW][T][kRowP];    // per-step partials over the row

  const ScanParams& F = P.fwd;
  const In* __restrict__ u = static_cast<const In*>(F.u);
  const In* __restrict__ dlt = static_cast<const In*>(F.delta);
  const In* __restrict__ z = static_cast<const In*>(F.z);
  const In* __restrict__ Bm = static_cast<const In*>(F.B);
  const In* __restrict__ Cm = static_cast<const In*>(F.C);
  const In* __restrict__ dyp = static_cast<const In*>(P.dy);
  In* __restrict__ du_out = static_cast<In*>(P.du);
  In* __restrict__ dd_out = static_cast<In*>(P.ddelta);
  In* __restrict__ dz_out = static_cast<In*>(P.dz);

  const int lane = threadIdx.x;
  const int r = lane / S, l = lane % S;
  const int b = blockIdx.y;
  const int d = blockIdx.x * RPW + r;
  const int L = F.seqlen, N = F.dstate;
  const bool row_ok = d < F.dim;
  const bool st_ok = row_ok && l < N;
  const bool has_z = z != nullptr;
  // time window: segment blockIdx.z (whole chunks), or the whole sequence
  const int seg = blockIdx.z;
  const int c_begin = lay.nseg > 1 ? seg * (lay.seg_len / T) : 0;
  const int c_end = lay.nseg > 1 ? min(lay.nck, c_begin + lay.seg_len / T) : lay.nck;
  const int dc = row_ok ? d : F.dim - 1;      // clamped row for addresses
  const int lc = min(l, N - 1);               // clamped state for addresses
  const int64_t rowi = (int64_t)b * F.dim + dc;
  const int64_t row_base = rowi * L;
  const int64_t rows = (int64_t)F.batch * F.dim;
  const int kpg = F.dim / F.ngroups;          // channels per group
  const int64_t bc_row = (((int64_t)b * F.ngroups + dc / kpg) * N + lc) * L;
  const float A = st_ok ? F.A[(int64_t)dc * N + lc] : 0.0f;
  const float A2 = A * kLog2e;
  const float Dd = (row_ok && F.D) ? F.D[dc] : 0.0f;
  const float bias = (row_ok && F.delta_bias) ? F.delta_bias[dc] : 0.0f;
  char* ws = static_cast<char*>(P.workspace);
  float* ck = reinterpret_cast<float*>(ws + lay.ck_off) + (rowi * N + lc) * lay.nck;
  // dB, dC of this (row, state): straight into the outputs for one channel
  // per group, else into the per-row arrays that the group sum adds up
  // (base pointers 16-byte aligned; the offset decides the store width)
  float* dB_base = P.dB;
  float* dC_base = P.dC;
  int64_t dbc_off = bc_row;
  if (kpg > 1) {
    dB_base = reinterpret_cast<float*>(ws + lay.rb_off);
    dC_base = dB_base + (int64_t)F.batch * F.dim * N * L;
    dbc_off = (rowi * N + lc) * L;
  }

  // Per-step values of the steps this lane owns (chunk step l + S j):
  // delta, delta*u, dyh = dy silu(z), softplus'; zero past the end.
  float ou[NOWN], oz[NOWN], ody[NOWN];
  auto own_steps = [&](int t0) {
#pragma unroll
    for (int j = 0; j < NOWN; ++j) {
      const int tt = l + S * j;
      if (tt >= T) continue;
      const int t = t0 + tt;
      const bool in = row_ok && t < L;
      const int64_t i = row_base + min(t, L - 1);
      const float uu = in ? Elem<In>::load(u, i) : 0.0f;
      const float x = (in ? Elem<In>::load(dlt, i) : 0.0f) + bias;
      const float zz = (in && has_z) ? Elem<In>::load(z, i) : 0.0f;
      const float dy = in ? Elem<In>::load(dyp, i) : 0.0f;
      float dl = x, sp = 1.0f;
      if (F.delta_softplus) {
        dl = softplus_in<In>(x);
        sp = fast_rcp(1.0f + fast_exp2(-x * kLog2e));
      }
      if (!in) dl = 0.0f;
      const float g = has_z ? silu_f(zz) : 1.0f;
      ou[j] = uu;
      oz[j] = zz;
      ody[j] = dy;
      sStep[r][tt] = make_float4(dl, dl * uu, dy * g, sp);
    }
  };
  // B and C of this lane's state for the chunk's steps (zero past the end,
  // and for lanes past dstate, whose terms must not reach the row's sums)
  float bv[T], cv[T];
  auto load_bc = [&](int t0) {
    RawSeg<In, T> rb, rc;
    load_raw<In, T>(Bm, bc_row, t0, L, rb);
    load_raw<In, T>(Cm, bc_row, t0, L, rc);
    decode_raw<In, T>(rb, bv);
    decode_raw<In, T>(rc, cv);
    if (!st_ok) {
#pragma unroll
      for (int tt = 0; tt < T; ++tt) bv[tt] = cv[tt] = 0.0f;
    }
  };

  // ---- forward sweep: h, the saved states, dC, dz, dD ---------------------------
  // the state entering the window: the initial state, or the segment's
  // carry-in left in slot seg - 1 by the forward's combine scan
  float h = (st_ok && F.h0) ? F.h0[rowi * N + l] : 0.0f;
  if (seg > 0 && st_ok)
    h = reinterpret_cast<const float*>(ws + lay.fwd_agg_off)[((seg - 1) * rows + rowi) * N * 2 +
                                                              2 * l + 1];
  float dD_acc = 0.0f, db_acc = 0.0f;
  for (int c = c_begin; c < c_end; ++c) {
    const int t0 = c * T;
    __builtin_amdgcn_wave_barrier();  // the previous chunk's LDS reads come first
    own_steps(t0);
    load_bc(t0);
    if (st_ok) ck[c] = h;
    __builtin_amdgcn_wave_barrier();
    float dcv[T];
#pragma unroll
    for (int tt = 0; tt < T; ++tt) {
      const float4 s = sStep[r][tt];
      h = __builtin_fmaf(fast_exp2(s.x * A2), h, s.y * bv[tt]);
      sP[0][r][tt][l] = cv[tt] * h;
      dcv[tt] = s.z * h;
    }
    if (st_ok) store_seg<float, T>(dC_base, dbc_off, t0, L, dcv);
    __builtin_amdgcn_wave_barrier();
#pragma unroll
    for (int j = 0; j < NOWN; ++j) {
      const int tt = l + S * j;
      if (tt >= T) continue;
      const int t = t0 + tt;
      if (!row_ok || t >= L) continue;
      const float* q = &sP[0][r][tt][0];
      float acc[4] = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
      for (int m = 0; m < S; m += 4) {
        const float4 v = *reinterpret_cast<const float4*>(q + m);
        acc[0] += v.x; acc[1] += v.y; acc[2] += v.z; acc[3] += v.w;
      }
      const float yh = ((acc[0] + acc[1]) + (acc[2] + acc[3])) + Dd * ou[j];
      const float dyh = sStep[r][tt].z;
      dD_acc = __builtin_fmaf(dyh, ou[j], dD_acc);
      if (has_z) {
        const float sg = fast_rcp(1.0f + fast_exp2(-oz[j] * kLog2e));
        const float dsilu = sg * (1.0f + oz[j] * (1.0f - sg));
        Elem<In>::store(dz_out, row_base + t, ody[j] * yh * dsilu);
      }
    }
  }

  // ---- reverse sweep: lam, du, ddelta, dA, dB, dinitial_state ----------------
  // the adjoint entering the window from the right: dlast, or the carry
  // left in slot seg by the adjoint's combine scan
  float lam = (st_ok && P.dlast) ? P.dlast[rowi * N + l] : 0.0f;
  if (seg < lay.nseg - 1 && st_ok)
    lam = reinterpret_cast<const float*>(ws + lay.lam_agg_off)[(seg * rows + rowi) * N * 2 +
                                                                2 * l + 1];
  float dA_acc = 0.0f;
  for (int c = c_end - 1; c >= c_begin; --c) {
    const int t0 = c * T;
    __builtin_amdgcn_wave_barrier();
    own_steps(t0);
    load_bc(t0);
    float hq = st_ok ? ck[c] : 0.0f;
    __builtin_amdgcn_wave_barrier();
    float q[T];  // a_t h_{t-1}
#pragma unroll
    for (int tt = 0; tt < T; ++tt) {
      const float4 s = sStep[r][tt];
      q[tt] = fast_exp2(s.x * A2) * hq;
      hq = __builtin_fmaf(s.y, bv[tt], q[tt]);
    }
    float dbv[T];
#pragma unroll
    for (int tt = T - 1; tt >= 0; --tt) {
      const float4 s = sStep[r][tt];
      lam = __builtin_fmaf(s.z, cv[tt], lam);
      dbv[tt] = lam * s.y;
      sP[0][r][tt][l] = lam * bv[tt];
      sP[1][r][tt][l] = lam * A * q[tt];
      dA_acc = __builtin_fmaf(lam * s.x, q[tt], dA_acc);
      lam *= fast_exp2(s.x * A2);
    }
    if (st_ok) store_seg<float, T>(dB_base, dbc_off, t0, L, dbv);
    __builtin_amdgcn_wave_barrier();
#pragma unroll
    for (int j = 0; j < NOWN; ++j) {
      const int tt = l + S * j;
      if (tt >= T) continue;
      const int t = t0 + tt;
      if (!row_ok || t >= L) continue;
      const float* q0 = &sP[0][r][tt][0];
      const float* q1 = &sP[1][r][tt][0];
      float a0[4] = {0.0f, 0.0f, 0.0f, 0.0f}, a1[4] = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
      for (int m = 0; m < S; m += 4) {
        const float4 v = *reinterpret_cast<const float4*>(q0 + m);
        const float4 w = *reinterpret_cast<const float4*>(q1 + m);
        a0[0] += v.x; a0[1] += v.y; a0[2] += v.z; a0[3] += v.w;
        a1[0] += w.x; a1[1] += w.y; a1[2] += w.z; a1[3] += w.w;
      }
      const float lb = (a0[0] + a0[1]) + (a0[2] + a0[3]);   // sum_n lam B_t
      const float laq = (a1[0] + a1[1]) + (a1[2] + a1[3]);  // sum_n lam A a_t h_{t-1}
      const float4 s = sStep[r][tt];
      Elem<In>::store(du_out, row_base + t, __builtin_fmaf(s.z, Dd, s.x * lb));
      const float dd = (laq + ou[j] * lb) * s.w;
      Elem<In>::store(dd_out, row_base + t, dd);
      db_acc += dd;
    }
  }
  if (seg == 0 && st_ok && P.dh0) P.dh0[rowi * N + l] = lam;

  // ---- per-row sums: dA per state, dD and ddelta_bias over the row's steps ---
  float* pa = reinterpret_cast<float*>(ws + lay.pa_off) + seg * rows * N;
  float* pd = reinterpret_cast<float*>(ws + lay.pd_off) + seg * 2 * rows;
  if (st_ok) pa[rowi * N + l] = dA_acc;
  __builtin_amdgcn_wave_barrier();
  sP[0][r][0][l] = dD_acc;
  sP[1][r][0][l] = db_acc;
  __builtin_amdgcn_wave_barrier();
  if (row_ok && l == 0) {
    float s0 = 0.0f, s1 = 0.0f;
    for (int m = 0; m < S; ++m) {  // fixed order
      s0 += sP[0][r][0][m];
      s1 += sP[1][r][0][m];
    }
    pd[rowi] = s0;
    pd[rows + rowi] = s1;
  }
}

// Aggregate of the adjoint recurrence over segment blockIdx.z + 1 (the
// segments after the first), from lam = 0, steps descending:
//   lam += C_t dyh_t;  lam *= a_t        (dyh = dy silu(z), a = exp(delta A))
// giving (prod a_t = exp2(A2 sum delta), lam) per (row, state): the adjoint
// leaving the segment to the left is (prod a) lam_in + lam for an adjoint
// lam_in entering it from the right ([EXPLAINED] eq. (10), run backwards).
template <typename In, int S>
__global__ void __launch_bounds__(64) bwd_rows_lam_agg_kernel(BwdParams P, RowsBwdLayout lay) {
  SSM_POISON_LDS_AT_ENTRY();
  constexpr int T = kRowsBwdT;
  constexpr int RPW = 64 / S;
  constexpr int NOWN = (T + S - 1) / S;
  __shared__ alignas(8) float2 sDy[RPW][T];  // delta, dyh of each step

  const ScanParams& F = P.fwd;
  const In* __restrict__ dlt = static_cast<const In*>(F.delta);
  const In* __restrict__ z = static_cast<const In*>(F.z);
  const In* __restrict__ Cm = static_cast<const In*>(F.C);
  const In* __restrict__ dyp = static_cast<const In*>(P.dy);
  const int lane = threadIdx.x;
  const int r = lane / S, l = lane % S;
  const int b = blockIdx.y;
  const int d = blockIdx.x * RPW + r;
  const int L = F.seqlen, N = F.dstate;
  const bool row_ok = d < F.dim;
  const bool st_ok = row_ok && l < N;
  const bool has_z = z != nullptr;
  const int dc = row_ok ? d : F.dim - 1;
  const int lc = min(l, N - 1);
  const int64_t rowi = (int64_t)b * F.dim + dc;
  const int64_t row_base = rowi * L;
  const int64_t rows = (int64_t)F.batch * F.dim;
  const int kpg = F.dim / F.ngroups;
  const int64_t bc_row = (((int64_t)b * F.ngroups + dc / kpg) * N + lc) * L;
  const float A2 = st_ok ? F.A[(int64_t)dc * N + lc] * kLog2e : 0.0f;
  const float bias = (row_ok && F.delta_bias) ? F.delta_bias[dc] : 0.0f;
  const int seg = blockIdx.z + 1;
  const int c_begin = seg * (lay.seg_len / T);
  const int c_end = min(lay.nck, c_begin + lay.seg_len / T);

  float lam = 0.0f, dsum = 0.0f;
  for (int c = c_end - 1; c >= c_begin; --c) {
    const int t0 = c * T;
    __builtin_amdgcn_wave_barrier();  // the previous chunk's LDS reads come first
#pragma unroll
    for (int j = 0; j < NOWN; ++j) {
      const int tt = l + S * j;
      if (tt >= T) continue;
      const bool in = row_ok && t0 + tt < L;
      const int64_t i = row_base + min(t0 + tt, L - 1);
      const float x = (in ? Elem<In>::load(dlt, i) : 0.0f) + bias;
      float dl = F.delta_softplus ? softplus_in<In>(x) : x;
      if (!in) dl = 0.0f;
      const float dy = in ? Elem<In>::load(dyp, i) : 0.0f;
      const float zz = (in && has_z) ? Elem<In>::load(z, i) : 0.0f;
      sDy[r][tt] = make_float2(dl, has_z ? dy * silu_f(zz) : dy);
    }
    RawSeg<In, T> rc;
    load_raw<In, T>(Cm, bc_row, t0, L, rc);
    float cv[T];
    decode_raw<In, T>(rc, cv);
    __builtin_amdgcn_wave_barrier();
#pragma unroll
    for (int tt = T - 1; tt >= 0; --tt) {
      const float2 s = sDy[r][tt];
      lam = __builtin_fmaf(st_ok ? cv[tt] : 0.0f, s.y, lam);
      lam *= fast_exp2(s.x * A2);
      dsum += s.x;
    }
  }
  if (st_ok) {
    float* ag = reinterpret_cast<float*>(static_cast<char*>(P.workspace) + lay.lam_agg_off) +
                ((seg - 1) * rows + rowi) * N * 2 + 2 * l;
    ag[0] = fast_exp2(A2 * dsum);
    ag[1] = lam;
  }
}

// dA[d][n], dD[d], ddelta_bias[d]: sums of the per-row partials over the
// segments and the batch, in a fixed order.
__global__ void __launch_bounds__(256) bwd_rows_params_kernel(BwdParams P, RowsBwdLayout lay) {
  const ScanParams& F = P.fwd;
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int64_t nA = (int64_t)F.dim * F.dstate;
  const char* ws = static_cast<const char*>(P.workspace);
  const float* pa = reinterpret_cast<const float*>(ws + lay.pa_off);
  const float* pd = reinterpret_cast<const float*>(ws + lay.pd_off);
  const int64_t rows = (int64_t)F.batch * F.dim;
  if (i < nA) {
    float s = 0.0f;
    for (int sg = 0; sg < lay.nseg; ++sg)
      for (int b = 0; b < F.batch; ++b) s += pa[(sg * F.batch + b) * nA + i];
    P.dA[i] = s;
  }
  if (i < F.dim) {
    float s0 = 0.0f, s1 = 0.0f;
    for (int sg = 0; sg < lay.nseg; ++sg)
      for (int b = 0; b < F.batch; ++b) {
        s0 += pd[sg * 2 * rows + (int64_t)b * F.dim + i];
        s1 += pd[sg * 2 * rows + rows + (int64_t)b * F.dim + i];
      }
    if (P.dD) P.dD[i] = s0;
    if (P.ddelta_bias) P.ddelta_bias[i] = s1;
  }
}

// dB[b][g][n][t] (and dC) = sum over the group's channels of the per-row
// values, in channel order; four consecutive steps per thread.
__global__ void __launch_bounds__(256) bwd_rows_group_sum_kernel(BwdParams P, RowsBwdLayout lay) {
  const ScanParams& F = P.fwd;
  const int L = F.seqlen, N = F.dstate;
  const int kpg = F.dim / F.ngroups;
  const int64_t L4 = (L + 3) / 4;
  const int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int64_t total = (int64_t)F.batch * F.ngroups * N * L4;
  if (idx >= total) return;
  const int t0 = (int)(idx % L4) * 4;
  const int64_t gn = idx / L4;                 // (b, g, n)
  const int n = (int)(gn % N);
  const int64_t bg = gn / N;
  const int g = (int)(bg % F.ngroups);
  const int b = (int)(bg / F.ngroups);
  const char* ws = static_cast<const char*>(P.workspace);
  const float* rb = reinterpret_cast<const float*>(ws + lay.rb_off);
  const int64_t per = (int64_t)F.batch * F.dim * N * L;
  const int cnt = min(4, L - t0);
  float sb[4] = {0.0f, 0.0f, 0.0f, 0.0f}, sc[4] = {0.0f, 0.0f, 0.0f, 0.0f};
  for (int k = 0; k < kpg; ++k) {
    const int64_t row = (int64_t)b * F.dim + (int64_t)g * kpg + k;
    const float* pb = rb + (row * N + n) * L + t0;
    for (int e = 0; e < cnt; ++e) {
      sb[e] += pb[e];
      sc[e] += pb[per + e];
    }
  }
  const int64_t o = (bg * N + n) * L + t0;
  for (int e = 0; e < cnt; ++e) {
    P.dB[o + e] = sb[e];
    P.dC[o + e] = sc[e];
  }
}

template <typename In, int S>
hipError_t launch_rows_bwd(const BwdParams& p, const RowsBwdLayout& lay, hipStream_t stream) {
  constexpr int RPW = 64 / S;
  const unsigned nblk = (unsigned)((p.fwd.dim + RPW - 1) / RPW);
  if (lay.nseg > 1) {
    // the adjoint's segment aggregates, then their combine scan from the right
    hipLaunchKernelGGL((bwd_rows_lam_agg_kernel<In, S>),
                       dim3(nblk, (unsigned)p.fwd.batch, (unsigned)(lay.nseg - 1)), dim3(64), 0,
                       stream, p, lay);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    e = launch_segment_carry(
        reinterpret_cast<float*>(static_cast<char*>(p.workspace) + lay.lam_agg_off),
        lay.nseg - 1, (int64_t)p.fwd.batch * p.fwd.dim * p.fwd.dstate, p.dlast, true, stream);
    if (e != hipSuccess) return e;
  }
  hipLaunchKernelGGL((bwd_rows_kernel<In, S>), dim3(nblk, (unsigned)p.fwd.batch,
                     (unsigned)lay.nseg), dim3(64), 0, stream, p, lay);
  return hipGetLastError();
}

template <typename In>
hipError_t launch_rows_bwd_typed(const BwdParams& p, const RowsBwdLayout& lay,
                                 hipStream_t stream) {
  if (p.fwd.dstate <= 16) return launch_rows_bwd<In, 16>(p, lay, stream);
  if (p.fwd.dstate <= 32) return launch_rows_bwd<In, 32>(p, lay, stream);
  return launch_rows_bwd<In, 64>(p, lay, stream);
}

}  // namespace

size_t selective_scan_bwd_rows_workspace(int batch, int dim, int dstate, int seqlen,
                                         int ngroups, int num_cus) {
  return rows_bwd_layout(batch, dim, dstate, seqlen, ngroups, num_cus).total;
}

hipError_t launch_selective_scan_bwd_rows(const BwdParams& p, bool bf16, int num_cus,
                                          hipStream_t stream) {
  const ScanParams& F = p.fwd;
  const RowsBwdLayout lay =
      rows_bwd_layout(F.batch, F.dim, F.dstate, F.seqlen, F.ngroups, num_cus);
  hipError_t e = hipSuccess;
  if (lay.nseg > 1) {
    // the forward's segment carry-ins: the per-row kernels' aggregate pass,
    // then the combine scan
    ScanParams fs = F;
    fs.y = nullptr;
    fs.last_state = nullptr;
    fs.seg_len = lay.seg_len;
    fs.seg_agg = reinterpret_cast<float*>(static_cast<char*>(p.workspace) + lay.fwd_agg_off);
    e = launch_selective_scan_rowbc_carries(fs, bf16, stream);
    if (e != hipSuccess) return e;
  }
  e = bf16 ? launch_rows_bwd_typed<uint16_t>(p, lay, stream)
           : launch_rows_bwd_typed<float>(p, lay, stream);
  if (e != hipSuccess) return e;
  const int64_t nA = std::max<int64_t>((int64_t)F.dim * F.dstate, F.dim);
  hipLaunchKernelGGL(bwd_rows_params_kernel, dim3((unsigned)((nA + 255) / 256)), dim3(256), 0,
                     stream, p, lay);
  e = hipGetLastError();
  if (e != hipSuccess || F.dim / F.ngroups == 1) return e;
  const int64_t total = (int64_t)F.batch * F.ngroups * F.dstate * ((F.seqlen + 3) / 4);
  hipLaunchKernelGGL(bwd_rows_group_sum_kernel, dim3((unsigned)((total + 255) / 256)), dim3(256),
                     0, stream, p, lay);
  return hipGetLastError();
}

}  // namespace ssm
