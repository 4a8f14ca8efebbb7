// selective_scan_launch.h -- internal interface between the C-ABI layer and
// the Mamba-1 scan kernels (not installed, not part of the public ABI).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "ssm_scan.h"

namespace ssm {

// Device pointers and sizes of one ssm_selective_scan_fwd call (already
// validated by the C-ABI layer).
struct ScanParams {
  const void* u;
  const void* delta;
  const float* A;
  const void* B;
  const void* C;
  const float* D;           // nullable
  const void* z;            // nullable
  const float* delta_bias;  // nullable
  void* y;
  float* last_state;        // nullable
  const float* h0;          // initial state [batch, dim, dstate], nullable (zero)
  int batch;
  int dim;
  int dstate;
  int seqlen;
  int delta_softplus;
  int ngroups;              // B, C: [batch, ngroups, dstate, seqlen]; channel d
                            // reads group d / (dim / ngroups)
  int seg_len = 0;          // > 0: time segments of this many steps (grid.z)
  float* seg_agg = nullptr; // [nseg-1, batch*dim, dstate, 2] segment aggregates
};

// Compiled kernel shapes.  "Seq": each wave runs the whole sequence for its
// rows (no time split).  "Split": each time chunk is split over several
// waves whose carries are combined with the associative operator (lane =
// row).  "Slot": the row-parallel lane layout with the waves of a workgroup
// on consecutive time slots of the same rows.
enum class ScanTileId : int {
  kN4_Seq, kN8_Seq, kN16_Seq, kN64_Seq,
  kN4_Split, kN8_Split, kN16_Split, kN64_Split,
  kN4_Slot, kN8_Slot, kN16_Slot,
};

struct ScanTile {
  ScanTileId id;
};

hipError_t launch_selective_scan(const ScanParams& p, const ScanTile& tile, bool bf16,
                                 hipStream_t stream);

// Rows one workgroup of `tile` covers; with ngroups > 1 the tile's kernels
// read one group per workgroup, so dim / ngroups must be a multiple of it,
// else launch_selective_scan_rowbc is used.
int scan_tile_rows(const ScanTile& tile);

// Row-parallel kernel that reads B and C per row (any ngroups dividing dim,
// e.g. ngroups = dim: per-channel B and C).
hipError_t launch_selective_scan_rowbc(const ScanParams& p, bool bf16, hipStream_t stream);

// Time segments for shapes whose rows alone leave SIMDs without a wave:
// nseg segments of seg_len steps each (nseg = 1: no split), run by the
// row-parallel kernel in two launches (segment aggregates, then each segment
// from its carry-in), with `bytes` of workspace for the aggregates.
struct ScanSegments {
  int nseg, seg_len, rows_per_workgroup;
  size_t bytes;
};
ScanSegments plan_scan_segments(int64_t batch, int64_t dim, int64_t dstate, int64_t seqlen,
                                int num_cus);
// p.seg_agg must point at sg.bytes of workspace.
hipError_t launch_selective_scan_segmented(const ScanParams& p, const ScanSegments& sg, bool bf16,
                                           hipStream_t stream);
// The same for the per-row B, C kernels (groups of channels smaller than a
// workgroup): segments of whole 64-step chunks.
ScanSegments plan_scan_segments_rowbc(int64_t batch, int64_t dim, int64_t dstate, int64_t seqlen,
                                      int num_cus);
hipError_t launch_selective_scan_rowbc_segmented(const ScanParams& p, const ScanSegments& sg,
                                                 bool bf16, hipStream_t stream);

// Scratch of ssm_selective_scan_fwd_noalloc: a file-scope device array in
// selective_scan.hip, one copy per GPU, holding the time-split aggregates.
// Every plan of plan_scan_segments fits on a 256-CU device: a split is
// planned only when the rows give W < 4*CUs waves, into nseg <=
// ceil(12*CUs / W) segments, and the rows of W waves hold at most W*64*NG
// (row, state) pairs (NG <= 16 states per lane), so the (nseg-1) aggregates
// of 8 bytes per pair take < (12*CUs + W) * 512 * NG < 8192 * NG * CUs
// bytes = 32 MiB.
constexpr size_t kNoAllocScratchBytes = SSM_NOALLOC_SCRATCH_BYTES;

// Device address of that array on the current device (hipGetSymbolAddress;
// call once per device with the device current).
hipError_t scan_scratch_address(void** out);

// Carry-ins of the time segments from their aggregates (in place), by a
// wave-level combine scan per (row, state) pair: slots [nslots][npairs]
// float2 (prod a, v), 1 <= nslots <= 64; init [npairs] nullable (zero).
// reverse = false: slot s gets the state entering segment s + 1; true (an
// adjoint scanned from the right): slot s holds segment s + 1's aggregate
// and gets the adjoint entering segment s.
hipError_t launch_segment_carry(float* slots, int nslots, int64_t npairs, const float* init,
                                bool reverse, hipStream_t stream);

// Carry-ins of the time segments of p (p.seg_len > 0, a multiple of 64;
// dstate <= 16): the aggregate pass over every segment but the last, then
// segment_carry_kernel; slot s of p.seg_agg then holds the state entering
// segment s + 1.
hipError_t launch_selective_scan_carries(const ScanParams& p, bool bf16, hipStream_t stream);
// The same with B, C read per row (the one-state-per-lane kernels; p.seg_len
// a multiple of 64, dstate <= 64).
hipError_t launch_selective_scan_rowbc_carries(const ScanParams& p, bool bf16, hipStream_t stream);

// Backward pass (selective_scan_bwd.hip).
struct BwdParams {
  ScanParams fwd;           // forward inputs (y, last_state unused); fwd.h0 nullable
  const void* dy;           // [batch, dim, seqlen] in_dtype
  const float* dlast;       // [batch, dim, dstate] nullable
  void* du;                 // [batch, dim, seqlen] in_dtype
  void* ddelta;             // [batch, dim, seqlen] in_dtype
  void* dz;                 // [batch, dim, seqlen] in_dtype, required iff z given
  float* dA;                // [dim, dstate]
  float* dB;                // [batch, dstate, seqlen]
  float* dC;                // [batch, dstate, seqlen]
  float* dD;                // [dim], nullable
  float* ddelta_bias;       // [dim], nullable
  float* dh0;               // [batch, dim, dstate], nullable
  void* workspace;
  // fwd.ngroups: B, C, dB, dC are [batch, ngroups, dstate, seqlen]; a group's
  // channels are a whole number of the kernels' workgroups.
  // State-block mode (set by the driver for dstate > 16, null otherwise):
  // the kernel adds its per-step sums over its states -- readout, d/d delta
  // before the softplus derivative, d/d u without the skip term -- to these
  // float32 [batch, dim, seqlen] arrays (writes them when acc_init) and
  // writes neither du, ddelta, dz nor the dD / ddelta_bias partials.
  float* acc_y = nullptr;
  float* acc_ddt = nullptr;
  float* acc_du = nullptr;
  int acc_init = 0;
};

// Workspace of the backward pass.  With nseg > 1 the sequence is cut into
// nseg segments of seg_len steps (small batches): the forward's segment
// aggregates, the adjoint's segment aggregates and per-segment partials of
// dA, dD, ddelta_bias are kept as well.
struct BwdLayout {
  size_t chunk_states_off, part_bc_off, part_a_off, part_d_off, fwd_agg_off, lam_agg_off, total;
  int nchunks, nwg, nseg, seg_len;
  // dstate > 16: the states are taken in blocks of 16 (nblocks of them),
  // each a backward pass of its own whose workspace is the layout above (at
  // offset 0, for 16 states); after it: the float32 per-step accumulators
  // acc[3][batch, dim, seqlen], the block's inputs and gradients (A, dA
  // [dim, 16]; B, C [batch, ngroups, 16, seqlen] in the input type; dB, dC float32;
  // initial state, dlast, dinitial_state [batch, dim, 16]) and per-row
  // dD, ddelta_bias sums [2][batch, dim].
  int nblocks;
  size_t acc_off, a_off, b_off, c_off, h0_off, dl_off, da_off, db_off, dc_off, dh0_off, prow_off;
};

BwdLayout selective_scan_bwd_layout(int batch, int dim, int dstate, int seqlen, int num_cus,
                                    int in_bytes = 4, int ngroups = 1);
// Channels per workgroup of the backward kernels for this dstate (64 for
// dstate 9..64, 128 for 5..8, 256 for 1..4): with ngroups > 1, dim / ngroups
// must be a multiple of it.
int selective_scan_bwd_rows_per_workgroup(int dstate);
// Backward with B, C read per row (groups of channels that are not a whole
// number of the workgroups above, down to one channel): workspace bytes and
// launch (BwdParams::workspace of at least that size).
size_t selective_scan_bwd_rows_workspace(int batch, int dim, int dstate, int seqlen, int ngroups,
                                         int num_cus);
hipError_t launch_selective_scan_bwd_rows(const BwdParams& p, bool bf16, int num_cus,
                                          hipStream_t stream);
hipError_t launch_selective_scan_bwd(const BwdParams& p, const BwdLayout& lay, bool bf16,
                                     hipStream_t stream);

// One decode step (state_update.hip).
struct StepParams {
  float* state;             // [batch, dim, dstate], read and written
  const void* u;            // [batch, dim]
  const void* delta;        // [batch, dim]
  const float* A;           // [dim, dstate]
  const void* B;            // [batch, ngroups, dstate]
  const void* C;            // [batch, ngroups, dstate]
  const float* D;           // nullable
  const void* z;            // nullable
  const float* delta_bias;  // nullable
  void* y;                  // [batch, dim]
  int batch;
  int dim;
  int dstate;
  int delta_softplus;
  int ngroups = 1;          // channel d reads group d / (dim / ngroups)
};

hipError_t launch_state_update(const StepParams& p, bool bf16, hipStream_t stream);

}  // namespace ssm
