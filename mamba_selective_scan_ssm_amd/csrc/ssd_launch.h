// ssd_launch.h -- internal interface between the C-ABI layer and the Mamba-2
// (SSD) chunked-scan kernels (not installed, not part of the public ABI).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <string>

#include "ssm_scan.h"

namespace ssm {

struct SsdShape {
  int batch, seqlen, nheads, headdim, dstate, ngroups, chunk;
  int nchunks;  // ceil(seqlen / chunk)
  // Tile sizes the kernels run at: headdim rounded up to 32, 64 or 128 and
  // dstate to 32, 64, 128 or 256.  When they differ from headdim / dstate
  // (padded), x, B, C (and the initial state) are first copied into
  // zero-padded workspace tensors of the tile sizes, the kernels run on
  // those, and y (and the final state) are copied back.  Zero padding is
  // exact: padded states and channels only ever meet zeros.
  int kheaddim, kdstate;
  bool padded() const { return kheaddim != headdim || kdstate != dstate; }
};

struct SsdParams {
  const void* x;
  const void* dt;
  const float* A;
  const void* B;
  const void* C;
  const float* D;        // nullable
  const float* dt_bias;  // nullable
  int dt_softplus;
  void* y;
  float* final_state;    // nullable
  const float* initial_state;  // [b, h, P, N], nullable (zero)
  void* workspace;
  SsdShape shape;
  int hshift = 0;        // internal: set when 128-channel heads run as pairs of 64
};

// Workspace layout (256-byte aligned sections), with P' = kheaddim and
// N' = kdstate:
//   states [batch, nchunks, nheads, P', N'] bf16: each chunk's local state
//          (chunk-state kernel), then, in place, the state entering that
//          chunk (state-pass kernel)
//   decay  [batch, nheads', nchunks] float32: exp(sum of A*dt over the chunk),
//          nheads' = nheads P' / ssd_tile_headdim(P', N') (heads the kernels see)
// and only for padded shapes:
//   x', y' [batch, seqlen, nheads, P'] bf16;  B', C' [batch, seqlen, ngroups, N'] bf16
//   init', final' [batch, nheads, P', N'] float32
struct SsdLayout {
  size_t states_off, decay_off, x_off, y_off, b_off, c_off, init_off, final_off, total;
};

inline size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

// Channels per head of the kernels' tiles for a (padded) head of P channels
// and N states: 32 with 256 states, else up to 64; wider heads run as
// P / tile heads of the tile's width.
inline int ssd_tile_headdim(int P, int N) { return N > 128 ? 32 : (P < 64 ? P : 64); }

inline SsdLayout ssd_layout(const SsdShape& s) {
  SsdLayout l;
  const size_t P = s.kheaddim, N = s.kdstate;
  l.states_off = 0;
  l.decay_off = align256((size_t)s.batch * s.nchunks * s.nheads * P * N * 2);
  const size_t hk = (size_t)s.nheads * (P / ssd_tile_headdim((int)P, (int)N));
  size_t end = align256(l.decay_off + (size_t)s.batch * hk * s.nchunks * sizeof(float));
  l.x_off = l.y_off = l.b_off = l.c_off = l.init_off = l.final_off = 0;
  if (s.padded()) {
    const size_t rows_x = (size_t)s.batch * s.seqlen * s.nheads;
    const size_t rows_bc = (size_t)s.batch * s.seqlen * s.ngroups;
    const size_t st = (size_t)s.batch * s.nheads * P * N * sizeof(float);
    l.x_off = end;
    l.y_off = end = align256(l.x_off + rows_x * P * 2);
    l.b_off = end = align256(l.y_off + rows_x * P * 2);
    l.c_off = end = align256(l.b_off + rows_bc * N * 2);
    l.init_off = end = align256(l.c_off + rows_bc * N * 2);
    l.final_off = end = align256(l.init_off + st);
    end = align256(l.final_off + st);
  }
  l.total = end;
  return l;
}

inline size_t ssd_workspace_bytes(const SsdShape& s) { return ssd_layout(s).total; }

// Validates sizes against the documented limits; fills *out on success and
// writes a reason into *msg on failure.
ssm_status ssd_validate_shape(int64_t batch, int64_t seqlen, int64_t nheads, int64_t headdim,
                              int64_t dstate, int64_t ngroups, int64_t chunk, SsdShape* out,
                              std::string* msg);

hipError_t launch_ssd(const SsdParams& p, hipStream_t stream);

// One decode step of the SSD recurrence (ssd_state_update.hip).
struct SsdStepParams {
  float* state;          // [batch, nheads, headdim, dstate], read and written
  const void* x;         // [batch, nheads, headdim]
  const void* dt;        // [batch, nheads]
  const float* A;        // [nheads]
  const void* B;         // [batch, ngroups, dstate]
  const void* C;         // [batch, ngroups, dstate]
  const float* D;        // [nheads], nullable
  const float* dt_bias;  // [nheads], nullable
  int dt_softplus;
  void* y;               // [batch, nheads, headdim]
  int batch, nheads, headdim, dstate, ngroups;
};

hipError_t launch_ssd_state_update(const SsdStepParams& p, bool bf16, hipStream_t stream);

}  // namespace ssm
