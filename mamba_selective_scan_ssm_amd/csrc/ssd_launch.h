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
};

// Workspace layout (256-byte aligned sections):
//   states [batch, nchunks, nheads, headdim, dstate] bf16: each chunk's
//          local state (chunk-state kernel), then, in place, the state
//          entering that chunk (state-pass kernel)
//   decay  [batch, nheads, nchunks] float32: exp(sum of A*dt over the chunk)
struct SsdLayout {
  size_t states_off, decay_off, total;
};

inline size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

inline SsdLayout ssd_layout(const SsdShape& s) {
  SsdLayout l;
  l.states_off = 0;
  l.decay_off = align256((size_t)s.batch * s.nchunks * s.nheads * s.headdim * s.dstate * 2);
  l.total = align256(l.decay_off + (size_t)s.batch * s.nheads * s.nchunks * sizeof(float));
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
