// api.cpp -- the C ABI of libssmscan.so: handles, argument validation,
// launch-shape selection and kernel launches.  See include/ssm_scan.h for the
// contract of every entry point.
#include <hip/hip_runtime.h>

#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <mutex>
#include <new>
#include <string>
#include <vector>

#include "selective_scan_launch.h"
#include "ssd_launch.h"
#include "ssm_scan.h"

namespace {

// The value of an ABI enum argument as an int.  A C caller may pass any int,
// and in C++ a load of an enum object holding a value outside its
// enumerators' range is undefined, so the bytes are copied instead.
int dtype_code(const ssm_dtype& d) {
  int c;
  memcpy(&c, &d, sizeof c);
  return c;
}

}  // namespace

struct ssm_scan_context {
  int device;
  int num_cus;
  char arch[64];
  void* scratch;  // device address of this device's no-allocation scratch
};

namespace {

thread_local std::string g_last_error;

ssm_status fail(ssm_status st, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  std::vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return st;
}

ssm_status ok() {
  g_last_error.clear();
  return SSM_OK;
}

// Device address of the no-allocation scratch, looked up once per device
// (hipGetSymbolAddress with that device current) and kept for the process.
ssm_status scratch_for_device(int device, void** out) {
  static std::mutex mu;
  static std::vector<void*> addr;
  std::lock_guard<std::mutex> lock(mu);
  if ((int)addr.size() <= device) addr.resize(device + 1, nullptr);
  if (!addr[device]) {
    int prev = -1;
    hipError_t e = hipGetDevice(&prev);
    if (e == hipSuccess && prev != device) e = hipSetDevice(device);
    void* p = nullptr;
    if (e == hipSuccess) e = ssm::scan_scratch_address(&p);
    if (prev >= 0 && prev != device) (void)hipSetDevice(prev);
    if (e != hipSuccess || !p)
      return fail(SSM_ERR_HIP, "hipGetSymbolAddress(scratch) on device %d: %s", device,
                  hipGetErrorString(e));
    addr[device] = p;
  }
  *out = addr[device];
  return SSM_OK;
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

struct Span {
  const char* name;
  const void* p;
  uint64_t bytes;
};

bool overlaps(const Span& a, const Span& b) {
  if (!a.p || !b.p || a.bytes == 0 || b.bytes == 0) return false;
  const uintptr_t a0 = reinterpret_cast<uintptr_t>(a.p), b0 = reinterpret_cast<uintptr_t>(b.p);
  return a0 < b0 + b.bytes && b0 < a0 + a.bytes;
}

// Checks that every non-null span is 16-byte aligned and that no output
// overlaps any other span.
ssm_status check_spans(const Span* in, int nin, const Span* out, int nout) {
  for (int i = 0; i < nin; ++i)
    if (in[i].p && !aligned16(in[i].p))
      return fail(SSM_ERR_INVALID_ARG, "%s is not 16-byte aligned", in[i].name);
  for (int i = 0; i < nout; ++i)
    if (out[i].p && !aligned16(out[i].p))
      return fail(SSM_ERR_INVALID_ARG, "%s is not 16-byte aligned", out[i].name);
  for (int i = 0; i < nout; ++i) {
    for (int j = 0; j < nin; ++j)
      if (overlaps(out[i], in[j]))
        return fail(SSM_ERR_INVALID_ARG, "output %s overlaps input %s", out[i].name, in[j].name);
    for (int j = i + 1; j < nout; ++j)
      if (overlaps(out[i], out[j]))
        return fail(SSM_ERR_INVALID_ARG, "outputs %s and %s overlap", out[i].name, out[j].name);
  }
  return SSM_OK;
}

// Makes the handle's device current for the duration of a call.
class DeviceGuard {
 public:
  explicit DeviceGuard(int device) : want_(device) {
    if (hipGetDevice(&prev_) != hipSuccess) { err_ = true; return; }
    if (prev_ != want_ && hipSetDevice(want_) != hipSuccess) err_ = true;
  }
  ~DeviceGuard() {
    if (!err_ && prev_ != want_) (void)hipSetDevice(prev_);
  }
  bool failed() const { return err_; }

 private:
  int want_;
  int prev_ = -1;
  bool err_ = false;
};

ssm::ScanTile pick_scan_tile(const ssm_scan_context* h, int64_t batch, int64_t dim,
                             int64_t dstate) {
  // Row-parallel shapes give one wave per SIMD or more on their own; below
  // that, each time chunk is also split over several waves.
  const int64_t row_tiles = batch * ((dim + 63) / 64);
  const int64_t simds = 4 * (int64_t)(h->num_cus > 0 ? h->num_cus : 256);
  using ssm::ScanTileId;
  // Too few rows: up to 16 states, the waves of a workgroup take
  // consecutive time slots of the same rows (the row-parallel lane layout);
  // above, lane = row with the states split over waves.
  if (dstate <= 4) {
    return {row_tiles >= simds ? ScanTileId::kN4_Seq : ScanTileId::kN4_Slot};
  } else if (dstate <= 8) {
    return {row_tiles * 2 >= simds ? ScanTileId::kN8_Seq : ScanTileId::kN8_Slot};
  } else if (dstate <= 16) {
    return {row_tiles * 4 >= simds ? ScanTileId::kN16_Seq : ScanTileId::kN16_Slot};
  }
  return {row_tiles * 4 >= simds ? ScanTileId::kN64_Seq : ScanTileId::kN64_Split};
}

}  // namespace

extern "C" {

const char* ssm_status_string(ssm_status status) {
  // A C caller may pass any int; read it as one (a C++ load of an enum
  // value outside its enumerators' range is undefined).
  int code;
  memcpy(&code, &status, sizeof code);
  switch (code) {
    case SSM_OK: return "SSM_OK";
    case SSM_ERR_INVALID_ARG: return "SSM_ERR_INVALID_ARG: invalid argument";
    case SSM_ERR_UNSUPPORTED: return "SSM_ERR_UNSUPPORTED: outside the supported limits";
    case SSM_ERR_HIP: return "SSM_ERR_HIP: HIP runtime error";
  }
  return "unknown ssm_status";
}

const char* ssm_last_error_message(void) { return g_last_error.c_str(); }

ssm_status ssm_scan_create(ssm_handle* out, int hip_device) {
  if (!out) return fail(SSM_ERR_INVALID_ARG, "out is NULL");
  *out = nullptr;
  int count = 0;
  hipError_t e = hipGetDeviceCount(&count);
  if (e != hipSuccess) return fail(SSM_ERR_HIP, "hipGetDeviceCount: %s", hipGetErrorString(e));
  if (hip_device < 0 || hip_device >= count)
    return fail(SSM_ERR_INVALID_ARG, "device %d out of range (%d devices)", hip_device, count);
  hipDeviceProp_t prop;
  e = hipGetDeviceProperties(&prop, hip_device);
  if (e != hipSuccess) return fail(SSM_ERR_HIP, "hipGetDeviceProperties: %s", hipGetErrorString(e));
  if (std::strncmp(prop.gcnArchName, "gfx950", 6) != 0)
    return fail(SSM_ERR_UNSUPPORTED, "device %d is %s; this library is built for gfx950",
                hip_device, prop.gcnArchName);
  void* scratch = nullptr;
  const ssm_status sst = scratch_for_device(hip_device, &scratch);
  if (sst != SSM_OK) return sst;
  ssm_scan_context* h = new (std::nothrow) ssm_scan_context;
  if (!h) return fail(SSM_ERR_HIP, "out of host memory");
  h->device = hip_device;
  h->num_cus = prop.multiProcessorCount;
  h->scratch = scratch;
  std::snprintf(h->arch, sizeof(h->arch), "%s", prop.gcnArchName);
  *out = h;
  return ok();
}

ssm_status ssm_scan_destroy(ssm_handle handle) {
  delete handle;
  return ok();
}

}  // extern "C"

namespace {

ssm_status selective_scan_impl(ssm_handle handle, const void* u, const void* delta,
                               const float* A, const void* B, const void* C, const float* D,
                               const void* z, const float* delta_bias, int delta_softplus,
                               const float* initial_state, void* y, float* last_state,
                               int64_t batch, int64_t dim, int64_t dstate, int64_t seqlen,
                               int64_t ngroups, void* workspace, size_t workspace_bytes,
                               int in_dtype, hipStream_t stream, bool use_scratch = false) {
  // ---- sizes -------------------------------------------------------------
  if (batch <= 0) return fail(SSM_ERR_INVALID_ARG, "batch must be >= 1 (got %lld)", (long long)batch);
  if (dim <= 0) return fail(SSM_ERR_INVALID_ARG, "dim must be >= 1 (got %lld)", (long long)dim);
  if (dstate <= 0) return fail(SSM_ERR_INVALID_ARG, "dstate must be >= 1 (got %lld)", (long long)dstate);
  if (seqlen <= 0) return fail(SSM_ERR_INVALID_ARG, "seqlen must be >= 1 (got %lld)", (long long)seqlen);
  if (ngroups <= 0 || dim % ngroups != 0)
    return fail(SSM_ERR_INVALID_ARG, "ngroups %lld must be >= 1 and divide dim %lld",
                (long long)ngroups, (long long)dim);
  if (in_dtype != SSM_F32 && in_dtype != SSM_BF16)
    return fail(SSM_ERR_INVALID_ARG, "unknown in_dtype %d", in_dtype);
  if (dstate > 64) return fail(SSM_ERR_UNSUPPORTED, "dstate %lld > 64", (long long)dstate);
  if (batch > 65535) return fail(SSM_ERR_UNSUPPORTED, "batch %lld > 65535", (long long)batch);
  if (seqlen > INT32_MAX || dim > INT32_MAX || batch * dim > INT32_MAX)
    return fail(SSM_ERR_UNSUPPORTED, "batch*dim and seqlen must fit in int32");
  if (batch * dim > (int64_t(1) << 62) / seqlen)
    return fail(SSM_ERR_UNSUPPORTED, "tensor too large");
  // ---- pointers ----------------------------------------------------------
  if (!u) return fail(SSM_ERR_INVALID_ARG, "u is NULL");
  if (!delta) return fail(SSM_ERR_INVALID_ARG, "delta is NULL");
  if (!A) return fail(SSM_ERR_INVALID_ARG, "A is NULL");
  if (!B) return fail(SSM_ERR_INVALID_ARG, "B is NULL");
  if (!C) return fail(SSM_ERR_INVALID_ARG, "C is NULL");
  if (!y) return fail(SSM_ERR_INVALID_ARG, "y is NULL");
  const uint64_t es = in_dtype == SSM_BF16 ? 2 : 4;
  const uint64_t nrow = (uint64_t)batch * dim * seqlen;
  const uint64_t nbc = (uint64_t)batch * ngroups * dstate * seqlen;
  const uint64_t state_bytes = (uint64_t)batch * dim * dstate * 4;
  // initial_state may be last_state itself (each entry is read once, before
  // the thread that reads it writes it); any other overlap with an output is
  // rejected like for the other inputs.
  const bool in_place = initial_state != nullptr && (const void*)initial_state == last_state;
  const Span in[] = {{"u", u, nrow * es},          {"delta", delta, nrow * es},
                     {"A", A, (uint64_t)dim * dstate * 4}, {"B", B, nbc * es},
                     {"C", C, nbc * es},           {"D", D, (uint64_t)dim * 4},
                     {"z", z, nrow * es},          {"delta_bias", delta_bias, (uint64_t)dim * 4},
                     {"initial_state", in_place ? nullptr : initial_state, state_bytes}};
  const Span out[] = {{"y", y, nrow * es}, {"last_state", last_state, state_bytes},
                      {"workspace", workspace, workspace_bytes}};
  ssm_status st = check_spans(in, 9, out, 3);
  if (st != SSM_OK) return st;
  if (!handle) return fail(SSM_ERR_INVALID_ARG, "handle is NULL");
  // Per-row B, C when the groups cover no whole workgroup of the kernel the
  // rows pick (each row then reads its own B and C).  Time segments when the
  // rows alone leave SIMDs idle and a workspace is given (shared B, C:
  // groups must also cover whole workgroups of the segmented kernel).
  const ssm::ScanTile tile = pick_scan_tile(handle, batch, dim, dstate);
  const bool per_row = ngroups > 1 && (dim / ngroups) % ssm::scan_tile_rows(tile) != 0;
  ssm::ScanSegments sg =
      per_row ? ssm::plan_scan_segments_rowbc(batch, dim, dstate, seqlen, handle->num_cus)
              : ssm::plan_scan_segments(batch, dim, dstate, seqlen, handle->num_cus);
  if (!per_row && ngroups > 1 && (dim / ngroups) % sg.rows_per_workgroup != 0) sg.nseg = 1;
  if (use_scratch) {  // the device's own scratch array stands in for the workspace
    workspace = handle->scratch;
    workspace_bytes = ssm::kNoAllocScratchBytes;
    if (sg.nseg > 1 && !in_place && sg.bytes > workspace_bytes)
      return fail(SSM_ERR_UNSUPPORTED, "time split needs %zu bytes of scratch, more than the "
                  "%zu of the no-allocation entry point", sg.bytes, workspace_bytes);
  }
  // (not in place: the last segment writes last_state while other segments
  // may still have to read the initial state)
  const bool segmented = sg.nseg > 1 && workspace != nullptr && !in_place;
  if (segmented && workspace_bytes < sg.bytes)
    return fail(SSM_ERR_INVALID_ARG, "workspace_bytes %zu < %zu needed", workspace_bytes,
                sg.bytes);

  // ---- launch ------------------------------------------------------------
  ssm::ScanParams p;
  p.u = u; p.delta = delta; p.A = A; p.B = B; p.C = C; p.D = D; p.z = z;
  p.delta_bias = delta_bias; p.y = y; p.last_state = last_state; p.h0 = initial_state;
  p.batch = (int)batch; p.dim = (int)dim; p.dstate = (int)dstate; p.seqlen = (int)seqlen;
  p.delta_softplus = delta_softplus ? 1 : 0;
  p.ngroups = (int)ngroups;
  DeviceGuard guard(handle->device);
  if (guard.failed()) return fail(SSM_ERR_HIP, "cannot select device %d", handle->device);
  const bool bf16 = in_dtype == SSM_BF16;
  hipError_t e;
  if (segmented) {
    p.seg_agg = static_cast<float*>(workspace);
    e = per_row ? ssm::launch_selective_scan_rowbc_segmented(p, sg, bf16, stream)
                : ssm::launch_selective_scan_segmented(p, sg, bf16, stream);
  } else if (!per_row) {
    e = ssm::launch_selective_scan(p, tile, bf16, stream);
  } else {
    e = ssm::launch_selective_scan_rowbc(p, bf16, stream);
  }
  if (e != hipSuccess) return fail(SSM_ERR_HIP, "kernel launch: %s", hipGetErrorString(e));
  return ok();
}

}  // namespace

extern "C" {

ssm_status ssm_selective_scan_fwd(ssm_handle handle, const void* u, const void* delta,
                                  const float* A, const void* B, const void* C, const float* D,
                                  const void* z, const float* delta_bias, int delta_softplus,
                                  void* y, float* last_state, int64_t batch, int64_t dim,
                                  int64_t dstate, int64_t seqlen, ssm_dtype in_dtype,
                                  hipStream_t stream) {
  return selective_scan_impl(handle, u, delta, A, B, C, D, z, delta_bias, delta_softplus,
                             nullptr, y, last_state, batch, dim, dstate, seqlen, 1, nullptr, 0,
                             dtype_code(in_dtype), stream);
}

ssm_status ssm_selective_scan_fwd_with_state(ssm_handle handle, const void* u,
                                             const void* delta, const float* A, const void* B,
                                             const void* C, const float* D, const void* z,
                                             const float* delta_bias, int delta_softplus,
                                             const float* initial_state, void* y,
                                             float* last_state, int64_t batch, int64_t dim,
                                             int64_t dstate, int64_t seqlen, ssm_dtype in_dtype,
                                             hipStream_t stream) {
  return selective_scan_impl(handle, u, delta, A, B, C, D, z, delta_bias, delta_softplus,
                             initial_state, y, last_state, batch, dim, dstate, seqlen, 1, nullptr,
                             0, dtype_code(in_dtype), stream);
}

ssm_status ssm_selective_scan_fwd_grouped(ssm_handle handle, const void* u, const void* delta,
                                          const float* A, const void* B, const void* C,
                                          const float* D, const void* z,
                                          const float* delta_bias, int delta_softplus,
                                          const float* initial_state, void* y,
                                          float* last_state, int64_t batch, int64_t dim,
                                          int64_t dstate, int64_t seqlen, int64_t ngroups,
                                          ssm_dtype in_dtype, hipStream_t stream) {
  return selective_scan_impl(handle, u, delta, A, B, C, D, z, delta_bias, delta_softplus,
                             initial_state, y, last_state, batch, dim, dstate, seqlen, ngroups,
                             nullptr, 0, dtype_code(in_dtype), stream);
}

ssm_status ssm_selective_scan_fwd_workspace_size(ssm_handle handle, int64_t batch, int64_t dim,
                                                 int64_t dstate, int64_t seqlen, int64_t ngroups,
                                                 size_t* bytes) {
  if (!bytes) return fail(SSM_ERR_INVALID_ARG, "bytes is NULL");
  *bytes = 0;
  if (batch <= 0 || dim <= 0 || dstate <= 0 || seqlen <= 0)
    return fail(SSM_ERR_INVALID_ARG, "all sizes must be >= 1");
  if (ngroups <= 0 || dim % ngroups != 0)
    return fail(SSM_ERR_INVALID_ARG, "ngroups %lld must be >= 1 and divide dim %lld",
                (long long)ngroups, (long long)dim);
  if (dstate > 64) return fail(SSM_ERR_UNSUPPORTED, "dstate %lld > 64", (long long)dstate);
  if (!handle) return fail(SSM_ERR_INVALID_ARG, "handle is NULL");
  const ssm::ScanTile tile = pick_scan_tile(handle, batch, dim, dstate);
  const bool per_row = ngroups > 1 && (dim / ngroups) % ssm::scan_tile_rows(tile) != 0;
  if (per_row) {
    const ssm::ScanSegments sg =
        ssm::plan_scan_segments_rowbc(batch, dim, dstate, seqlen, handle->num_cus);
    if (sg.nseg > 1) *bytes = sg.bytes;
    return ok();
  }
  const ssm::ScanSegments sg = ssm::plan_scan_segments(batch, dim, dstate, seqlen, handle->num_cus);
  if (sg.nseg > 1 && (ngroups == 1 || (dim / ngroups) % sg.rows_per_workgroup == 0))
    *bytes = sg.bytes;
  return ok();
}

ssm_status ssm_selective_scan_fwd_ws(ssm_handle handle, const void* u, const void* delta,
                                     const float* A, const void* B, const void* C, const float* D,
                                     const void* z, const float* delta_bias, int delta_softplus,
                                     const float* initial_state, void* y, float* last_state,
                                     int64_t batch, int64_t dim, int64_t dstate, int64_t seqlen,
                                     int64_t ngroups, void* workspace, size_t workspace_bytes,
                                     ssm_dtype in_dtype, hipStream_t stream) {
  return selective_scan_impl(handle, u, delta, A, B, C, D, z, delta_bias, delta_softplus,
                             initial_state, y, last_state, batch, dim, dstate, seqlen, ngroups,
                             workspace, workspace_bytes, dtype_code(in_dtype), stream);
}

ssm_status ssm_selective_scan_fwd_noalloc(ssm_handle handle, const void* u, const void* delta,
                                          const float* A, const void* B, const void* C,
                                          const float* D, const void* z,
                                          const float* delta_bias, int delta_softplus,
                                          const float* initial_state, void* y,
                                          float* last_state, int64_t batch, int64_t dim,
                                          int64_t dstate, int64_t seqlen, int64_t ngroups,
                                          ssm_dtype in_dtype, hipStream_t stream) {
  return selective_scan_impl(handle, u, delta, A, B, C, D, z, delta_bias, delta_softplus,
                             initial_state, y, last_state, batch, dim, dstate, seqlen, ngroups,
                             nullptr, 0, dtype_code(in_dtype), stream, /*use_scratch=*/true);
}

namespace {

// The grouped backward's condition on ngroups.
ssm_status check_bwd_groups(int64_t dim, int64_t ngroups) {
  if (ngroups <= 0 || dim % ngroups != 0)
    return fail(SSM_ERR_INVALID_ARG, "ngroups %lld must be >= 1 and divide dim %lld",
                (long long)ngroups, (long long)dim);
  return SSM_OK;
}

// B, C read per row: a group's channels are not a whole number of the
// shared-B/C backward workgroups (those sum dB, dC over whole workgroups).
bool bwd_per_row(int64_t dim, int64_t dstate, int64_t ngroups) {
  const int rpw = ssm::selective_scan_bwd_rows_per_workgroup((int)dstate);
  return ngroups > 1 && (dim / ngroups) % rpw != 0;
}

}  // namespace

ssm_status ssm_selective_scan_bwd_workspace_size(ssm_handle handle, int64_t batch, int64_t dim,
                                                int64_t dstate, int64_t seqlen, size_t* bytes) {
  return ssm_selective_scan_bwd_grouped_workspace_size(handle, batch, dim, dstate, seqlen, 1,
                                                       bytes);
}

ssm_status ssm_selective_scan_bwd_grouped_workspace_size(ssm_handle handle, int64_t batch,
                                                        int64_t dim, int64_t dstate,
                                                        int64_t seqlen, int64_t ngroups,
                                                        size_t* bytes) {
  if (!bytes) return fail(SSM_ERR_INVALID_ARG, "bytes is NULL");
  *bytes = 0;
  if (batch <= 0 || dim <= 0 || dstate <= 0 || seqlen <= 0)
    return fail(SSM_ERR_INVALID_ARG, "all sizes must be >= 1");
  if (dstate > 64) return fail(SSM_ERR_UNSUPPORTED, "backward: dstate %lld > 64", (long long)dstate);
  ssm_status gs = check_bwd_groups(dim, ngroups);
  if (gs != SSM_OK) return gs;
  if (batch > 65535) return fail(SSM_ERR_UNSUPPORTED, "batch %lld > 65535", (long long)batch);
  if (seqlen > INT32_MAX || dim > INT32_MAX || batch * dim > INT32_MAX)
    return fail(SSM_ERR_UNSUPPORTED, "batch*dim and seqlen must fit in int32");
  if (batch * dim > (int64_t(1) << 62) / seqlen / 64)
    return fail(SSM_ERR_UNSUPPORTED, "tensor too large");
  if (!handle) return fail(SSM_ERR_INVALID_ARG, "handle is NULL");
  *bytes = bwd_per_row(dim, dstate, ngroups)
               ? ssm::selective_scan_bwd_rows_workspace((int)batch, (int)dim, (int)dstate,
                                                        (int)seqlen, (int)ngroups, handle->num_cus)
               : ssm::selective_scan_bwd_layout((int)batch, (int)dim, (int)dstate, (int)seqlen,
                                                handle->num_cus, 4, (int)ngroups).total;
  return ok();
}

static ssm_status selective_scan_bwd_impl(
    ssm_handle handle, const void* u, const void* delta, const float* A, const void* B,
    const void* C, const float* D, const void* z, const float* delta_bias, int delta_softplus,
    const float* initial_state, const void* dy, const float* dlast_state, void* du,
    void* ddelta, float* dA, float* dB, float* dC, float* dD, void* dz, float* ddelta_bias,
    float* dinitial_state, void* workspace, size_t workspace_bytes, int64_t batch, int64_t dim,
    int64_t dstate, int64_t seqlen, int64_t ngroups, int in_dtype, hipStream_t stream);

ssm_status ssm_selective_scan_bwd(ssm_handle handle, const void* u, const void* delta,
                                  const float* A, const void* B, const void* C, const float* D,
                                  const void* z, const float* delta_bias, int delta_softplus,
                                  const float* initial_state, const void* dy,
                                  const float* dlast_state, void* du, void* ddelta, float* dA,
                                  float* dB, float* dC, float* dD, void* dz, float* ddelta_bias,
                                  float* dinitial_state, void* workspace, size_t workspace_bytes,
                                  int64_t batch, int64_t dim, int64_t dstate, int64_t seqlen,
                                  ssm_dtype in_dtype, hipStream_t stream) {
  return selective_scan_bwd_impl(handle, u, delta, A, B, C, D, z, delta_bias,
                                        delta_softplus, initial_state, dy, dlast_state, du,
                                        ddelta, dA, dB, dC, dD, dz, ddelta_bias, dinitial_state,
                                        workspace, workspace_bytes, batch, dim, dstate, seqlen, 1,
                                        dtype_code(in_dtype), stream);
}

static ssm_status selective_scan_bwd_impl(
    ssm_handle handle, const void* u, const void* delta, const float* A, const void* B,
    const void* C, const float* D, const void* z, const float* delta_bias, int delta_softplus,
    const float* initial_state, const void* dy, const float* dlast_state, void* du,
    void* ddelta, float* dA, float* dB, float* dC, float* dD, void* dz, float* ddelta_bias,
    float* dinitial_state, void* workspace, size_t workspace_bytes, int64_t batch, int64_t dim,
    int64_t dstate, int64_t seqlen, int64_t ngroups, int in_dtype, hipStream_t stream) {
  if (batch <= 0) return fail(SSM_ERR_INVALID_ARG, "batch must be >= 1 (got %lld)", (long long)batch);
  if (dim <= 0) return fail(SSM_ERR_INVALID_ARG, "dim must be >= 1 (got %lld)", (long long)dim);
  if (dstate <= 0) return fail(SSM_ERR_INVALID_ARG, "dstate must be >= 1 (got %lld)", (long long)dstate);
  if (seqlen <= 0) return fail(SSM_ERR_INVALID_ARG, "seqlen must be >= 1 (got %lld)", (long long)seqlen);
  if (in_dtype != SSM_F32 && in_dtype != SSM_BF16)
    return fail(SSM_ERR_INVALID_ARG, "unknown in_dtype %d", in_dtype);
  if (dstate > 64) return fail(SSM_ERR_UNSUPPORTED, "backward: dstate %lld > 64", (long long)dstate);
  if (batch > 65535) return fail(SSM_ERR_UNSUPPORTED, "batch %lld > 65535", (long long)batch);
  if (seqlen > INT32_MAX || dim > INT32_MAX || batch * dim > INT32_MAX)
    return fail(SSM_ERR_UNSUPPORTED, "batch*dim and seqlen must fit in int32");
  if (batch * dim > (int64_t(1) << 62) / seqlen / 64)
    return fail(SSM_ERR_UNSUPPORTED, "tensor too large");
  ssm_status gs = check_bwd_groups(dim, ngroups);
  if (gs != SSM_OK) return gs;
  const struct { const char* name; const void* p; } required[] = {
      {"u", u}, {"delta", delta}, {"A", A}, {"B", B}, {"C", C}, {"dy", dy}, {"du", du},
      {"ddelta", ddelta}, {"dA", dA}, {"dB", dB}, {"dC", dC}, {"workspace", workspace}};
  for (const auto& r : required)
    if (!r.p) return fail(SSM_ERR_INVALID_ARG, "%s is NULL", r.name);
  if (z && !dz) return fail(SSM_ERR_INVALID_ARG, "dz is NULL while z is given");
  const uint64_t es = in_dtype == SSM_BF16 ? 2 : 4;
  const uint64_t nrow = (uint64_t)batch * dim * seqlen;
  const uint64_t nbc = (uint64_t)batch * ngroups * dstate * seqlen;
  const uint64_t nst = (uint64_t)batch * dim * dstate * 4;
  const Span in[] = {{"u", u, nrow * es},          {"delta", delta, nrow * es},
                     {"A", A, (uint64_t)dim * dstate * 4}, {"B", B, nbc * es},
                     {"C", C, nbc * es},           {"D", D, (uint64_t)dim * 4},
                     {"z", z, nrow * es},          {"delta_bias", delta_bias, (uint64_t)dim * 4},
                     {"initial_state", initial_state, nst}, {"dy", dy, nrow * es},
                     {"dlast_state", dlast_state, nst}};
  const Span out[] = {{"du", du, nrow * es},       {"ddelta", ddelta, nrow * es},
                      {"dA", dA, (uint64_t)dim * dstate * 4}, {"dB", dB, nbc * 4},
                      {"dC", dC, nbc * 4},         {"dD", dD, (uint64_t)dim * 4},
                      {"dz", z ? dz : nullptr, nrow * es},
                      {"ddelta_bias", ddelta_bias, (uint64_t)dim * 4},
                      {"dinitial_state", dinitial_state, nst},
                      {"workspace", workspace, workspace_bytes}};
  ssm_status st = check_spans(in, 11, out, 10);
  if (st != SSM_OK) return st;
  if (!handle) return fail(SSM_ERR_INVALID_ARG, "handle is NULL");
  const bool per_row = bwd_per_row(dim, dstate, ngroups);
  const ssm::BwdLayout lay = ssm::selective_scan_bwd_layout(
      (int)batch, (int)dim, (int)dstate, (int)seqlen, handle->num_cus, 4, (int)ngroups);
  const size_t need = per_row ? ssm::selective_scan_bwd_rows_workspace(
                                    (int)batch, (int)dim, (int)dstate, (int)seqlen, (int)ngroups,
                                    handle->num_cus)
                              : lay.total;
  if (workspace_bytes < need)
    return fail(SSM_ERR_INVALID_ARG, "workspace too small: %zu < %zu bytes", workspace_bytes,
                need);

  ssm::BwdParams p;
  ssm::ScanParams& f = p.fwd;
  f.u = u; f.delta = delta; f.A = A; f.B = B; f.C = C; f.D = D; f.z = z;
  f.delta_bias = delta_bias; f.y = nullptr; f.last_state = nullptr; f.h0 = initial_state;
  f.batch = (int)batch; f.dim = (int)dim; f.dstate = (int)dstate; f.seqlen = (int)seqlen;
  f.delta_softplus = delta_softplus ? 1 : 0;
  f.ngroups = (int)ngroups;
  p.dy = dy; p.dlast = dlast_state; p.du = du; p.ddelta = ddelta; p.dz = z ? dz : nullptr;
  p.dA = dA; p.dB = dB; p.dC = dC; p.dD = dD; p.ddelta_bias = ddelta_bias;
  p.dh0 = dinitial_state; p.workspace = workspace;
  DeviceGuard guard(handle->device);
  if (guard.failed()) return fail(SSM_ERR_HIP, "cannot select device %d", handle->device);
  hipError_t e = per_row ? ssm::launch_selective_scan_bwd_rows(p, in_dtype == SSM_BF16,
                                                                handle->num_cus, stream)
                         : ssm::launch_selective_scan_bwd(p, lay, in_dtype == SSM_BF16, stream);
  if (e != hipSuccess) return fail(SSM_ERR_HIP, "kernel launch: %s", hipGetErrorString(e));
  return ok();
}

ssm_status ssm_selective_scan_bwd_grouped(
    ssm_handle handle, const void* u, const void* delta, const float* A, const void* B,
    const void* C, const float* D, const void* z, const float* delta_bias, int delta_softplus,
    const float* initial_state, const void* dy, const float* dlast_state, void* du,
    void* ddelta, float* dA, float* dB, float* dC, float* dD, void* dz, float* ddelta_bias,
    float* dinitial_state, void* workspace, size_t workspace_bytes, int64_t batch, int64_t dim,
    int64_t dstate, int64_t seqlen, int64_t ngroups, ssm_dtype in_dtype, hipStream_t stream) {
  return selective_scan_bwd_impl(handle, u, delta, A, B, C, D, z, delta_bias, delta_softplus,
                                 initial_state, dy, dlast_state, du, ddelta, dA, dB, dC, dD, dz,
                                 ddelta_bias, dinitial_state, workspace, workspace_bytes, batch,
                                 dim, dstate, seqlen, ngroups, dtype_code(in_dtype), stream);
}

static ssm_status selective_state_update_impl(ssm_handle handle, float* state, const void* u,
                                              const void* delta, const float* A, const void* B,
                                              const void* C, const float* D, const void* z,
                                              const float* delta_bias, int delta_softplus,
                                              void* y, int64_t batch, int64_t dim,
                                              int64_t dstate, int64_t ngroups,
                                              int in_dtype, hipStream_t stream);

ssm_status ssm_selective_state_update(ssm_handle handle, float* state, const void* u,
                                      const void* delta, const float* A, const void* B,
                                      const void* C, const float* D, const void* z,
                                      const float* delta_bias, int delta_softplus, void* y,
                                      int64_t batch, int64_t dim, int64_t dstate,
                                      ssm_dtype in_dtype, hipStream_t stream) {
  return selective_state_update_impl(handle, state, u, delta, A, B, C, D, z, delta_bias,
                                            delta_softplus, y, batch, dim, dstate, 1, dtype_code(in_dtype),
                                            stream);
}

static ssm_status selective_state_update_impl(ssm_handle handle, float* state, const void* u,
                                              const void* delta, const float* A, const void* B,
                                              const void* C, const float* D, const void* z,
                                              const float* delta_bias, int delta_softplus,
                                              void* y, int64_t batch, int64_t dim,
                                              int64_t dstate, int64_t ngroups,
                                              int in_dtype, hipStream_t stream) {
  if (batch <= 0) return fail(SSM_ERR_INVALID_ARG, "batch must be >= 1 (got %lld)", (long long)batch);
  if (dim <= 0) return fail(SSM_ERR_INVALID_ARG, "dim must be >= 1 (got %lld)", (long long)dim);
  if (dstate <= 0) return fail(SSM_ERR_INVALID_ARG, "dstate must be >= 1 (got %lld)", (long long)dstate);
  if (in_dtype != SSM_F32 && in_dtype != SSM_BF16)
    return fail(SSM_ERR_INVALID_ARG, "unknown in_dtype %d", in_dtype);
  if (ngroups <= 0 || dim % ngroups != 0)
    return fail(SSM_ERR_INVALID_ARG, "ngroups %lld must be >= 1 and divide dim %lld",
                (long long)ngroups, (long long)dim);
  if (dstate > 64) return fail(SSM_ERR_UNSUPPORTED, "dstate %lld > 64", (long long)dstate);
  if (dim > INT32_MAX || batch > INT32_MAX || batch * dim > (int64_t(1) << 40))
    return fail(SSM_ERR_UNSUPPORTED, "batch*dim too large");
  if (!state) return fail(SSM_ERR_INVALID_ARG, "state is NULL");
  if (!u) return fail(SSM_ERR_INVALID_ARG, "u is NULL");
  if (!delta) return fail(SSM_ERR_INVALID_ARG, "delta is NULL");
  if (!A) return fail(SSM_ERR_INVALID_ARG, "A is NULL");
  if (!B) return fail(SSM_ERR_INVALID_ARG, "B is NULL");
  if (!C) return fail(SSM_ERR_INVALID_ARG, "C is NULL");
  if (!y) return fail(SSM_ERR_INVALID_ARG, "y is NULL");
  const uint64_t es = in_dtype == SSM_BF16 ? 2 : 4;
  const uint64_t nrow = (uint64_t)batch * dim;
  const uint64_t nbc = (uint64_t)batch * ngroups * dstate;
  const Span in[] = {{"u", u, nrow * es},          {"delta", delta, nrow * es},
                     {"A", A, (uint64_t)dim * dstate * 4}, {"B", B, nbc * es},
                     {"C", C, nbc * es},           {"D", D, (uint64_t)dim * 4},
                     {"z", z, nrow * es},          {"delta_bias", delta_bias, (uint64_t)dim * 4}};
  const Span out[] = {{"y", y, nrow * es}, {"state", state, nrow * dstate * 4}};
  ssm_status st = check_spans(in, 8, out, 2);
  if (st != SSM_OK) return st;
  if (!handle) return fail(SSM_ERR_INVALID_ARG, "handle is NULL");

  ssm::StepParams p;
  p.state = state; p.u = u; p.delta = delta; p.A = A; p.B = B; p.C = C; p.D = D; p.z = z;
  p.delta_bias = delta_bias; p.y = y;
  p.batch = (int)batch; p.dim = (int)dim; p.dstate = (int)dstate;
  p.delta_softplus = delta_softplus ? 1 : 0;
  p.ngroups = (int)ngroups;
  DeviceGuard guard(handle->device);
  if (guard.failed()) return fail(SSM_ERR_HIP, "cannot select device %d", handle->device);
  hipError_t e = ssm::launch_state_update(p, in_dtype == SSM_BF16, stream);
  if (e != hipSuccess) return fail(SSM_ERR_HIP, "kernel launch: %s", hipGetErrorString(e));
  return ok();
}

ssm_status ssm_selective_state_update_grouped(ssm_handle handle, float* state, const void* u,
                                              const void* delta, const float* A, const void* B,
                                              const void* C, const float* D, const void* z,
                                              const float* delta_bias, int delta_softplus,
                                              void* y, int64_t batch, int64_t dim,
                                              int64_t dstate, int64_t ngroups,
                                              ssm_dtype in_dtype, hipStream_t stream) {
  return selective_state_update_impl(handle, state, u, delta, A, B, C, D, z, delta_bias,
                                     delta_softplus, y, batch, dim, dstate, ngroups,
                                     dtype_code(in_dtype), stream);
}

ssm_status ssd_state_update(ssm_handle handle, float* state, const void* x, const void* dt,
                            const float* A, const void* B, const void* C, const float* D,
                            const float* dt_bias, int dt_softplus, void* y, int64_t batch,
                            int64_t nheads, int64_t headdim, int64_t dstate, int64_t ngroups,
                            ssm_dtype in_dtype, hipStream_t stream) {
  if (batch <= 0 || nheads <= 0 || headdim <= 0 || dstate <= 0 || ngroups <= 0)
    return fail(SSM_ERR_INVALID_ARG, "all sizes must be >= 1");
  if (nheads % ngroups != 0)
    return fail(SSM_ERR_INVALID_ARG, "nheads must be a multiple of ngroups");
  if (dtype_code(in_dtype) != SSM_F32 && dtype_code(in_dtype) != SSM_BF16)
    return fail(SSM_ERR_INVALID_ARG, "unknown in_dtype %d", dtype_code(in_dtype));
  if (dstate > 256) return fail(SSM_ERR_UNSUPPORTED, "dstate %lld > 256", (long long)dstate);
  if (batch > INT32_MAX || nheads > INT32_MAX || headdim > INT32_MAX ||
      batch * nheads * headdim > (int64_t(1) << 40))
    return fail(SSM_ERR_UNSUPPORTED, "batch*nheads*headdim too large");
  const struct { const char* name; const void* p; } required[] = {
      {"state", state}, {"x", x}, {"dt", dt}, {"A", A}, {"B", B}, {"C", C}, {"y", y}};
  for (const auto& r : required)
    if (!r.p) return fail(SSM_ERR_INVALID_ARG, "%s is NULL", r.name);
  const uint64_t es = dtype_code(in_dtype) == SSM_BF16 ? 2 : 4;
  const uint64_t nx = (uint64_t)batch * nheads * headdim;
  const uint64_t nbc = (uint64_t)batch * ngroups * dstate;
  const Span in[] = {{"x", x, nx * es},
                     {"dt", dt, (uint64_t)batch * nheads * es},
                     {"A", A, (uint64_t)nheads * 4},
                     {"B", B, nbc * es},
                     {"C", C, nbc * es},
                     {"D", D, (uint64_t)nheads * 4},
                     {"dt_bias", dt_bias, (uint64_t)nheads * 4}};
  const Span out[] = {{"y", y, nx * es}, {"state", state, nx * dstate * 4}};
  ssm_status st = check_spans(in, 7, out, 2);
  if (st != SSM_OK) return st;
  if (!handle) return fail(SSM_ERR_INVALID_ARG, "handle is NULL");

  ssm::SsdStepParams p;
  p.state = state; p.x = x; p.dt = dt; p.A = A; p.B = B; p.C = C; p.D = D; p.dt_bias = dt_bias;
  p.dt_softplus = dt_softplus ? 1 : 0; p.y = y;
  p.batch = (int)batch; p.nheads = (int)nheads; p.headdim = (int)headdim;
  p.dstate = (int)dstate; p.ngroups = (int)ngroups;
  DeviceGuard guard(handle->device);
  if (guard.failed()) return fail(SSM_ERR_HIP, "cannot select device %d", handle->device);
  hipError_t e = ssm::launch_ssd_state_update(p, dtype_code(in_dtype) == SSM_BF16, stream);
  if (e != hipSuccess) return fail(SSM_ERR_HIP, "kernel launch: %s", hipGetErrorString(e));
  return ok();
}

ssm_status ssd_chunk_scan_workspace_size(ssm_handle handle, int64_t batch, int64_t seqlen,
                                         int64_t nheads, int64_t headdim, int64_t dstate,
                                         int64_t ngroups, int64_t chunk_size, size_t* bytes) {
  if (!bytes) return fail(SSM_ERR_INVALID_ARG, "bytes is NULL");
  *bytes = 0;
  ssm::SsdShape s;
  ssm_status st = ssm::ssd_validate_shape(batch, seqlen, nheads, headdim, dstate, ngroups,
                                          chunk_size, &s, &g_last_error);
  if (st != SSM_OK) return st;
  if (!handle) return fail(SSM_ERR_INVALID_ARG, "handle is NULL");
  *bytes = ssm::ssd_workspace_bytes(s);
  return ok();
}

}  // extern "C"

namespace {

ssm_status ssd_impl(ssm_handle handle, const void* x, const void* dt, const float* A,
                    const void* B, const void* C, const float* D, const float* dt_bias,
                    int dt_softplus, const float* initial_state, void* y, float* final_state,
                    void* workspace, size_t workspace_bytes, int64_t batch, int64_t seqlen,
                    int64_t nheads, int64_t headdim, int64_t dstate, int64_t ngroups,
                    int64_t chunk_size, int in_dtype, hipStream_t stream) {
  ssm::SsdShape s;
  ssm_status st = ssm::ssd_validate_shape(batch, seqlen, nheads, headdim, dstate, ngroups,
                                          chunk_size, &s, &g_last_error);
  if (st != SSM_OK) return st;
  if (in_dtype != SSM_BF16 && in_dtype != SSM_F32)
    return fail(SSM_ERR_INVALID_ARG, "unknown in_dtype %d", in_dtype);
  if (in_dtype != SSM_BF16)
    return fail(SSM_ERR_UNSUPPORTED, "ssd_chunk_scan_fwd supports bf16 inputs only");
  if (!x) return fail(SSM_ERR_INVALID_ARG, "x is NULL");
  if (!dt) return fail(SSM_ERR_INVALID_ARG, "dt is NULL");
  if (!A) return fail(SSM_ERR_INVALID_ARG, "A is NULL");
  if (!B) return fail(SSM_ERR_INVALID_ARG, "B is NULL");
  if (!C) return fail(SSM_ERR_INVALID_ARG, "C is NULL");
  if (!y) return fail(SSM_ERR_INVALID_ARG, "y is NULL");
  if (!workspace) return fail(SSM_ERR_INVALID_ARG, "workspace is NULL");
  const size_t need = ssm::ssd_workspace_bytes(s);
  if (workspace_bytes < need)
    return fail(SSM_ERR_INVALID_ARG, "workspace too small: %zu < %zu bytes", workspace_bytes, need);
  const uint64_t es = 2;
  const uint64_t nx = (uint64_t)batch * seqlen * nheads * headdim;
  const uint64_t nbc = (uint64_t)batch * seqlen * ngroups * dstate;
  const uint64_t state_bytes = (uint64_t)batch * nheads * headdim * dstate * 4;
  // initial_state may be final_state itself (each entry is read once, by the
  // thread that later writes it); any other overlap with an output is an error.
  const bool in_place = initial_state != nullptr && (const void*)initial_state == final_state;
  const Span in[] = {{"x", x, nx * es},
                     {"dt", dt, (uint64_t)batch * seqlen * nheads * es},
                     {"A", A, (uint64_t)nheads * 4},
                     {"B", B, nbc * es},
                     {"C", C, nbc * es},
                     {"D", D, (uint64_t)nheads * 4},
                     {"dt_bias", dt_bias, (uint64_t)nheads * 4},
                     {"initial_state", in_place ? nullptr : initial_state, state_bytes}};
  const Span out[] = {{"y", y, nx * es},
                      {"final_state", final_state, state_bytes},
                      {"workspace", workspace, need}};
  st = check_spans(in, 8, out, 3);
  if (st != SSM_OK) return st;
  if (!handle) return fail(SSM_ERR_INVALID_ARG, "handle is NULL");

  ssm::SsdParams p;
  p.x = x; p.dt = dt; p.A = A; p.B = B; p.C = C; p.D = D; p.dt_bias = dt_bias;
  p.dt_softplus = dt_softplus ? 1 : 0; p.y = y; p.final_state = final_state;
  p.initial_state = initial_state; p.workspace = workspace; p.shape = s;
  DeviceGuard guard(handle->device);
  if (guard.failed()) return fail(SSM_ERR_HIP, "cannot select device %d", handle->device);
  hipError_t e = ssm::launch_ssd(p, stream);
  if (e != hipSuccess) return fail(SSM_ERR_HIP, "kernel launch: %s", hipGetErrorString(e));
  return ok();
}

}  // namespace

extern "C" {

ssm_status ssd_chunk_scan_fwd(ssm_handle handle, const void* x, const void* dt, const float* A,
                              const void* B, const void* C, const float* D, const float* dt_bias,
                              int dt_softplus, void* y, float* final_state, void* workspace,
                              size_t workspace_bytes, int64_t batch, int64_t seqlen,
                              int64_t nheads, int64_t headdim, int64_t dstate, int64_t ngroups,
                              int64_t chunk_size, ssm_dtype in_dtype, hipStream_t stream) {
  return ssd_impl(handle, x, dt, A, B, C, D, dt_bias, dt_softplus, nullptr, y, final_state,
                  workspace, workspace_bytes, batch, seqlen, nheads, headdim, dstate, ngroups,
                  chunk_size, dtype_code(in_dtype), stream);
}

ssm_status ssd_chunk_scan_fwd_with_state(ssm_handle handle, const void* x, const void* dt,
                                         const float* A, const void* B, const void* C,
                                         const float* D, const float* dt_bias, int dt_softplus,
                                         const float* initial_state, void* y, float* final_state,
                                         void* workspace, size_t workspace_bytes, int64_t batch,
                                         int64_t seqlen, int64_t nheads, int64_t headdim,
                                         int64_t dstate, int64_t ngroups, int64_t chunk_size,
                                         ssm_dtype in_dtype, hipStream_t stream) {
  return ssd_impl(handle, x, dt, A, B, C, D, dt_bias, dt_softplus, initial_state, y,
                  final_state, workspace, workspace_bytes, batch, seqlen, nheads, headdim, dstate,
                  ngroups, chunk_size, dtype_code(in_dtype), stream);
}

}  // extern "C"
