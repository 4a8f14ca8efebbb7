// ssd_chunk_scan.hip -- Mamba-2 (SSD) chunked scan for gfx950.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <cstdio>

#include "ssd_launch.h"

namespace ssm {

ssm_status ssd_validate_shape(int64_t batch, int64_t seqlen, int64_t nheads, int64_t headdim,
                              int64_t dstate, int64_t ngroups, int64_t chunk, SsdShape* out,
                              std::string* msg) {
  char buf[256];
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
  if (dstate != 16 && dstate != 32 && dstate != 64 && dstate != 128 && dstate != 256)
    return bad(SSM_ERR_UNSUPPORTED, "dstate must be 16, 32, 64, 128 or 256");
  if (batch > 65535 || nheads > 65535 || seqlen > (1 << 30)) {
    std::snprintf(buf, sizeof(buf), "batch/nheads must be <= 65535 and seqlen <= 2^30");
    return bad(SSM_ERR_UNSUPPORTED, buf);
  }
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

hipError_t launch_ssd(const SsdParams&, hipStream_t) { return hipErrorNotSupported; }

}  // namespace ssm
