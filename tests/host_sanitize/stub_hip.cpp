// Definitions behind the host-only HIP stand-in (stub/hip/hip_runtime.h) and
// the kernel launchers that api.cpp calls, for a sanitizer build of the host
// layer with no GPU.  The runtime reports no device, exactly as the real one
// does on a machine without a GPU; a launcher checks the resolved
// parameters the way a kernel would rely on them and launches nothing.
#include <hip/hip_runtime.h>

#include <cstdio>
#include <cstdlib>

#include "internal.h"

hipError_t hipGetDevice(int*) { return hipErrorNoDevice; }
hipError_t hipDeviceGetAttribute(int*, hipDeviceAttribute_t, int) { return hipErrorNoDevice; }
hipError_t hipMemcpyAsync(void*, const void*, size_t, hipMemcpyKind, hipStream_t) {
  return hipErrorNoDevice;
}
hipError_t hipStreamSynchronize(hipStream_t) { return hipErrorNoDevice; }

namespace {

void require(bool ok, const char* what) {
  if (!ok) {
    std::fprintf(stderr, "stub launch: parameter check failed: %s\n", what);
    std::abort();
  }
}

}  // namespace

namespace smla {

// What every decode kernel assumes of its parameters.
hipError_t launch_decode(const DecodeParams& p, int, int, hipStream_t) {
  require(p.T > 0 && (p.H == 64 || p.H == 128) && p.K >= 1, "shape");
  require(p.S >= 1 && p.split_cols >= 1, "plan");
  require((int64_t)p.S * p.split_cols >= p.K && (int64_t)p.S * p.split_cols <= (1 << 30),
          "split span");
  require(p.q && p.out, "pointers");
  require(p.S == 1 || (p.mid_out && p.mid_lse), "split partials");
  require(p.row_stride_bytes >= 512, "row stride");
  return hipSuccess;
}
hipError_t launch_combine(const CombineParams& p, hipStream_t) {
  require(p.T > 0 && p.S >= 1 && p.stride >= p.S && p.mid_out && p.mid_lse && p.out,
          "combine");
  return hipSuccess;
}
hipError_t launch_gather_only(const DecodeParams& p, hipStream_t) {
  require(p.H == 128 && p.T > 0, "gather-only shape");
  return hipSuccess;
}
hipError_t launch_clear_error(int32_t* err, hipStream_t) {
  require(err != nullptr, "error block");
  return hipSuccess;
}
hipError_t launch_build_indices(const BuildParams& p, hipStream_t) {
  require(p.T > 0 && p.out && p.out_lens, "builder");
  return hipSuccess;
}
hipError_t noalloc_scratch(void**) { return hipErrorNoDevice; }

}  // namespace smla
