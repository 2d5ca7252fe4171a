// Allocation-free variable-length AllToAll (plr_copy_v_noalloc): plr_copy_v with its
// scratch in a file-scope device array instead of a caller buffer, for callers that
// cannot allocate device memory (code under stream capture, tight serving loops,
// harnesses that forbid allocation).
//
// The array lives in this code object, one copy per GPU the library runs on, for the
// life of the process. In host code its name is only a host-side stand-in, so its
// device address is looked up once per device (hipGetSymbolAddress, with that device
// current) and kept; kernels receive that address, exactly as they receive a caller's
// scratch buffer. The array starts at zero when the code object loads; the only part
// that must be zero at a call's start is the ticket word of the scratch header, and
// every call leaves it at zero (the last rank workgroup stores 0), while the keys and
// segment tables are written in full before they are read. Calls on one GPU share the
// array: calls that overlap on one GPU race.
#include <hip/hip_runtime.h>

#include <mutex>

#include "kernels.h"

namespace plr {

constexpr size_t kNoAllocScratchBytes = 4u << 20;  // 4 MiB per GPU
constexpr int kNoAllocMaxDevices = 64;

static __device__ __align__(256) uint8_t scratch[kNoAllocScratchBytes];

namespace {

std::once_flag g_once[kNoAllocMaxDevices];
void* g_ptr[kNoAllocMaxDevices];
hipError_t g_err[kNoAllocMaxDevices];

// Device address of `scratch` on device `dev`, looked up once with `dev` current.
hipError_t scratch_ptr(int dev, void** out) {
  if (dev < 0 || dev >= kNoAllocMaxDevices) return hipErrorInvalidDevice;
  std::call_once(g_once[dev], [dev] {
    int cur = -1;
    hipError_t e = hipGetDevice(&cur);
    if (e == hipSuccess && cur != dev) e = hipSetDevice(dev);
    void* p = nullptr;
    if (e == hipSuccess) e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (cur >= 0 && cur != dev) {
      const hipError_t r = hipSetDevice(cur);
      if (e == hipSuccess) e = r;
    }
    g_err[dev] = e;
    g_ptr[dev] = e == hipSuccess ? p : nullptr;
  });
  *out = g_ptr[dev];
  return g_err[dev];
}

}  // namespace
}  // namespace plr

extern "C" size_t plr_copy_v_noalloc_max_scratch_bytes(void) { return plr::kNoAllocScratchBytes; }

extern "C" int plr_copy_v_noalloc(int world, const void* const* srcs, const int64_t* rows_per_src,
                                  const int32_t* const* dest_of_row, size_t row_bytes, void* dst,
                                  int64_t* counts, int64_t* offsets, void* stream) {
  if (world < 1 || !rows_per_src) return PLR_EINVAL;
  if (world > PLR_MAX_WORLD) return PLR_EUNSUPPORTED;
  const int rows_rc = plr::copy_v_check_rows(world, rows_per_src);
  if (rows_rc != PLR_OK) return rows_rc;
  if (plr_copy_v_scratch_bytes(world, rows_per_src) > plr::kNoAllocScratchBytes) return PLR_ETOOLARGE;
  // the device the kernels will run on: the stream's, or the current one
  int dev = -1;
  hipError_t e = stream ? hipStreamGetDevice(static_cast<hipStream_t>(stream), &dev) : hipGetDevice(&dev);
  void* ptr = nullptr;
  if (e == hipSuccess) e = plr::scratch_ptr(dev, &ptr);
  if (e != hipSuccess) return plr::record_hip_error(e);
  return plr_copy_v(world, srcs, rows_per_src, dest_of_row, row_bytes, dst, counts, offsets, ptr, stream);
}
