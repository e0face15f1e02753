// pp_attn_decode for callers that cannot allocate device memory: the
// workspace is a fixed scratch array of this library in each GPU's memory.
//
// The array is a file-scope __device__ variable: every GPU the library runs
// on holds its own copy (PP_NOALLOC_SCRATCH_BYTES) from the load of the code
// object until the process ends.  Host code never passes the array's name to
// a kernel (on the host that name is only a stand-in, not a device address):
// the first call on a device, with that device current, looks up the
// device's address of the array once and keeps it; every later call passes
// that address as the workspace of the ordinary decode step.  The decode
// step writes every workspace byte it reads within the call (plan, lists,
// split partials), so nothing needs clearing between calls; two calls that
// overlap on one GPU share the array and race.
#include <mutex>

#include "pp_internal.h"

namespace {

static __device__ __align__(256) unsigned char scratch[PP_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::once_flag g_once[kMaxDevices];
void* g_ptr[kMaxDevices];
hipError_t g_err[kMaxDevices];

// The device address of this device's scratch array (nullptr on failure,
// with the HIP error in *err).
void* scratch_address(int dev, hipError_t* err) {
  std::call_once(g_once[dev], [dev] {
    void* p = nullptr;
    g_err[dev] = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    g_ptr[dev] = g_err[dev] == hipSuccess ? p : nullptr;
  });
  *err = g_err[dev];
  return g_ptr[dev];
}

}  // namespace

extern "C" pp_status_t pp_attn_decode_noalloc(const void* q, const void* k_cache, const void* v_cache,
                                              const int32_t* stream_id, int64_t seq_len, int32_t P, int32_t H,
                                              int32_t d, float scale, void* out, pp_dtype_t dtype, void* hip_stream) {
  const size_t need = pp_attn_workspace_bytes(seq_len, P, H, d, dtype);
  if (need == 0) {  // the shape itself is invalid: reuse the decode step's message and status
    return pp_attn_decode(q, k_cache, v_cache, stream_id, seq_len, P, H, d, scale, out, dtype, nullptr, 0, hip_stream);
  }
  if (need > PP_NOALLOC_SCRATCH_BYTES) {
    char msg[200];
    snprintf(msg, sizeof msg, "this shape needs %zu bytes of workspace; the fixed scratch holds %zu", need,
             (size_t)PP_NOALLOC_SCRATCH_BYTES);
    return pp::set_error(PP_ERR_WORKSPACE, msg);
  }
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices)
    return pp::set_error(PP_ERR_HIP, "could not get the current device");
  // the scratch used is the current device's: a stream of another device
  // would run the step against memory of the wrong GPU
  if (hip_stream) {
    int sdev = -1;
    if (hipStreamGetDevice(static_cast<hipStream_t>(hip_stream), &sdev) != hipSuccess)
      return pp::set_error(PP_ERR_HIP, "could not get the stream's device");
    if (sdev != dev) return pp::set_error(PP_ERR_INVALID_ARG, "hip_stream belongs to another device than the current one");
  }
  hipError_t e = hipSuccess;
  void* ws = scratch_address(dev, &e);
  if (!ws) {
    char msg[200];
    snprintf(msg, sizeof msg, "hipGetSymbolAddress of the scratch array failed: %s", hipGetErrorString(e));
    return pp::set_error(PP_ERR_HIP, msg);
  }
  return pp_attn_decode(q, k_cache, v_cache, stream_id, seq_len, P, H, d, scale, out, dtype, ws,
                        (size_t)PP_NOALLOC_SCRATCH_BYTES, hip_stream);
}
