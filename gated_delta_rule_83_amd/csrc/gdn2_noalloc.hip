// gdn2_noalloc.hip -- gdn2_chunk_forward_noalloc: the prefill with its
// scratch (the split-sequence states and transition matrices) in a static
// device array of this library instead of a caller-supplied workspace, for
// callers that cannot allocate device memory.
//
// The array `scratch` lives in the library's code object: each device that
// runs the library holds its own copy (GDN2_NOALLOC_SCRATCH_BYTES) until the
// process ends. In host code its name is only a host-side stand-in, so its
// device address is looked up once per device with hipGetSymbolAddress, with
// that device current, and only that address is passed to the kernels.
#include <mutex>

#include "gdn2.h"
#include "gdn2_internal.hpp"

namespace {

constexpr size_t kScratchBytes = (size_t)GDN2_NOALLOC_SCRATCH_BYTES;
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

constexpr int kMaxDevices = 128;
std::mutex g_mu;
void *g_scratch_ptr[kMaxDevices];  // device address of `scratch` per device (null: not looked up yet)

// Device address of this device's `scratch`: looked up on the first call on
// the device, with the device current (restored afterwards).
gdn2_status scratch_on(int dev, void **out) {
  if (dev < 0 || dev >= kMaxDevices) return GDN2_ERR_HIP;
  std::lock_guard<std::mutex> lock(g_mu);
  if (!g_scratch_ptr[dev]) {
    int cur = -1;
    if (hipGetDevice(&cur) != hipSuccess) return GDN2_ERR_HIP;
    if (cur != dev && hipSetDevice(dev) != hipSuccess) return GDN2_ERR_HIP;
    void *p = nullptr;
    const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (cur != dev) (void)hipSetDevice(cur);
    if (e != hipSuccess || !p) return GDN2_ERR_HIP;
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return GDN2_OK;
}

}  // namespace

namespace gdn2 {
size_t chunk_forward_workspace_capped(const gdn2_desc *desc, size_t ws_cap);
gdn2_status chunk_forward_capped(const gdn2_desc *d, const void *q, const void *k, const void *v, const float *a,
                                 const float *b, const float *w, const float *S0, void *o, float *S_T,
                                 void *workspace, size_t workspace_bytes, size_t ws_cap, void *stream);
}  // namespace gdn2

extern "C" gdn2_status gdn2_chunk_forward_noalloc(const gdn2_desc *d, const void *q, const void *k, const void *v,
                                                  const float *a, const float *b, const float *w, const float *S0,
                                                  void *o, float *S_T, void *stream) {
  // The split is planned within the scratch: the form whose workspace fits
  // (the output correction needs a row of d_k per token, so long problems
  // run their segments a second time instead). 0 for an invalid
  // description too: the forward then reports it.
  const size_t need = gdn2::chunk_forward_workspace_capped(d, kScratchBytes);
  if (need > kScratchBytes) return GDN2_ERR_SCRATCH;
  void *ws = nullptr;
  if (need > 0) {
    // the device the work is enqueued on: the stream's (the current one for
    // the null stream)
    int dev = -1;
    hipStream_t st = reinterpret_cast<hipStream_t>(stream);
    if ((st ? hipStreamGetDevice(st, &dev) : hipGetDevice(&dev)) != hipSuccess) return GDN2_ERR_HIP;
    const gdn2_status s = scratch_on(dev, &ws);
    if (s != GDN2_OK) return s;
  }
  // Every piece of the split's scratch is written before it is read (each
  // segment's state and transition by the first pass), so nothing needs
  // clearing between calls.
  return gdn2::chunk_forward_capped(d, q, k, v, a, b, w, S0, o, S_T, ws, need > 0 ? kScratchBytes : 0, kScratchBytes,
                                    stream);
}
