// Allocation-free decode: ekv_decode_attention with its split scratch taken
// from a fixed device array of this library instead of a caller buffer.
//
// For callers that cannot allocate device memory (code under graph capture,
// tight serving loops, harnesses that forbid allocation).  The kernels, plan
// and results are those of ekv_decode_attention; only where the partial
// results live differs.
//
// The array is a file-scope __device__ variable: every GPU the library runs
// on holds its own copy, at its own address, until the process ends.  In
// host code the variable's name is only a host-side stand-in, so its device
// address is looked up once per device (hipGetSymbolAddress, with that device
// current) and that address, never the name, is what the kernels receive.
// Calls on one GPU share the array: calls that overlap in time on one GPU
// (different streams, or different host threads without ordering) race.
#include <mutex>

#include "ekv.h"
#include "ekv_internal.hpp"

namespace {

constexpr size_t kNoAllocBytes = EKV_NOALLOC_SCRATCH_BYTES;
constexpr int kMaxDevices = 64;

}  // namespace

static __device__ __align__(256) unsigned char scratch[kNoAllocBytes];

namespace {

std::mutex g_mu;
void* g_scratch_ptr[kMaxDevices];  // device address of `scratch` per device, once looked up

// Device the launch goes to: the stream's device, else the current one.
hipError_t launch_device(void* stream, int* dev) {
  if (stream) {
    hipDevice_t d;
    const hipError_t e = hipStreamGetDevice(static_cast<hipStream_t>(stream), &d);
    if (e != hipSuccess) return e;
    *dev = (int)d;
    return hipSuccess;
  }
  return hipGetDevice(dev);
}

// Device address of this device's copy of `scratch` (looked up on the first
// call on that device, with that device current).
ekv_status scratch_address(int dev, void** out) {
  if (dev < 0 || dev >= kMaxDevices)
    return ekv::fail(EKV_ERR_UNSUPPORTED, "device %d outside the %d devices the static scratch table covers", dev,
                     kMaxDevices);
  std::lock_guard<std::mutex> lock(g_mu);
  if (!g_scratch_ptr[dev]) {
    int cur = -1;
    hipError_t e = hipGetDevice(&cur);
    if (e != hipSuccess) return ekv::hip_status(e, "hipGetDevice");
    if (cur != dev && (e = hipSetDevice(dev)) != hipSuccess) return ekv::hip_status(e, "hipSetDevice");
    void* ptr = nullptr;
    e = hipGetSymbolAddress((void**)&ptr, HIP_SYMBOL(scratch));
    const hipError_t back = cur != dev ? hipSetDevice(cur) : hipSuccess;
    if (e != hipSuccess) return ekv::hip_status(e, "hipGetSymbolAddress of the static decode scratch");
    if (back != hipSuccess) return ekv::hip_status(back, "hipSetDevice");
    if (!ptr || ((uintptr_t)ptr & 255u) != 0)
      return ekv::fail(EKV_ERR_HIP, "static decode scratch has no usable device address");
    g_scratch_ptr[dev] = ptr;
  }
  *out = g_scratch_ptr[dev];
  return EKV_OK;
}

}  // namespace

extern "C" {

ekv_status ekv_decode_attention_noalloc(const ekv_paged_kv* kv, const void* q, int32_t batch,
                                        int32_t num_q_heads, const int32_t* page_table, int32_t pt_stride,
                                        const uint8_t* fidelity, const int32_t* seq_lens, int32_t max_seq_len,
                                        float sm_scale, void* out, ekv_dtype out_dtype, float* lse,
                                        int32_t pages_per_split, void* stream) {
  if (kv) {
    const size_t need = ekv_decode_scratch_bytes(batch, num_q_heads, kv->num_kv_heads, kv->head_dim, max_seq_len,
                                                 pages_per_split);
    if (need > kNoAllocBytes)
      return ekv::fail(EKV_ERR_WORKSPACE_TOO_SMALL,
                       "this plan needs %zu scratch bytes, more than the %zu bytes of the static decode scratch "
                       "(use ekv_decode_attention with a caller buffer, or a plan with fewer splits)",
                       need, kNoAllocBytes);
  }
  int dev = -1;
  const hipError_t e = launch_device(stream, &dev);
  if (e != hipSuccess) return ekv::hip_status(e, "device of the stream");
  void* ptr = nullptr;
  const ekv_status s = scratch_address(dev, &ptr);
  if (s != EKV_OK) return s;
  return ekv::decode_entry(kv, q, batch, num_q_heads, page_table, pt_stride, fidelity, nullptr, 0, seq_lens,
                           max_seq_len, sm_scale, out, out_dtype, lse, pages_per_split, ptr, kNoAllocBytes,
                           stream);
}

}  // extern "C"
