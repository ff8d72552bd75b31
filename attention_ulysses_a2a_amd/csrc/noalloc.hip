// xstage_attn_a2a_fwd_noalloc: the fused call with its split workspace in a static device
// array, for callers that cannot allocate (code under stream capture, serving loops, hosts
// that forbid allocation): the call allocates nothing, ever.
//
// `scratch` is a file-scope device array of kScratchBytes, one copy per GPU, loaded with the
// code object and held until the process ends.  Its name in host code is only a host-side
// stand-in: the device address of each GPU's copy comes from hipGetSymbolAddress, taken once
// per device (with that device current) on the first call there, and only that address is
// passed to kernels.  The same call zeroes the copy's arrival counters with a fill kernel
// on its stream; every call leaves them at zero.  All calls on one GPU share its copy, so
// calls that may overlap on one GPU (different streams, threads) race.
#include <mutex>

#include "attn_a2a.hpp"
#include "common.hpp"
#include "validate.hpp"
#include "workspace.hpp"

namespace xstage {

namespace {

// 32 MiB: the arrival counters (kCounterAreaBytes) and the split partials of every plan
// that fits the rest (the FLUX-1024 share's fastest plan needs 15.2 MiB).
constexpr size_t kScratchBytes = size_t(32) << 20;
static_assert(kScratchBytes > kCounterAreaBytes, "scratch must hold the counters");

static __device__ __align__(256) unsigned char scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_mu;
void* g_ptr[kMaxDevices] = {};

__global__ void zero_counters(uint32_t* p, int n) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) p[i] = 0u;
}

// Device address of the current device's copy of `scratch`, looked up (and its counters
// zeroed on `stream`) on the first call on that device; nullptr on a HIP error.
void* scratch_ptr(hipStream_t stream) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
  std::lock_guard<std::mutex> lk(g_mu);
  if (g_ptr[dev] == nullptr) {
    void* ptr = nullptr;
    if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || ptr == nullptr) return nullptr;
    constexpr int n = (int)(kCounterAreaBytes / 4);
    hipLaunchKernelGGL(zero_counters, dim3((n + 255) / 256), dim3(256), 0, stream, static_cast<uint32_t*>(ptr), n);
    if (hipGetLastError() != hipSuccess) return nullptr;
    g_ptr[dev] = ptr;
  }
  return g_ptr[dev];
}

}  // namespace
}  // namespace xstage

using namespace xstage;

extern "C" int xstage_attn_a2a_fwd_noalloc(const void* q, const void* k, const void* v, void* const* out_slabs, int B,
                                           int S, int H_local, int D, int P, float scale, void* stream) {
  int st = check_shape(B, S, H_local, D, P);
  if (st != XSTAGE_OK) return st;
  st = check_qkv(q, k, v, scale);
  if (st != XSTAGE_OK) return st;
  const unsigned long long tb = tensor_bytes(B, S, H_local, D);
  const Range others[3] = {range_of(q, tb), range_of(k, tb), range_of(v, tb)};
  st = check_slabs(out_slabs, P, tb / (unsigned long long)P, others, 3);
  if (st != XSTAGE_OK) return st;
  // The plan is the one a workspace of kScratchBytes gives; one that needed more would be
  // refused here rather than run past the array.
  if (attn_ws_used(B, S, H_local, D, kScratchBytes) > kScratchBytes) return XSTAGE_ERR_UNSUPPORTED;
  hipStream_t s = static_cast<hipStream_t>(stream);
  void* ws = scratch_ptr(s);
  if (ws == nullptr) return XSTAGE_ERR_HIP;
  SlabTable t;
  for (int i = 0; i < XSTAGE_MAX_P; ++i) t.p[i] = i < P ? static_cast<uint16_t*>(out_slabs[i]) : nullptr;
  return launch_attn_any(q, k, v, t, B, S, H_local, D, P, scale, ws, kScratchBytes, s, 0, nullptr, nullptr);
}
