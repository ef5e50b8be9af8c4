// Debug scan of output tensors for non-finite values (enabled per call by the
// ATTN_CHECK_FINITE environment variable in the C ABI).  Not on any hot path:
// it runs after a call's kernels and waits for them.
#include <algorithm>
#include <mutex>

#include "attn_device.h"
#include "attn_internal.h"

// One buffer of results per device, held until the process ends; its device
// address comes from hipGetSymbolAddress, looked up once per device with that
// device current (the array's name is not a device address in host code).
static __device__ __align__(256) unsigned long long finite_first[attn::kMaxFiniteViews];

namespace attn {
namespace {

constexpr int NT = 256;

// Every first[i] starts at the largest index ("none found").
__global__ __launch_bounds__(NT) void finite_reset_kernel(unsigned long long* first, int n) {
  const int i = blockIdx.x * NT + threadIdx.x;
  if (i < n) first[i] = ~0ull;
}

// Grid-stride walk over the view in flat index order; each bad element offers
// its index to the minimum.
__global__ __launch_bounds__(NT) void finite_scan_kernel(FiniteView v, unsigned long long* first) {
  const int64_t total = v.n[0] * v.n[1] * v.n[2] * v.n[3];
  const int64_t step = (int64_t)gridDim.x * NT;
  for (int64_t i = (int64_t)blockIdx.x * NT + threadIdx.x; i < total; i += step) {
    int64_t r = i, off = 0;
#pragma unroll
    for (int k = 3; k >= 0; --k) {
      off += (r % v.n[k]) * v.st[k];
      r /= v.n[k];
    }
    const float x = v.f32 ? ((const float*)v.ptr)[off] : bf16_to_f32(((const u16*)v.ptr)[off]);
    const bool nan = x != x;
    const bool inf = fabsf(x) == __builtin_huge_valf();
    if (nan || (inf && !(v.allow_neg_inf && x < 0.f))) atomicMin(first, (unsigned long long)i);
  }
}

constexpr int kMaxDevices = 64;
std::once_flag g_once[kMaxDevices];
unsigned long long* g_ptr[kMaxDevices];
hipError_t g_err[kMaxDevices];
std::mutex g_mu;

}  // namespace

hipError_t finite_scan(const FiniteView* v, int n, hipStream_t s, int64_t* first) {
  if (n < 0 || n > kMaxFiniteViews) return hipErrorInvalidValue;
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::call_once(g_once[dev], [dev] {
    g_err[dev] = hipGetSymbolAddress((void**)&g_ptr[dev], HIP_SYMBOL(finite_first));
  });
  if (g_err[dev] != hipSuccess) return g_err[dev];
  unsigned long long* buf = g_ptr[dev];
  std::lock_guard<std::mutex> lock(g_mu);
  hipLaunchKernelGGL(finite_reset_kernel, dim3((kMaxFiniteViews + NT - 1) / NT), dim3(NT), 0, s, buf,
                     kMaxFiniteViews);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  for (int i = 0; i < n; ++i) {
    const int64_t total = v[i].n[0] * v[i].n[1] * v[i].n[2] * v[i].n[3];
    if (total <= 0 || !v[i].ptr) continue;
    const int64_t blocks = std::min<int64_t>((total + NT - 1) / NT, 8192);
    hipLaunchKernelGGL(finite_scan_kernel, dim3((unsigned)blocks), dim3(NT), 0, s, v[i], buf + i);
    if ((e = hipGetLastError()) != hipSuccess) return e;
  }
  unsigned long long host[kMaxFiniteViews];
  if ((e = hipMemcpyAsync(host, buf, sizeof(unsigned long long) * (size_t)n, hipMemcpyDeviceToHost, s)) !=
      hipSuccess)
    return e;
  if ((e = hipStreamSynchronize(s)) != hipSuccess) return e;
  for (int i = 0; i < n; ++i) first[i] = host[i] == ~0ull ? -1 : (int64_t)host[i];
  return hipSuccess;
}

}  // namespace attn
