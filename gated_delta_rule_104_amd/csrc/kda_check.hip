// Input check of the gate's precondition, used when the "check" option is set.
//
// The kernels assume log alpha in [-1, 0], the lower-bounded decay the pages
// give KDA's gate (blog.csdn.net article on the Kimi K3 report, section 一.1):
// with it the cumulative log-decay inside a 64-token chunk stays within 64 in
// magnitude, and e^{+-g} within the fp32 range.  beta is a mixing weight in
// [0, 1].  This pass reads log_alpha and beta once and ORs a bit into a flag
// for every value out of range or not finite (1: log_alpha, 2: beta); the host
// reads the flag back before launching anything else.
#include <mutex>

#include "kda_device.hpp"
#include "kda_launch.hpp"

namespace kda {

namespace {

// One flag per device (each GPU holds its own copy).  The host reaches it
// through the address hipGetSymbolAddress gives on that device, never through
// the symbol's name.
__device__ unsigned int g_check_bits;

__device__ __forceinline__ unsigned int bad_gate(float x) { return (x >= -1.f && x <= 0.f) ? 0u : 1u; }
__device__ __forceinline__ unsigned int bad_beta(float x) { return (x >= 0.f && x <= 1.f) ? 0u : 2u; }

__device__ __forceinline__ float elem(const bf16* p, long long i) { return (float)p[i]; }
__device__ __forceinline__ float elem(const float* p, long long i) { return p[i]; }

__global__ void kda_check_clear_kernel(unsigned int* bits) { *bits = 0u; }

template <typename T>
__global__ __launch_bounds__(256) void kda_check_kernel(const T* __restrict__ la, long long n_la,
                                                        const T* __restrict__ beta, long long n_beta,
                                                        unsigned int* bits) {
  constexpr int V = 16 / (int)sizeof(T);  // elements per 16-byte load
  const long long stride = (long long)gridDim.x * blockDim.x;
  const long long tid = (long long)blockIdx.x * blockDim.x + threadIdx.x;
  unsigned int b = 0u;
  const long long nv = n_la / V;
  for (long long i = tid; i < nv; i += stride) {
    const u32x4 w = reinterpret_cast<const u32x4*>(la)[i];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      if constexpr (sizeof(T) == 2) {
        b |= bad_gate(__uint_as_float(w[e] << 16));
        b |= bad_gate(__uint_as_float(w[e] & 0xffff0000u));
      } else {
        b |= bad_gate(__uint_as_float(w[e]));
      }
    }
  }
  for (long long i = nv * V + tid; i < n_la; i += stride) b |= bad_gate(elem(la, i));
  for (long long i = tid; i < n_beta; i += stride) b |= bad_beta(elem(beta, i));
  if (b) atomicOr(bits, b);
}

}  // namespace

hipError_t check_gates(const void* la, long long n_la, const void* beta, long long n_beta, bool bf16_io,
                       hipStream_t stream, unsigned int* bits_out) {
  static std::mutex mu;
  static unsigned int* flag[64] = {nullptr};
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= 64) return hipErrorInvalidDevice;
  // one check at a time per process: the flag is shared by every call on a device
  std::lock_guard<std::mutex> lk(mu);
  if (!flag[dev]) {
    void* p = nullptr;
    if ((e = hipGetSymbolAddress(&p, HIP_SYMBOL(g_check_bits))) != hipSuccess) return e;
    flag[dev] = static_cast<unsigned int*>(p);
  }
  unsigned int* f = flag[dev];
  hipLaunchKernelGGL(kda_check_clear_kernel, dim3(1), dim3(1), 0, stream, f);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  const long long work = n_la / 8 > n_beta ? n_la / 8 : n_beta;
  long long nb = (work + 255) / 256;
  if (nb < 1) nb = 1;
  if (nb > 2048) nb = 2048;
  if (bf16_io)
    hipLaunchKernelGGL(kda_check_kernel<bf16>, dim3((unsigned)nb), dim3(256), 0, stream,
                       static_cast<const bf16*>(la), n_la, static_cast<const bf16*>(beta), n_beta, f);
  else
    hipLaunchKernelGGL(kda_check_kernel<float>, dim3((unsigned)nb), dim3(256), 0, stream,
                       static_cast<const float*>(la), n_la, static_cast<const float*>(beta), n_beta, f);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  unsigned int h = 0u;
  if ((e = hipMemcpyAsync(&h, f, sizeof(h), hipMemcpyDeviceToHost, stream)) != hipSuccess) return e;
  if ((e = hipStreamSynchronize(stream)) != hipSuccess) return e;
  *bits_out = h;
  return hipSuccess;
}

}  // namespace kda
