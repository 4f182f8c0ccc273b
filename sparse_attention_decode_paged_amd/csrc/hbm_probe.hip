// Streaming-read reference for the HBM roofline: one pass of 16-byte nontemporal loads
// over a buffer, nothing written. Its rate is the ceiling that a kernel reading each
// byte once can reach on this device, next to the nominal 8 TB/s.
#include "common.h"
#include "internal.h"

namespace dsa {

// Workgroup g reads the 16-KB chunks g, g + G, g + 2G, ... (G = grid size): thread t
// takes 16-byte words t, t + 256, t + 512 and t + 768 of a chunk, so every load
// instruction covers 4 KB of consecutive lines and four are in flight per thread. A
// partial last chunk is read word by word. The XOR of everything read is stored only
// if it equals a fixed constant, which keeps the loads without writing.
__global__ __launch_bounds__(256) void hbm_read_kernel(const v4i* __restrict__ p, int64_t n16,
                                                       uint32_t* __restrict__ sink) {
  const int64_t nfull = n16 / 1024;  // whole chunks
  uint32_t acc = 0;
  for (int64_t ch = blockIdx.x; ch < nfull; ch += gridDim.x) {
    const v4i* q = p + ch * 1024 + threadIdx.x;
    const v4i a = __builtin_nontemporal_load(q);
    const v4i b = __builtin_nontemporal_load(q + 256);
    const v4i c = __builtin_nontemporal_load(q + 512);
    const v4i d = __builtin_nontemporal_load(q + 768);
    const v4i x = (a ^ b) ^ (c ^ d);
    acc ^= (uint32_t)(x[0] ^ x[1] ^ x[2] ^ x[3]);
  }
  for (int64_t i = nfull * 1024 + (int64_t)blockIdx.x * 256 + threadIdx.x; i < n16; i += (int64_t)gridDim.x * 256) {
    const v4i a = __builtin_nontemporal_load(p + i);
    acc ^= (uint32_t)(a[0] ^ a[1] ^ a[2] ^ a[3]);
  }
  if (acc == 0x9E3779B9u) sink[0] = acc;
}

hipError_t launch_hbm_read(const void* p, size_t bytes, uint32_t* sink, int grid, hipStream_t stream) {
  hipLaunchKernelGGL(hbm_read_kernel, dim3(grid), dim3(256), 0, stream, static_cast<const v4i*>(p),
                     (int64_t)(bytes / 16), sink);
  return hipGetLastError();
}

}  // namespace dsa
