// Streaming-read probe: the HBM read bandwidth that a plain kernel reaches on
// this GPU, the practical ceiling beside the 8 TB/s of the data sheet against
// which the expert GEMMs' weight streams are measured.  Measurement only: no
// step of the MoE layer calls it.
//
// Workgroup b reads its own contiguous range of the buffer (an equal share,
// rounded up to whole tiles of 256 x kUnroll 16-byte pieces); each thread has
// kUnroll loads in flight, and every load instruction of a wave covers 1 KB of
// consecutive bytes.  The pieces are folded with XOR and each wave stores one
// dword (the sink keeps the loads from being removed).  With `nontemporal` the
// loads carry the non-temporal hint, as the expert kernels' weight loads do
// where each weight byte is read once.  (Contiguous ranges per workgroup
// measured faster than a grid-stride loop over the whole buffer: 7.1 against
// 6.7 TB/s at best, non-temporal, 2 GiB.)
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "hbm_probe.h"

namespace hbm_probe {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
constexpr int kThreads = 256;
constexpr int kUnroll = 16;

template <bool NT>
__global__ void __launch_bounds__(kThreads) hbm_read_kernel(const u32x4* __restrict__ src, size_t n, uint32_t* sink) {
  typedef const __attribute__((address_space(1))) u32x4* gp;
  const gp p = (gp)src;
  constexpr size_t kTile = (size_t)kThreads * kUnroll;
  size_t per = (n + gridDim.x - 1) / gridDim.x;
  per = (per + kTile - 1) / kTile * kTile;
  const size_t b0 = (size_t)blockIdx.x * per;
  const size_t b1 = b0 + per < n ? b0 + per : n;  // b1 <= b0 for workgroups past the end: no loads
  size_t i = b0 + threadIdx.x;
  uint32_t acc = 0;
  for (; i + (kUnroll - 1) * kThreads < b1; i += kTile) {
    u32x4 v[kUnroll];
#pragma unroll
    for (int j = 0; j < kUnroll; ++j)
      v[j] = NT ? __builtin_nontemporal_load(p + i + j * kThreads) : p[i + j * kThreads];
#pragma unroll
    for (int j = 0; j < kUnroll; ++j) acc ^= v[j][0] ^ v[j][1] ^ v[j][2] ^ v[j][3];
  }
  for (; i < b1; i += kThreads) {
    const u32x4 v = NT ? __builtin_nontemporal_load(p + i) : p[i];
    acc ^= v[0] ^ v[1] ^ v[2] ^ v[3];
  }
#pragma unroll
  for (int m = 1; m < 64; m <<= 1) acc ^= __shfl_xor(acc, m, 64);
  if ((threadIdx.x & 63) == 0) sink[(size_t)blockIdx.x * (kThreads / 64) + (threadIdx.x >> 6)] = acc;
}

}  // namespace hbm_probe

using namespace hbm_probe;

extern "C" int hbm_read_probe(const void* src, size_t bytes, int nontemporal, uint32_t* sink, int workgroups,
                              hipStream_t stream) {
  if (src == nullptr || sink == nullptr || workgroups <= 0 || bytes % 16 != 0 || ((uintptr_t)src & 15) != 0)
    return -1;
  const size_t n = bytes / 16;
  if (nontemporal)
    hipLaunchKernelGGL(hbm_read_kernel<true>, dim3((unsigned)workgroups), dim3(kThreads), 0, stream,
                       (const u32x4*)src, n, sink);
  else
    hipLaunchKernelGGL(hbm_read_kernel<false>, dim3((unsigned)workgroups), dim3(kThreads), 0, stream,
                       (const u32x4*)src, n, sink);
  return hipGetLastError() == hipSuccess ? 0 : -4;
}

extern "C" int hbm_probe_sink_words(int workgroups) { return workgroups * (kThreads / 64); }
