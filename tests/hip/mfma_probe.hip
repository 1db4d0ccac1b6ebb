// Single-wave probes of the gfx950 instructions the expert kernels rely on:
// the scaled FP4 x FP8 (and FP4 x FP6) MFMA (operand lane layout, scale byte
// selection, result layout) and the FP8 (E4M3) conversions.  Test-only; every access is within
// the 64-lane buffers the host passes.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../mxfp4_routed_expert_sqrt_amd/csrc/common.h"

using namespace moe;

template <int JA, int JB, int FA, int FB>
__global__ void probe_mfma_kernel(const u32x4* a, const u32x4* b, const uint32_t* sa, const uint32_t* sb, v4f* d) {
  const int l = threadIdx.x;
  const u32x4 a0 = a[2 * l], a1 = a[2 * l + 1];
  const u32x4 b0 = b[2 * l], b1 = b[2 * l + 1];
  const v8i av = {(int)a0[0], (int)a0[1], (int)a0[2], (int)a0[3], (int)a1[0], (int)a1[1], (int)a1[2], (int)a1[3]};
  const v8i bv = {(int)b0[0], (int)b0[1], (int)b0[2], (int)b0[3], (int)b1[0], (int)b1[1], (int)b1[2], (int)b1[3]};
  v4f c = {0.f, 0.f, 0.f, 0.f};
  d[l] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(av, bv, c, FA, FB, JA, (int)sa[l], JB, (int)sb[l]);
}

__global__ void probe_fp8_kernel(const float* in, uint32_t* packed, float* back, int n4) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= n4) return;
  const uint32_t w = pack4_fp8(in[4 * i], in[4 * i + 1], in[4 * i + 2], in[4 * i + 3]);
  packed[i] = w;
  for (int b = 0; b < 4; ++b) back[4 * i + b] = fp8_byte_to_f32(w, b);
}

// a, b: 64 lanes x 32 bytes; sa, sb: 64 dwords; d: 64 x 4 floats.
// variant 0: A E2M1, B E4M3, scale bytes 0/0; 1: same with scale bytes 2 (A) / 1 (B);
// variant 2: A E2M1, B E2M1, scale bytes 0/0; 3: A E2M1, B E2M3 (FP6), scale bytes 0/0.
extern "C" int probe_mfma(const void* a, const void* b, const void* sa, const void* sb, void* d, int variant) {
  const u32x4* A = (const u32x4*)a;
  const u32x4* B = (const u32x4*)b;
  const uint32_t* SA = (const uint32_t*)sa;
  const uint32_t* SB = (const uint32_t*)sb;
  v4f* D = (v4f*)d;
  if (variant == 0)
    hipLaunchKernelGGL((probe_mfma_kernel<0, 0, 4, 0>), dim3(1), dim3(64), 0, 0, A, B, SA, SB, D);
  else if (variant == 1)
    hipLaunchKernelGGL((probe_mfma_kernel<2, 1, 4, 0>), dim3(1), dim3(64), 0, 0, A, B, SA, SB, D);
  else if (variant == 2)
    hipLaunchKernelGGL((probe_mfma_kernel<0, 0, 4, 4>), dim3(1), dim3(64), 0, 0, A, B, SA, SB, D);
  else if (variant == 3)
    hipLaunchKernelGGL((probe_mfma_kernel<0, 0, 4, 2>), dim3(1), dim3(64), 0, 0, A, B, SA, SB, D);
  else
    return -1;
  if (hipGetLastError() != hipSuccess) return -4;
  return hipDeviceSynchronize() == hipSuccess ? 0 : -4;
}

extern "C" int probe_fp8(const void* in, void* packed, void* back, int n4) {
  if (n4 <= 0) return 0;
  hipLaunchKernelGGL(probe_fp8_kernel, dim3((n4 + 255) / 256), dim3(256), 0, 0, (const float*)in, (uint32_t*)packed,
                     (float*)back, n4);
  if (hipGetLastError() != hipSuccess) return -4;
  return hipDeviceSynchronize() == hipSuccess ? 0 : -4;
}

// Two-term FP6 split of n blocks of 32 floats (split_fp6_32, the helper the
// prologue and the tall gate/up epilogue use): codes [n][2][6] dwords,
// exponents [n][2], residual after term 1 [n][32] (ev/od interleaved back).
__global__ void probe_fp6_kernel(const float* in, uint32_t* codes, int* exps, float* res, int n) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= n) return;
  v16f ev, od;
  for (int j = 0; j < 16; ++j) {
    ev[j] = in[32 * i + 2 * j];
    od[j] = in[32 * i + 2 * j + 1];
  }
  u32x6 t1, t2;
  int e1, e2;
  split_fp6_32(ev, od, &t1, &t2, &e1, &e2);
  for (int j = 0; j < 6; ++j) {
    codes[12 * i + j] = t1[j];
    codes[12 * i + 6 + j] = t2[j];
  }
  exps[2 * i] = e1;
  exps[2 * i + 1] = e2;
  for (int j = 0; j < 16; ++j) {
    res[32 * i + 2 * j] = ev[j];
    res[32 * i + 2 * j + 1] = od[j];
  }
}

// swap32 and swap16 on one wave: in [2][64] (x then y), out [4][64]
// (x, y after swap32; x, y after swap16, each from the inputs).
__global__ void probe_swap_kernel(const float* in, float* out) {
  const int l = threadIdx.x;
  float x = in[l], y = in[64 + l];
  swap32(x, y);
  out[l] = x;
  out[64 + l] = y;
  x = in[l];
  y = in[64 + l];
  swap16(x, y);
  out[128 + l] = x;
  out[192 + l] = y;
}

extern "C" int probe_fp6(const void* in, void* codes, void* exps, void* res, int n) {
  if (n <= 0) return 0;
  hipLaunchKernelGGL(probe_fp6_kernel, dim3((n + 63) / 64), dim3(64), 0, 0, (const float*)in, (uint32_t*)codes,
                     (int*)exps, (float*)res, n);
  if (hipGetLastError() != hipSuccess) return -4;
  return hipDeviceSynchronize() == hipSuccess ? 0 : -4;
}

extern "C" int probe_swap(const void* in, void* out) {
  hipLaunchKernelGGL(probe_swap_kernel, dim3(1), dim3(64), 0, 0, (const float*)in, (float*)out);
  if (hipGetLastError() != hipSuccess) return -4;
  return hipDeviceSynchronize() == hipSuccess ? 0 : -4;
}
