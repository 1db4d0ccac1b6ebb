// Weight packing: MXFP4 matrices from the natural layout into MFMA fragments.
#include "kernels.h"

namespace moe {

// One thread per 16-byte fragment lane: copies the 32 E2M1 values of one
// (row, 32-block) so that a wave's 64 lanes read one contiguous kilobyte.
__global__ void __launch_bounds__(256) pack_q_kernel(const uint8_t* __restrict__ q, int n_mat, int rows, int K,
                                                      uint8_t* __restrict__ q_out) {
  const int nks = K / 128;
  const size_t per_mat = (size_t)(rows / 16) * nks * 64;  // lanes per matrix
  const size_t total = per_mat * n_mat;
  for (size_t t = (size_t)blockIdx.x * blockDim.x + threadIdx.x; t < total; t += (size_t)gridDim.x * blockDim.x) {
    const size_t m = t / per_mat;
    const size_t rem = t % per_mat;
    const int lane = (int)(rem % 64);
    const size_t frag = rem / 64;
    const int ks = (int)(frag % nks), rt = (int)(frag / nks);
    const int row = rt * 16 + (lane & 15), blk = 4 * ks + (lane >> 4);
    const uint8_t* src = q + (m * rows + row) * (size_t)(K / 2) + (size_t)blk * 16;
    uint8_t* dst = q_out + m * (size_t)rows * (K / 2) + frag * 1024 + (size_t)lane * 16;
    *(u32x4*)dst = *(const u32x4*)src;
  }
}

// One thread per scale-group lane: gathers the 4 E8M0 bytes a lane uses over
// 4 consecutive k-steps into one dword.
__global__ void __launch_bounds__(256) pack_s_kernel(const uint8_t* __restrict__ s, int n_mat, int rows, int K,
                                                      uint8_t* __restrict__ s_out) {
  const int nks = K / 128, n_sg = (nks + 3) / 4, nkb = K / 32;
  const size_t per_mat = (size_t)(rows / 16) * n_sg * 64;
  const size_t total = per_mat * n_mat;
  for (size_t t = (size_t)blockIdx.x * blockDim.x + threadIdx.x; t < total; t += (size_t)gridDim.x * blockDim.x) {
    const size_t m = t / per_mat;
    const size_t rem = t % per_mat;
    const int lane = (int)(rem % 64);
    const size_t grp = rem / 64;
    const int sg = (int)(grp % n_sg), rt = (int)(grp / n_sg);
    const int row = rt * 16 + (lane & 15);
    uint32_t word = 0;
    for (int j = 0; j < 4; ++j) {
      const int ks = 4 * sg + j;
      uint32_t b = 127;
      if (ks < nks) b = s[(m * rows + row) * (size_t)nkb + 4 * ks + (lane >> 4)];
      word |= b << (8 * j);
    }
    *(uint32_t*)(s_out + m * packed_s_bytes(rows, K) + grp * 256 + (size_t)lane * 4) = word;
  }
}

// bf16 matrices into bf16-MFMA fragments (v_mfma_f32_16x16x32_bf16 A
// operand): one thread per 16-byte lane piece; fragment (rt, ks) of a matrix
// [rows][K] at byte (rt * K/32 + ks) * 1024, lane l = row 16 rt + l % 16,
// values 32 ks + 8 (l / 16) .. +7.
__global__ void __launch_bounds__(256) pack_bf16_kernel(const uint8_t* __restrict__ w, int n_mat, int rows, int K,
                                                         uint8_t* __restrict__ out) {
  const int nks = K / 32;
  const size_t per_mat = (size_t)(rows / 16) * nks * 64;
  const size_t total = per_mat * n_mat;
  for (size_t t = (size_t)blockIdx.x * blockDim.x + threadIdx.x; t < total; t += (size_t)gridDim.x * blockDim.x) {
    const size_t m = t / per_mat;
    const size_t rem = t % per_mat;
    const int lane = (int)(rem % 64);
    const size_t frag = rem / 64;
    const int ks = (int)(frag % nks), rt = (int)(frag / nks);
    const int row = rt * 16 + (lane & 15), k0 = 32 * ks + 8 * (lane >> 4);
    const uint8_t* src = w + ((m * rows + row) * (size_t)K + k0) * 2;
    uint8_t* dst = out + m * (size_t)rows * K * 2 + frag * 1024 + (size_t)lane * 16;
    *(u32x4*)dst = *(const u32x4*)src;
  }
}

hipError_t launch_pack_bf16(const uint8_t* w, int n_mat, int rows, int K, uint8_t* out, hipStream_t stream) {
  const size_t n = (size_t)n_mat * (rows / 16) * (K / 32) * 64;
  const int b = (int)((n + 255) / 256 < 65536 ? (n + 255) / 256 : 65536);
  if (b > 0) hipLaunchKernelGGL(pack_bf16_kernel, dim3(b), dim3(256), 0, stream, w, n_mat, rows, K, out);
  return hipGetLastError();
}

hipError_t launch_pack_mxfp4(const uint8_t* q, const uint8_t* s, int n_mat, int rows, int K, uint8_t* q_out,
                             uint8_t* s_out, hipStream_t stream) {
  const size_t nq = (size_t)n_mat * (rows / 16) * (K / 128) * 64;
  const size_t ns = (size_t)n_mat * (rows / 16) * ((K / 128 + 3) / 4) * 64;
  const int bq = (int)((nq + 255) / 256 < 65536 ? (nq + 255) / 256 : 65536);
  const int bs = (int)((ns + 255) / 256 < 65536 ? (ns + 255) / 256 : 65536);
  if (bq > 0) hipLaunchKernelGGL(pack_q_kernel, dim3(bq), dim3(256), 0, stream, q, n_mat, rows, K, q_out);
  if (bs > 0) hipLaunchKernelGGL(pack_s_kernel, dim3(bs), dim3(256), 0, stream, s, n_mat, rows, K, s_out);
  return hipGetLastError();
}

}  // namespace moe
