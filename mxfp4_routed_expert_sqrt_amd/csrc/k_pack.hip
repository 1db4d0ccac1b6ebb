// Layout kernels: MXFP4 weight packing into MFMA fragments, and the two-term
// FP8 split of bf16 activation rows.
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

// ---------------------------------------------------------------------------
// Two-term FP8 split of activations.  Each 32-value block v is written as
// v ~= q1 * 2^e1 + q2 * 2^e2 with q1, q2 E4M3 and e1, e2 E8M0 shared
// exponents: q1 rounds v / 2^e1, q2 rounds the exact fp32 residual
// (v - q1 * 2^e1) / 2^e2.  For bf16 inputs (8 significant bits) the two 4-bit
// terms reproduce every element of normal range exactly.
//
// Row layout (K values), shaped for the 8-bit operand of the scaled MFMA, whose
// lane group g (lanes 16g..16g+15) reads K values 16g..16g+15 and
// 64+16g..64+16g+15 of each 128-wide k-step: the k-step ks occupies 256
// bytes at ks*256, as [group g][term][32 bytes] with the group's two 16-value
// runs back to back.  Scales [2 terms][n_sg][4][4]: byte (term, block b) at
// ((term*n_sg + ks/4)*4 + b%4)*4 + ks%4 with ks = b/4, so lane group g reads
// the scales of block g of 4 consecutive k-steps as one dword.

__device__ __forceinline__ void split_block32(const float* v, uint32_t* q /*16 dwords*/, int* e1_out,
                                              int* e2_out) {
  float amax = 0.f;
#pragma unroll
  for (int i = 0; i < 32; ++i) amax = fmaxf(amax, fabsf(v[i]));
  const int e1 = split_exponent(amax);
  const float inv1 = ldexpf(1.f, -e1), sc1 = ldexpf(1.f, e1);
  float r[32];
  float amax2 = 0.f;
#pragma unroll
  for (int i = 0; i < 32; i += 4) {
    const uint32_t w = pack4_fp8(v[i] * inv1, v[i + 1] * inv1, v[i + 2] * inv1, v[i + 3] * inv1);
    q[i / 4] = w;
#pragma unroll
    for (int b = 0; b < 4; ++b) {
      r[i + b] = v[i + b] - fp8_byte_to_f32(w, b) * sc1;
      amax2 = fmaxf(amax2, fabsf(r[i + b]));
    }
  }
  const int e2 = split_exponent(amax2);
  const float inv2 = ldexpf(1.f, -e2);
#pragma unroll
  for (int i = 0; i < 32; i += 4)
    q[8 + i / 4] = pack4_fp8(r[i] * inv2, r[i + 1] * inv2, r[i + 2] * inv2, r[i + 3] * inv2);
  *e1_out = e1;
  *e2_out = e2;
}

__device__ __forceinline__ size_t split_scale_offset(int term, int blk, int n_sg) {
  const int ks = blk >> 2;
  return (size_t)(((term * n_sg + (ks >> 2)) * 4 + (blk & 3)) * 4 + (ks & 3));
}

__global__ void __launch_bounds__(256) split_bf16_kernel(const uint16_t* __restrict__ x, int n_rows, int K,
                                                          uint8_t* __restrict__ xq, uint8_t* __restrict__ xs) {
  const int nkb = K / 32, n_sg = (K / 128 + 3) / 4;
  const size_t t = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (t >= (size_t)n_rows * nkb) return;
  const size_t row = t / nkb;
  const int blk = (int)(t % nkb);
  const u32x4* src = (const u32x4*)(x + row * K + (size_t)blk * 32);
  float v[32];
#pragma unroll
  for (int c = 0; c < 4; ++c) {
    const u32x4 w = src[c];
#pragma unroll
    for (int h = 0; h < 4; ++h) {
      v[c * 8 + 2 * h] = __uint_as_float(w[h] << 16);
      v[c * 8 + 2 * h + 1] = __uint_as_float(w[h] & 0xffff0000u);
    }
  }
  uint32_t q[16];
  int e1, e2;
  split_block32(v, q, &e1, &e2);
  // values 16h..16h+15 of block b = 4ks + bb sit in group 2*(bb%2) + h, at byte 16*(bb/2) of its run
  uint8_t* step = xq + row * split_q_row_bytes(K) + (size_t)(blk >> 2) * 256;
  const int bb = blk & 3;
#pragma unroll
  for (int term = 0; term < 2; ++term)
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int g = 2 * (bb & 1) + h;
      const uint32_t* src_q = q + 8 * term + 4 * h;
      *(u32x4*)(step + g * 64 + term * 32 + 16 * (bb >> 1)) = u32x4{src_q[0], src_q[1], src_q[2], src_q[3]};
    }
  uint8_t* srow = xs + row * split_s_row_bytes(K);
  srow[split_scale_offset(0, blk, n_sg)] = (uint8_t)(e1 + 127);
  srow[split_scale_offset(1, blk, n_sg)] = (uint8_t)(e2 + 127);
}

hipError_t launch_split_bf16(const uint16_t* x, int n_rows, int K, uint8_t* xq, uint8_t* xs, hipStream_t stream) {
  const size_t n = (size_t)n_rows * (K / 32);
  if (n == 0) return hipSuccess;
  hipLaunchKernelGGL(split_bf16_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, stream, x, n_rows, K, xq,
                     xs);
  return hipGetLastError();
}

}  // namespace moe
