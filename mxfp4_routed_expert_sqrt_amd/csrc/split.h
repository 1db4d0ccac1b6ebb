// Two-term FP8 and FP6 splits of activation rows (device code shared by the
// kernels that produce the splits).
#pragma once
#include "kernels.h"

namespace moe {

// ---------------------------------------------------------------------------
// Two-term FP8 split of activations.  Each 32-value block v is written as
// v ~= q1 * 2^e1 + q2 * 2^e2 with q1, q2 E4M3 and e1, e2 E8M0 shared
// exponents: q1 rounds v / 2^e1, q2 rounds the exact fp32 residual
// (v - q1 * 2^e1) / 2^e2.  For bf16 inputs (8 significant bits) the two 4-bit
// terms reproduce exactly every element of at least 2^-12 of the block's
// largest magnitude (the residual is a multiple of the element's bf16 ulp,
// which the second term's grid, at most 2^-20 of the block maximum, resolves);
// a smaller element next to a large one can miss its low bits, by at most
// half that grid, 2^-21 of the block maximum.
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


// ---------------------------------------------------------------------------
// Two-term FP6 (E2M3) split, used for batches of tall work units: v ~= q1 *
// 2^e1 + q2 * 2^e2 with q1, q2 E2M3 (the same scheme as the FP8 split, made
// by the hardware conversions of split_fp6_32; the second term leaves a
// residual of about 2^-10 of the block maximum).
//
// Row layout: k-step ks occupies 192 bytes at ks*192 (inside a row of the FP8
// split's length), term t at t*96 as two planes of the lane groups' 6-dword
// operands: dwords 0-3 of group g at g*16, dwords 4-5 at 64 + g*8.  Group g
// = the 32-block 4ks+g.  Scales as for the FP8 split.

// Split of one 32-value block t = row * (K/32) + block of x (t < n_rows * K/32),
// FP6 when fp6 is set, else FP8.
__device__ __forceinline__ void split_bf16_block(const uint16_t* __restrict__ x, int K, uint8_t* __restrict__ xq,
                                                 uint8_t* __restrict__ xs, size_t t, bool fp6) {
  const int nkb = K / 32, n_sg = (K / 128 + 3) / 4;
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
  if (fp6) {
    v16f ev, od;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      ev[i] = v[2 * i];
      od[i] = v[2 * i + 1];
    }
    u32x6 w[2];
    int e1, e2;
    split_fp6_32(ev, od, &w[0], &w[1], &e1, &e2);
    uint8_t* step = xq + row * split_q_row_bytes(K) + (size_t)(blk >> 2) * kFp6StepBytes;
    const int g = blk & 3;
#pragma unroll
    for (int term = 0; term < 2; ++term) {
      *(u32x4*)(step + term * kFp6TermBytes + g * 16) = u32x4{w[term][0], w[term][1], w[term][2], w[term][3]};
      *(uint2*)(step + term * kFp6TermBytes + 64 + g * 8) = uint2{w[term][4], w[term][5]};
    }
    uint8_t* srow = xs + row * split_s_row_bytes(K);
    srow[split_scale_offset(0, blk, n_sg)] = (uint8_t)(e1 + 127);
    srow[split_scale_offset(1, blk, n_sg)] = (uint8_t)(e2 + 127);
    return;
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

}  // namespace moe
