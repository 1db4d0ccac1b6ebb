// Grouped expert GEMMs on v_mfma_scale_f32_16x16x128_f8f6f4.
//
// A operand = the expert's MXFP4 weight rows (E2M1, with their E8M0 scales
// fed to the MFMA directly, so there is no dequantisation step); B operand =
// activations as two FP8 (E4M3) terms with per-32 E8M0 scales (x ~= q1*2^e1 +
// q2*2^e2), so every product is weight * (q1 + q2) accumulated in fp32.
//
// One workgroup = one work unit = (group of <= 16 rows of one expert = one
// MFMA column tile, 128 output features).  gate/up: 4 waves x 32 features (two
// 16-row weight tiles per matrix); down: 2 waves x 64 features (four tiles).
// Weight fragments are read straight from HBM into registers: the packed
// layout makes each wave's 16-byte-per-lane load one contiguous kilobyte, and
// every weight byte is used by exactly one wave, so no LDS staging is needed.
//
// Lane layout of the 16x16x128 scaled MFMA (measured on gfx950; the probe test
// pins it): lane l supplies row/column l%16; a 4-bit operand holds K values
// 32*(l/16)..+31 (low nibble first), an 8-bit operand holds K values
// 16*(l/16)..+15 and 64+16*(l/16)..+15; the E8M0 scale of 32-block b of
// row/column n is byte `opsel` of lane n+16b's scale register; the fp32 result
// has D[4*(l/16) + i][l%16] in element i of lane l.
#include "kernels.h"

namespace moe {

__device__ __forceinline__ size_t split_scale_offset_h(int term, int blk, int n_sg) {
  const int ks = blk >> 2;
  return (size_t)(((term * n_sg + (ks >> 2)) * 4 + (blk & 3)) * 4 + (ks & 3));
}

template <int J>
__device__ __forceinline__ v4f mfma_fp4_fp8(const u32x4& a, const v8i& b, const v4f& c, uint32_t sa, uint32_t sb) {
  const v8i av = {(int)a[0], (int)a[1], (int)a[2], (int)a[3], 0, 0, 0, 0};
  return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(av, b, c, 4 /* A: E2M1 */, 0 /* B: E4M3 */, J, (int)sa, J,
                                                          (int)sb);
}

// Operand fragments of one 128-wide k-step: NA weight tiles, NT token tiles x 2 terms.
template <int NA, int NT>
struct Frag {
  u32x4 A[NA];
  v8i B[NT][2];
};

template <int NA, int NT>
__device__ __forceinline__ void load_frag(Frag<NA, NT>& f, const uint8_t* const (&aq)[NA],
                                          const uint8_t* const (&bq)[NT], int ks) {
#pragma unroll
  for (int a = 0; a < NA; ++a) f.A[a] = *(const u32x4*)(aq[a] + (size_t)ks * 1024);
#pragma unroll
  for (int t = 0; t < NT; ++t) {
#pragma unroll
    for (int term = 0; term < 2; ++term) {
      const u32x4 lo = *(const u32x4*)(bq[t] + (size_t)ks * 256 + term * 32);
      const u32x4 hi = *(const u32x4*)(bq[t] + (size_t)ks * 256 + term * 32 + 16);
      f.B[t][term] = v8i{(int)lo[0], (int)lo[1], (int)lo[2], (int)lo[3], (int)hi[0], (int)hi[1], (int)hi[2], (int)hi[3]};
    }
  }
}

// J = k-step index within its group of 4 = the scale byte to use.
template <int J, int NA, int NT>
__device__ __forceinline__ void mma_frag(const Frag<NA, NT>& f, const uint32_t (&sa)[NA], const uint32_t (&sb)[NT][2],
                                         v4f (&acc)[NA][NT]) {
#pragma unroll
  for (int a = 0; a < NA; ++a)
#pragma unroll
    for (int t = 0; t < NT; ++t)
#pragma unroll
      for (int term = 0; term < 2; ++term) acc[a][t] = mfma_fp4_fp8<J>(f.A[a], f.B[t][term], acc[a][t], sa[a], sb[t][term]);
}

template <int NA, int NT>
__device__ __forceinline__ void load_scales(uint32_t (&sa)[NA], uint32_t (&sb)[NT][2], const uint8_t* const (&as)[NA],
                                            const uint8_t* const (&bs)[NT], int sg, int n_sg) {
#pragma unroll
  for (int a = 0; a < NA; ++a) sa[a] = *(const uint32_t*)(as[a] + (size_t)sg * 256);
#pragma unroll
  for (int t = 0; t < NT; ++t) {
    sb[t][0] = *(const uint32_t*)(bs[t] + (size_t)sg * 16);
    sb[t][1] = *(const uint32_t*)(bs[t] + (size_t)(n_sg + sg) * 16);
  }
}

// K loop with a 4-deep register ring: while k-step ks is multiplied, the
// fragments of ks+1..ks+3 are in flight, and the scales of the next group of
// 4 k-steps are fetched one group ahead, so each wave keeps ~3 k-steps of
// weight bytes outstanding.  Every load is unconditional (indices past the
// end are clamped to the last k-step, a cache hit) so that the compiler's
// in-order load counter waits only for the fragment about to be used; only
// the MFMAs of a partial last group are skipped.
template <int NA, int NT>
__device__ __forceinline__ void mainloop(const uint8_t* const (&aq)[NA], const uint8_t* const (&as)[NA],
                                         const uint8_t* const (&bq)[NT], const uint8_t* const (&bs)[NT], int nks,
                                         v4f (&acc)[NA][NT]) {
  const int n_sg = (nks + 3) / 4, last = nks - 1;
  Frag<NA, NT> f0, f1, f2, f3;
  uint32_t sa[NA], sb[NT][2], sa_n[NA], sb_n[NT][2];
  load_scales(sa, sb, as, bs, 0, n_sg);
  load_frag(f0, aq, bq, 0);
  load_frag(f1, aq, bq, min(1, last));
  load_frag(f2, aq, bq, min(2, last));
  // sched_barrier(0) keeps the compiler from moving loads across these
  // points, so the issue order (and hence each wait) is exactly as written.
  for (int sg = 0; sg < n_sg; ++sg) {
    const int k0 = 4 * sg;
    load_scales(sa_n, sb_n, as, bs, min(sg + 1, n_sg - 1), n_sg);
    load_frag(f3, aq, bq, min(k0 + 3, last));
    __builtin_amdgcn_sched_barrier(0);
    mma_frag<0>(f0, sa, sb, acc);
    __builtin_amdgcn_sched_barrier(0);
    load_frag(f0, aq, bq, min(k0 + 4, last));
    __builtin_amdgcn_sched_barrier(0);
    if (k0 + 1 < nks) mma_frag<1>(f1, sa, sb, acc);
    __builtin_amdgcn_sched_barrier(0);
    load_frag(f1, aq, bq, min(k0 + 5, last));
    __builtin_amdgcn_sched_barrier(0);
    if (k0 + 2 < nks) mma_frag<2>(f2, sa, sb, acc);
    __builtin_amdgcn_sched_barrier(0);
    load_frag(f2, aq, bq, min(k0 + 6, last));
    __builtin_amdgcn_sched_barrier(0);
    if (k0 + 3 < nks) mma_frag<3>(f3, sa, sb, acc);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int a = 0; a < NA; ++a) sa[a] = sa_n[a];
#pragma unroll
    for (int t = 0; t < NT; ++t) {
      sb[t][0] = sb_n[t][0];
      sb[t][1] = sb_n[t][1];
    }
  }
}

// ---------------------------------------------------------------------------
// gate/up: h = silu(min(gate, L)) * clamp(up, -L, L), written as the two-term
// FP8 split that the down GEMM consumes (same layout as the x split, K = I).

template <int NT>
__device__ __forceinline__ void gateup_unit(const ExpertArgs& a, const Group g, int fb) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int col = lane & 15, grp = lane >> 4;
  const int K = a.K, R = a.R, nks = K / 128, n_sg = (nks + 3) / 4;
  const int f0 = fb * kFeatPerWG + wave * kFeatPerWave, rt0 = f0 / 16;
  const bool shared = g.e == a.E;
  const size_t mq = packed_q_bytes(R, K), ms = packed_s_bytes(R, K);
  const uint8_t* gq = shared ? a.sq0 : a.q0 + (size_t)g.e * mq;
  const uint8_t* gs = shared ? a.ss0 : a.s0 + (size_t)g.e * ms;
  const uint8_t* uq = shared ? a.sq1 : a.q1 + (size_t)g.e * mq;
  const uint8_t* us = shared ? a.ss1 : a.s1 + (size_t)g.e * ms;
  const size_t tq = (size_t)nks * 1024, ts = (size_t)n_sg * 256;  // one 16-row tile
  const uint8_t* aq[4] = {gq + rt0 * tq + lane * 16, gq + (rt0 + 1) * tq + lane * 16, uq + rt0 * tq + lane * 16,
                          uq + (rt0 + 1) * tq + lane * 16};
  const uint8_t* as[4] = {gs + rt0 * ts + lane * 4, gs + (rt0 + 1) * ts + lane * 4, us + rt0 * ts + lane * 4,
                          us + (rt0 + 1) * ts + lane * 4};
  const uint8_t* bq[NT];
  const uint8_t* bs[NT];
#pragma unroll
  for (int t = 0; t < NT; ++t) {
    const int i = t * 16 + col;
    const int p = g.p0 + (i < g.cnt ? i : 0);  // padding columns reuse the group's first row
    const int row = shared ? p - a.P : a.perm[p] / a.k;
    bq[t] = a.aq + (size_t)row * split_q_row_bytes(K) + grp * 64;
    bs[t] = a.as + (size_t)row * split_s_row_bytes(K) + grp * 4;
  }
  v4f acc[4][NT];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int t = 0; t < NT; ++t) acc[i][t] = v4f{0.f, 0.f, 0.f, 0.f};
  mainloop<4, NT>(aq, as, bq, bs, nks, acc);

  const int n_sg_h = (R / 128 + 3) / 4;
  const int blk_h = f0 / 32;
  const float L = a.limit;
#pragma unroll
  for (int t = 0; t < NT; ++t) {
    float h[8];
#pragma unroll
    for (int tt = 0; tt < 2; ++tt)
#pragma unroll
      for (int ii = 0; ii < 4; ++ii) {
        float gv = acc[tt][t][ii], uv = acc[2 + tt][t][ii];
        if (L > 0.f) {
          gv = fminf(gv, L);
          uv = fminf(fmaxf(uv, -L), L);
        }
        h[tt * 4 + ii] = gv / (1.f + __expf(-gv)) * uv;
      }
    // 32-feature block of one token = 4 lanes (grp 0..3) x 8 values
    float amax = 0.f;
#pragma unroll
    for (int j = 0; j < 8; ++j) amax = fmaxf(amax, fabsf(h[j]));
    amax = shfl_xor_max<16>(amax);
    amax = shfl_xor_max<32>(amax);
    const int e1 = split_exponent(amax);
    const float inv1 = ldexpf(1.f, -e1), sc1 = ldexpf(1.f, e1);
    uint32_t w1[2], w2[2];
    float res[8];
    float amax2 = 0.f;
#pragma unroll
    for (int tt = 0; tt < 2; ++tt) {
      w1[tt] = pack4_fp8(h[4 * tt] * inv1, h[4 * tt + 1] * inv1, h[4 * tt + 2] * inv1, h[4 * tt + 3] * inv1);
#pragma unroll
      for (int ii = 0; ii < 4; ++ii) {
        res[4 * tt + ii] = h[4 * tt + ii] - fp8_byte_to_f32(w1[tt], ii) * sc1;
        amax2 = fmaxf(amax2, fabsf(res[4 * tt + ii]));
      }
    }
    amax2 = shfl_xor_max<16>(amax2);
    amax2 = shfl_xor_max<32>(amax2);
    const int e2 = split_exponent(amax2);
    const float inv2 = ldexpf(1.f, -e2);
#pragma unroll
    for (int tt = 0; tt < 2; ++tt)
      w2[tt] = pack4_fp8(res[4 * tt] * inv2, res[4 * tt + 1] * inv2, res[4 * tt + 2] * inv2, res[4 * tt + 3] * inv2);
    const int i = t * 16 + col;
    if (i < g.cnt) {
      const size_t p = (size_t)g.p0 + i;
      // feature 16tt + 4grp + ii of block blk_h = 4ks + bb: group 2*(bb%2) + tt, byte 16*(bb/2) + 4grp + ii
      const int bb = blk_h & 3;
      uint8_t* dst = a.hq + p * split_q_row_bytes(R) + (size_t)(blk_h >> 2) * 256 + 16 * (bb >> 1) + 4 * grp;
#pragma unroll
      for (int tt = 0; tt < 2; ++tt) {
        uint8_t* gdst = dst + (2 * (bb & 1) + tt) * 64;
        *(uint32_t*)(gdst) = w1[tt];
        *(uint32_t*)(gdst + 32) = w2[tt];
      }
      if (grp == 0) {
        uint8_t* srow = a.hs + p * split_s_row_bytes(R);
        srow[split_scale_offset_h(0, blk_h, n_sg_h)] = (uint8_t)(e1 + 127);
        srow[split_scale_offset_h(1, blk_h, n_sg_h)] = (uint8_t)(e2 + 127);
      }
    }
  }
}

__global__ void __launch_bounds__(256) gateup_kernel(ExpertArgs a) {
  const int n_fb = a.R / kFeatPerWG;
  int unit;
  if (!xcd_unit(*a.n_groups * n_fb, &unit)) return;
  const Group g = a.groups[unit / n_fb];
  const int fb = unit % n_fb;
  gateup_unit<1>(a, g, fb);
}

// ---------------------------------------------------------------------------
// down: y[p][f] = sum_n W_down[e][f][n] h[p][n], fp32 rows in expert-major
// pair order (routed) followed by the shared expert's rows.

template <int NT>
__device__ __forceinline__ void down_unit(const ExpertArgs& a, const Group g, int fb) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int col = lane & 15, grp = lane >> 4;
  const int K = a.K, R = a.R, nks = K / 128, n_sg = (nks + 3) / 4;
  const int f0 = fb * kFeatPerWG + wave * kDownFeatPerWave, rt0 = f0 / 16;
  const bool shared = g.e == a.E;
  const size_t mq = packed_q_bytes(R, K), ms = packed_s_bytes(R, K);
  const uint8_t* dq = shared ? a.sq0 : a.q0 + (size_t)g.e * mq;
  const uint8_t* ds = shared ? a.ss0 : a.s0 + (size_t)g.e * ms;
  const size_t tq = (size_t)nks * 1024, ts = (size_t)n_sg * 256;
  const uint8_t* aq[4];
  const uint8_t* as[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    aq[i] = dq + (rt0 + i) * tq + lane * 16;
    as[i] = ds + (rt0 + i) * ts + lane * 4;
  }
  const uint8_t* bq[NT];
  const uint8_t* bs[NT];
#pragma unroll
  for (int t = 0; t < NT; ++t) {
    const int i = t * 16 + col;
    const size_t p = (size_t)g.p0 + (i < g.cnt ? i : 0);
    bq[t] = a.aq + p * split_q_row_bytes(K) + grp * 64;
    bs[t] = a.as + p * split_s_row_bytes(K) + grp * 4;
  }
  v4f acc[4][NT];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int t = 0; t < NT; ++t) acc[i][t] = v4f{0.f, 0.f, 0.f, 0.f};
  mainloop<4, NT>(aq, as, bq, bs, nks, acc);
#pragma unroll
  for (int t = 0; t < NT; ++t) {
    const int i = t * 16 + col;
    if (i < g.cnt) {
      float* dst = a.y + ((size_t)g.p0 + i) * R + f0 + 4 * grp;
#pragma unroll
      for (int tt = 0; tt < 4; ++tt) *(v4f*)(dst + 16 * tt) = acc[tt][t];
    }
  }
}

__global__ void __launch_bounds__(kDownThreads) down_kernel(ExpertArgs a) {
  const int n_fb = a.R / kFeatPerWG;
  int unit;
  if (!xcd_unit(*a.n_groups * n_fb, &unit)) return;
  const Group g = a.groups[unit / n_fb];
  const int fb = unit % n_fb;
  down_unit<1>(a, g, fb);
}

static unsigned unit_grid(int max_groups, int n_fb) {
  const size_t units = (size_t)max_groups * n_fb;
  return (unsigned)(kXcds * ((units + kXcds - 1) / kXcds));
}

hipError_t launch_gateup(const ExpertArgs& a, int max_groups, hipStream_t stream) {
  hipLaunchKernelGGL(gateup_kernel, dim3(unit_grid(max_groups, a.R / kFeatPerWG)), dim3(256), 0, stream, a);
  return hipGetLastError();
}

hipError_t launch_down(const ExpertArgs& a, int max_groups, hipStream_t stream) {
  hipLaunchKernelGGL(down_kernel, dim3(unit_grid(max_groups, a.R / kFeatPerWG)), dim3(kDownThreads), 0, stream, a);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// out[r] = y_shared[r] + route_scale * sum_j g[r][j] * y[inv[r][j]], fp32 in
// ascending slot order, rounded once to bf16 (nearest even).

__global__ void __launch_bounds__(256) combine_kernel(const float* __restrict__ y, const int32_t* __restrict__ inv,
                                                       const float* __restrict__ gates, int d, int k, int P,
                                                       int has_shared, float route_scale,
                                                       uint16_t* __restrict__ out) {
  constexpr int kMaxK = 8;
  const int r = blockIdx.x;
  const float* src[kMaxK];
  float gw[kMaxK];
#pragma unroll
  for (int j = 0; j < kMaxK; ++j) {
    src[j] = (j < k) ? y + (size_t)inv[(size_t)r * k + j] * d : y;
    gw[j] = (j < k) ? gates[(size_t)r * k + j] : 0.f;
  }
  const float* ysh = has_shared ? y + ((size_t)P + r) * d : nullptr;
  for (int c = threadIdx.x * 4; c < d; c += blockDim.x * 4) {
    v4f acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int j = 0; j < kMaxK; ++j) {
      if (j < k) {
        const v4f v = *(const v4f*)(src[j] + c);
#pragma unroll
        for (int i = 0; i < 4; ++i) acc[i] = fmaf(gw[j], v[i], acc[i]);
      }
    }
    v4f sh = {0.f, 0.f, 0.f, 0.f};
    if (ysh) sh = *(const v4f*)(ysh + c);
    uint2 packed;
    packed.x = (uint32_t)f32_to_bf16_rne(fmaf(route_scale, acc[0], sh[0])) |
               ((uint32_t)f32_to_bf16_rne(fmaf(route_scale, acc[1], sh[1])) << 16);
    packed.y = (uint32_t)f32_to_bf16_rne(fmaf(route_scale, acc[2], sh[2])) |
               ((uint32_t)f32_to_bf16_rne(fmaf(route_scale, acc[3], sh[3])) << 16);
    *(uint2*)(out + (size_t)r * d + c) = packed;
  }
}

hipError_t launch_combine(const float* y, const int32_t* inv, const float* gates, int n_rows, int d, int k, int P,
                          int has_shared, float route_scale, uint16_t* out, hipStream_t stream) {
  hipLaunchKernelGGL(combine_kernel, dim3(n_rows), dim3(256), 0, stream, y, inv, gates, d, k, P, has_shared,
                     route_scale, out);
  return hipGetLastError();
}

}  // namespace moe
