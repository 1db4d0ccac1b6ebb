// The shared expert with bf16 weights (MOE_SHARED_BF16): two dense GEMMs over
// all N token rows on bf16 MFMA (v_mfma_f32_16x16x32_bf16, fp32 accumulation):
//   gate/up: h[r][n] = silu(min(g, L)) * clamp(u, -L, L),  g = Wg[n] . x[r],
//            u = Wu[n] . x[r], rounded once to bf16 (h [N][I]);
//   down:    y[P + r][m] = Wd[m] . h[r] in fp32: the shared rows of y that the
//            combine adds to the routed sum.
// bf16 times bf16 is exact in fp32, so the only roundings are the fp32 sums
// and the one of h.
//
// A workgroup (4 waves) computes a 64-row x 64-feature tile over the whole
// contraction, staged in 64-wide K chunks through two LDS buffers: the token
// rows (x or h) and the NW weight matrices' 64 rows (gate and up, or down),
// each row padded by 16 bytes so that the 16 rows of an MFMA fragment fall in
// distinct banks.  Row-contiguous 16-byte loads fetch chunk c+1 into
// registers while chunk c is multiplied.  Wave w takes features 16w..16w+15
// of each weight matrix as the B operand against four 16-row blocks of tokens
// as A operands; lane group g supplies k = kk+8g..kk+8g+7 of each 32-wide
// k-step for A and B alike, and the lane then holds D[token 4g+i][feature
// col] of each row block.
//
// Tiles are numbered feature-tile first, so the workgroups of one XCD
// (blockIdx % 8) share one eighth of the weight tiles and read every token
// tile: each XCD's L2 holds a slice of the weights instead of all of them.
#include "kernels.h"

namespace moe {

constexpr int kSbRows = 64, kSbFeat = 64, kSbChunk = 64;
constexpr int kSbStride = kSbChunk * 2 + 16;  // bytes per staged row

template <int NW>
struct SbStage {
  static constexpr int kPieces = (kSbRows + NW * kSbFeat) * (kSbChunk / 8);  // 16-byte pieces per chunk
  static constexpr int kPerThread = kPieces / 256;
  static constexpr int kBufBytes = (kSbRows + NW * kSbFeat) * kSbStride;
  u32x4 v[kPerThread];
};

// Piece p of a chunk: rows 0..63 are token rows, then 64 rows per weight
// matrix; 8 pieces of 8 bf16 per row.
template <int NW>
__device__ __forceinline__ void sb_fetch(SbStage<NW>& st, const uint16_t* __restrict__ a, int n_rows, int r0,
                                         const uint16_t* __restrict__ w0, const uint16_t* __restrict__ w1, int f0,
                                         int K, int k0) {
#pragma unroll
  for (int i = 0; i < SbStage<NW>::kPerThread; ++i) {
    const int p = threadIdx.x + 256 * i, row = p >> 3, col = 8 * (p & 7);
    const uint16_t* src;
    if (row < kSbRows) {
      src = a + (size_t)min(r0 + row, n_rows - 1) * K;
    } else {
      const int wr = row - kSbRows;
      src = (NW == 2 && wr >= kSbFeat ? w1 : w0) + (size_t)(f0 + (wr & (kSbFeat - 1))) * K;
    }
    st.v[i] = *(const u32x4*)(src + k0 + col);
  }
}

template <int NW>
__device__ __forceinline__ void sb_stash(const SbStage<NW>& st, uint8_t* buf) {
#pragma unroll
  for (int i = 0; i < SbStage<NW>::kPerThread; ++i) {
    const int p = threadIdx.x + 256 * i;
    *(u32x4*)(buf + (p >> 3) * kSbStride + 16 * (p & 7)) = st.v[i];
  }
}

template <int NW>
__device__ __forceinline__ void sb_step(const uint8_t* buf, int kk, v4f (*acc)[4]) {
  typedef __bf16 v8bf __attribute__((ext_vector_type(8)));
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int col = lane & 15, grp = lane >> 4;
  v8bf b[NW];
#pragma unroll
  for (int j = 0; j < NW; ++j)
    b[j] = *(const v8bf*)(buf + (kSbRows + j * kSbFeat + 16 * wave + col) * kSbStride + 2 * (kk + 8 * grp));
#pragma unroll
  for (int rb = 0; rb < 4; ++rb) {
    const v8bf av = *(const v8bf*)(buf + (16 * rb + col) * kSbStride + 2 * (kk + 8 * grp));
#pragma unroll
    for (int j = 0; j < NW; ++j) acc[j][rb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av, b[j], acc[j][rb], 0, 0, 0);
  }
}

// NW = 2: gate/up tile, writes bf16 h [N][n_feat]; NW = 1: down tile, writes
// fp32 y rows y_row0 + r of width n_feat.
// The bound of two workgroups per CU (at most 256 registers per lane) keeps
// the MFMA accumulators in VGPRs; with the whole register file the compiler
// placed them in AGPRs and copied them on every chunk.
template <int NW>
__global__ void __launch_bounds__(256, 2) shared_bf16_kernel(const uint16_t* __restrict__ a, int n_rows, int K,
                                                          const uint16_t* __restrict__ w0,
                                                          const uint16_t* __restrict__ w1, int n_feat, float limit,
                                                          uint16_t* __restrict__ h, float* __restrict__ y) {
  __shared__ __attribute__((aligned(16))) uint8_t lds[2 * SbStage<NW>::kBufBytes];
  const int n_ft = n_feat / kSbFeat;
  const int ft = blockIdx.x % n_ft, rt = blockIdx.x / n_ft;
  const int r0 = rt * kSbRows, f0 = ft * kSbFeat;
  const int nch = K / kSbChunk;
  v4f acc[NW][4];
#pragma unroll
  for (int j = 0; j < NW; ++j)
#pragma unroll
    for (int rb = 0; rb < 4; ++rb) acc[j][rb] = v4f{0.f, 0.f, 0.f, 0.f};
  SbStage<NW> st;
  sb_fetch<NW>(st, a, n_rows, r0, w0, w1, f0, K, 0);
  sb_stash<NW>(st, lds);
  if (nch > 1) sb_fetch<NW>(st, a, n_rows, r0, w0, w1, f0, K, kSbChunk);
  __syncthreads();
  for (int c = 0; c < nch; ++c) {
    uint8_t* cur = lds + (c & 1) * SbStage<NW>::kBufBytes;
    uint8_t* nxt = lds + ((c + 1) & 1) * SbStage<NW>::kBufBytes;
    sb_step<NW>(cur, 0, acc);
    sb_step<NW>(cur, 32, acc);
    if (c + 1 < nch) {
      sb_stash<NW>(st, nxt);  // chunk c+1, loaded during chunk c
      if (c + 2 < nch) sb_fetch<NW>(st, a, n_rows, r0, w0, w1, f0, K, (c + 2) * kSbChunk);
    }
    __syncthreads();
  }
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int col = lane & 15, grp = lane >> 4;
  const int f = f0 + 16 * wave + col;
#pragma unroll
  for (int rb = 0; rb < 4; ++rb)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int r = r0 + 16 * rb + 4 * grp + i;
      if (r >= n_rows) continue;
      if constexpr (NW == 2) {
        float gv = acc[0][rb][i], uv = acc[1][rb][i];
        if (limit > 0.f) {
          gv = fminf(gv, limit);
          uv = fminf(fmaxf(uv, -limit), limit);
        }
        h[(size_t)r * n_feat + f] = f32_to_bf16_rne(gv * __builtin_amdgcn_rcpf(1.f + __expf(-gv)) * uv);
      } else {
        y[(size_t)r * n_feat + f] = acc[0][rb][i];
      }
    }
}

hipError_t launch_shared_bf16_gateup(const uint16_t* x, int n_rows, int d, int I, const uint16_t* wg,
                                     const uint16_t* wu, float limit, uint16_t* h, hipStream_t stream) {
  if (d % kSbChunk || I % kSbFeat) return hipErrorInvalidValue;
  const unsigned grid = (unsigned)(((n_rows + kSbRows - 1) / kSbRows) * (I / kSbFeat));
  hipLaunchKernelGGL(shared_bf16_kernel<2>, dim3(grid), dim3(256), 0, stream, x, n_rows, d, wg, wu, I, limit, h,
                     nullptr);
  return hipGetLastError();
}

hipError_t launch_shared_bf16_down(const uint16_t* h, int n_rows, int d, int I, const uint16_t* wd, float* y_sh,
                                   hipStream_t stream) {
  if (I % kSbChunk || d % kSbFeat) return hipErrorInvalidValue;
  const unsigned grid = (unsigned)(((n_rows + kSbRows - 1) / kSbRows) * (d / kSbFeat));
  hipLaunchKernelGGL(shared_bf16_kernel<1>, dim3(grid), dim3(256), 0, stream, h, n_rows, I, wd, nullptr, d, 0.f,
                     nullptr, y_sh);
  return hipGetLastError();
}

}  // namespace moe
