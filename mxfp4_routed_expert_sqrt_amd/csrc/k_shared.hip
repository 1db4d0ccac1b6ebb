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

// ---------------------------------------------------------------------------
// The same GEMMs for large batches, on weights packed into bf16-MFMA fragments
// (launch_pack_bf16): a workgroup (8 waves) takes 64 token rows and
// 8 * TW * 16 features of each of its NW weight matrices.  Each wave streams
// its NW * TW weight tiles straight from global memory into an 8-deep
// register ring (one contiguous kilobyte per tile and 32-wide k-step), as the
// routed experts' kernels do; only the 64 token rows, which all waves share,
// go through LDS, in chunks of 256 K values (double-buffered, one barrier per
// chunk).  A = weights (16 features), B = tokens (16 rows), so a lane holds 4
// consecutive features of one token and stores them together.  The k-steps are
// accumulated in the same order as the LDS-tiled kernel's.
// Workgroups are numbered feature block first: with 8 feature blocks each XCD
// streams one block of the weights.
constexpr int kSsRows = 64, kSsWaves = 8, kSsSteps = 8;  // token rows; waves; 32-wide k-steps per chunk
constexpr int kSsRowBytes = 32 * kSsSteps * 2 + 16;       // staged token row, padded: 16 mod 128
constexpr int kSsBuf = kSsRows * kSsRowBytes;

template <int NW, int TW>
__global__ void __launch_bounds__(64 * kSsWaves) shared_stream_kernel(const uint16_t* __restrict__ a, int n_rows,
                                                                      int K, const uint8_t* __restrict__ w0,
                                                                      const uint8_t* __restrict__ w1, int n_feat,
                                                                      float limit, uint16_t* __restrict__ h,
                                                                      float* __restrict__ y) {
  typedef __bf16 v8bf __attribute__((ext_vector_type(8)));
  typedef const __attribute__((address_space(1))) uint8_t* gp;
  constexpr int NA = NW * TW, RING = kSsSteps, kFeat = kSsWaves * TW * 16, kPieces = kSsRows * 32 / (64 * kSsWaves);
  extern __shared__ __attribute__((aligned(16))) uint8_t lds[];  // 2 * kSsBuf
  const int n_fb = n_feat / kFeat;
  const int fb = blockIdx.x % n_fb, rt = blockIdx.x / n_fb;
  const int tid = threadIdx.x, lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int col = lane & 15, grp = lane >> 4;
  const int r0 = rt * kSsRows, f0 = fb * kFeat + wave * TW * 16;
  const int nks = K / 32, nch = K / (32 * kSsSteps);
  // weight tile i: matrix i / TW, 16-row tile f0/16 + i % TW (nks kilobytes each)
  gp wq[NA];
#pragma unroll
  for (int i = 0; i < NA; ++i) {
    const uint64_t v = (uint64_t)((i < TW ? w0 : w1) + (size_t)(f0 / 16 + i % TW) * nks * 1024);
    const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)v), hi = __builtin_amdgcn_readfirstlane((uint32_t)(v >> 32));
    wq[i] = (gp)(((uint64_t)hi << 32) | lo);
  }
  auto load_step = [&](u32x4 (&dst)[NA], int ks) {  // clamped: past the end any valid step, never multiplied
    const uint32_t off = (uint32_t)lane * 16 + (uint32_t)min(ks, nks - 1) * 1024;
#pragma unroll
    for (int i = 0; i < NA; ++i) dst[i] = *(const __attribute__((address_space(1))) u32x4*)(wq[i] + off);
  };
  // token chunk c (K values 256c .. 256c+255 of rows r0 .. r0+63, rows past the batch repeat its last row):
  // piece p = tid + 512 j, row p / 32, 16 bytes at (p % 32) * 16
  u32x4 st[kPieces];
  auto stage_load = [&](int c) {
    c = min(c, nch - 1);
#pragma unroll
    for (int j = 0; j < kPieces; ++j) {
      const int pc = tid + 64 * kSsWaves * j, row = min(r0 + (pc >> 5), n_rows - 1);
      st[j] = *(const __attribute__((address_space(1))) u32x4*)((gp)a + ((size_t)row * K + 256 * (size_t)c) * 2 +
                                                                 (pc & 31) * 16);
    }
  };
  auto stage_store = [&](uint8_t* buf) {
#pragma unroll
    for (int j = 0; j < kPieces; ++j) {
      const int pc = tid + 64 * kSsWaves * j;
      *(u32x4*)(buf + (pc >> 5) * kSsRowBytes + (pc & 31) * 16) = st[j];
    }
  };
  v4f acc[NA][4];
#pragma unroll
  for (int i = 0; i < NA; ++i)
#pragma unroll
    for (int cc = 0; cc < 4; ++cc) acc[i][cc] = v4f{0.f, 0.f, 0.f, 0.f};
  u32x4 f[RING][NA];
  stage_load(0);
#pragma unroll
  for (int i = 0; i < RING - 1; ++i) load_step(f[i], i);
  stage_store(lds);
  __syncthreads();
  for (int c = 0; c < nch; ++c) {
    const uint8_t* cur = lds + (c & 1) * kSsBuf;
    stage_load(c + 1);
#pragma unroll
    for (int j = 0; j < kSsSteps; ++j) {
      load_step(f[(j + RING - 1) % RING], kSsSteps * c + j + RING - 1);
      __builtin_amdgcn_sched_barrier(0);
      v8bf b[4];
#pragma unroll
      for (int cc = 0; cc < 4; ++cc)
        b[cc] = *(const v8bf*)(cur + (16 * cc + col) * kSsRowBytes + (32 * j + 8 * grp) * 2);
#pragma unroll
      for (int i = 0; i < NA; ++i) {
        const v8bf av = __builtin_bit_cast(v8bf, f[j][i]);
#pragma unroll
        for (int cc = 0; cc < 4; ++cc) acc[i][cc] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av, b[cc], acc[i][cc], 0, 0, 0);
      }
      __builtin_amdgcn_sched_barrier(0);
    }
    if (c + 1 < nch) stage_store(lds + ((c + 1) & 1) * kSsBuf);
    __syncthreads();
  }
  // lane: features f0 + 16t + 4grp .. +3 of token r0 + 16cc + col
#pragma unroll
  for (int cc = 0; cc < 4; ++cc) {
    const int r = r0 + 16 * cc + col;
    if (r >= n_rows) continue;
#pragma unroll
    for (int t = 0; t < TW; ++t) {
      const int f = f0 + 16 * t + 4 * grp;
      if constexpr (NW == 2) {
        uint32_t hb[4];
#pragma unroll
        for (int ii = 0; ii < 4; ++ii) {
          float gv = acc[t][cc][ii], uv = acc[TW + t][cc][ii];
          if (limit > 0.f) {
            gv = fminf(gv, limit);
            uv = fminf(fmaxf(uv, -limit), limit);
          }
          hb[ii] = f32_to_bf16_rne(gv * __builtin_amdgcn_rcpf(1.f + __expf(-gv)) * uv);
        }
        *(uint2*)(h + (size_t)r * n_feat + f) = uint2{hb[0] | (hb[1] << 16), hb[2] | (hb[3] << 16)};
      } else {
        *(v4f*)(y + (size_t)r * n_feat + f) = acc[t][cc];
      }
    }
  }
}

template <int NW, int TW>
static hipError_t shared_stream_launch(const uint16_t* a, int n_rows, int K, const uint8_t* w0, const uint8_t* w1,
                                       int n_feat, float limit, uint16_t* h, float* y, hipStream_t stream) {
  static std::atomic<uint64_t> attr{0};
  constexpr int kFeat = kSsWaves * TW * 16;
  if (K % (32 * kSsSteps) || n_feat % kFeat) return hipErrorInvalidValue;
  hipError_t err = ensure_dynamic_lds(shared_stream_kernel<NW, TW>, 2 * kSsBuf, attr);
  if (err != hipSuccess) return err;
  const unsigned grid = (unsigned)(((n_rows + kSsRows - 1) / kSsRows) * (n_feat / kFeat));
  hipLaunchKernelGGL((shared_stream_kernel<NW, TW>), dim3(grid), dim3(64 * kSsWaves), 2 * kSsBuf, stream, a, n_rows,
                     K, w0, w1, n_feat, limit, h, y);
  return hipGetLastError();
}

hipError_t launch_shared_stream_gateup(const uint16_t* x, int n_rows, int d, int I, const uint8_t* wg_p,
                                       const uint8_t* wu_p, float limit, uint16_t* h, hipStream_t stream) {
  return shared_stream_launch<2, 2>(x, n_rows, d, wg_p, wu_p, I, limit, h, nullptr, stream);
}

hipError_t launch_shared_stream_down(const uint16_t* h, int n_rows, int d, int I, const uint8_t* wd_p, float* y_sh,
                                     hipStream_t stream) {
  return shared_stream_launch<1, 4>(h, n_rows, I, wd_p, nullptr, d, 0.f, nullptr, y_sh, stream);
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
