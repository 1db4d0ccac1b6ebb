// Router and routing bookkeeping, in two launches:
//  1. prologue: router logits (bf16 MFMA on an exact three-term split of the
//     fp32 weights) and, in the same grid, the two-term FP8 split of x for the
//     expert GEMMs;
//  2. select+route: sqrt-softplus scores with a wave-level top-k per row, and
//     the expert-major bookkeeping (histogram, scan, stable permute, work
//     list), which the last workgroup to finish its rows performs.
#include "kernels.h"
#include "split.h"

namespace moe {

// ---------------------------------------------------------------------------
// Router logits z[r][e] = sum_i x[r][i] * W[e][i] on bf16 MFMA
// (v_mfma_f32_16x16x32_bf16, fp32 accumulation) without loss of precision:
// each fp32 weight is cut into three bf16 terms by truncation,
//   hi = w with the low 16 bits cleared, mid = (w - hi) likewise, lo = w - hi - mid,
// where both differences are exact and lo has at most 8 significant bits, so
// hi + mid + lo = w exactly; bf16 x times a bf16 term is exact in fp32.  The
// three products are accumulated like the fp32 dot product, in a different
// order.
//
// A workgroup computes a 64-row x 64-expert tile over one of S contiguous
// K-ranges (split-K when the row count gives too few tiles).  K advances in
// 64-wide chunks staged through LDS: the workgroup reads the chunk's x rows
// (bf16) and W rows (fp32) with row-contiguous 16-byte loads into registers
// one chunk ahead, and stores them to one of two LDS buffers whose rows are
// padded by 16 bytes so that the 16 rows of an MFMA fragment fall in distinct
// banks.  Wave w takes experts e0+16w..e0+16w+15 as the B operand (it alone
// splits those weights) against four 16-row blocks of x as A operands; lane
// group g supplies k = kk+8g..kk+8g+7 of each 32-wide k-step for A and B
// alike.  The partial sums go to z_part[s][r][e]; the selection adds the S
// partials in s order and the bias.
constexpr int kLgRows = 64, kLgExperts = 64, kLgChunk = 64;
constexpr int kLgXStride = kLgChunk * 2 + 16;  // bytes per x row in LDS
constexpr int kLgWStride = kLgChunk * 4 + 16;  // bytes per W row in LDS
constexpr int kLgBufBytes = kLgRows * kLgXStride + kLgExperts * kLgWStride;

__host__ __device__ inline int logits_row_tiles(int n_rows) { return (n_rows + kLgRows - 1) / kLgRows; }

struct LgRegs {
  u32x4 x[2];  // pieces t and t+256 of the x chunk: row p/8, 16-byte column p%8
  u32x4 w[4];  // pieces t+256i of the W chunk: expert p/16, column p%16
};

__device__ __forceinline__ void lg_fetch(LgRegs& g, const uint16_t* __restrict__ x, const float* __restrict__ w,
                                         int n_rows, int d, int E, int r0, int e0, int k0) {
  const int t = threadIdx.x;
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int p = t + 256 * i, row = min(r0 + (p >> 3), n_rows - 1);
    g.x[i] = *(const u32x4*)(x + (size_t)row * d + k0 + 8 * (p & 7));
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int p = t + 256 * i, ex = min(e0 + (p >> 4), E - 1);
    g.w[i] = *(const u32x4*)(w + (size_t)ex * d + k0 + 4 * (p & 15));
  }
}

__device__ __forceinline__ void lg_stash(const LgRegs& g, uint8_t* buf) {
  const int t = threadIdx.x;
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int p = t + 256 * i;
    *(u32x4*)(buf + (p >> 3) * kLgXStride + 16 * (p & 7)) = g.x[i];
  }
  uint8_t* wb = buf + kLgRows * kLgXStride;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int p = t + 256 * i;
    *(u32x4*)(wb + (p >> 4) * kLgWStride + 16 * (p & 15)) = g.w[i];
  }
}

// One 32-wide k-step (kk within the chunk) of the wave's 64x16 tile from LDS.
__device__ __forceinline__ void lg_step(const uint8_t* buf, int kk, v4f* acc) {
  typedef __bf16 v8bf __attribute__((ext_vector_type(8)));
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int col = lane & 15, grp = lane >> 4;
  const float* wr = (const float*)(buf + kLgRows * kLgXStride + (16 * wave + col) * kLgWStride) + kk + 8 * grp;
  const float4 b0 = *(const float4*)wr, b1 = *(const float4*)(wr + 4);
  const float wv[8] = {b0.x, b0.y, b0.z, b0.w, b1.x, b1.y, b1.z, b1.w};
  uint32_t hi[8], mid[8], lo[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    hi[i] = __float_as_uint(wv[i]) & 0xffff0000u;
    const float r1 = wv[i] - __uint_as_float(hi[i]);
    mid[i] = __float_as_uint(r1) & 0xffff0000u;
    lo[i] = __float_as_uint(r1 - __uint_as_float(mid[i]));
  }
  u32x4 th, tm, tl;
#pragma unroll
  for (int j = 0; j < 4; ++j) {  // upper halves of elements 2j (low) and 2j+1 (high)
    th[j] = __builtin_amdgcn_perm(hi[2 * j + 1], hi[2 * j], 0x07060302u);
    tm[j] = __builtin_amdgcn_perm(mid[2 * j + 1], mid[2 * j], 0x07060302u);
    tl[j] = __builtin_amdgcn_perm(lo[2 * j + 1], lo[2 * j], 0x07060302u);
  }
  const v8bf bh = __builtin_bit_cast(v8bf, th), bm = __builtin_bit_cast(v8bf, tm), bl = __builtin_bit_cast(v8bf, tl);
#pragma unroll
  for (int rb = 0; rb < 4; ++rb) {
    const v8bf av = *(const v8bf*)(buf + (16 * rb + col) * kLgXStride + 2 * (kk + 8 * grp));
    acc[rb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av, bl, acc[rb], 0, 0, 0);
    acc[rb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av, bm, acc[rb], 0, 0, 0);
    acc[rb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av, bh, acc[rb], 0, 0, 0);
  }
}

__device__ __forceinline__ void logits_tile(const uint16_t* __restrict__ x, const float* __restrict__ w, int n_rows,
                                            int d, int E, int S, float* __restrict__ z_part, int tile,
                                            uint8_t* lds) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int col = lane & 15, grp = lane >> 4;
  const int n_rt = logits_row_tiles(n_rows), n_et = (E + kLgExperts - 1) / kLgExperts;
  const int rt = tile % n_rt, et = (tile / n_rt) % n_et, sp = tile / (n_rt * n_et);
  const int r0 = rt * kLgRows, e0 = et * kLgExperts;
  const int nch = d / kLgChunk, c_beg = sp * nch / S, c_end = (sp + 1) * nch / S;
  v4f acc[4];
#pragma unroll
  for (int rb = 0; rb < 4; ++rb) acc[rb] = v4f{0.f, 0.f, 0.f, 0.f};
  LgRegs g;
  lg_fetch(g, x, w, n_rows, d, E, r0, e0, c_beg * kLgChunk);
  lg_stash(g, lds);
  if (c_beg + 1 < c_end) lg_fetch(g, x, w, n_rows, d, E, r0, e0, (c_beg + 1) * kLgChunk);
  __syncthreads();
  for (int c = c_beg; c < c_end; ++c) {
    uint8_t* cur = lds + ((c - c_beg) & 1) * kLgBufBytes;
    uint8_t* nxt = lds + ((c - c_beg + 1) & 1) * kLgBufBytes;
    lg_step(cur, 0, acc);
    lg_step(cur, 32, acc);
    if (c + 1 < c_end) {
      lg_stash(g, nxt);  // chunk c+1, loaded during chunk c
      if (c + 2 < c_end) lg_fetch(g, x, w, n_rows, d, E, r0, e0, (c + 2) * kLgChunk);
    }
    __syncthreads();
  }
  // lane holds D[row 4*grp + i][expert col] of each row block
  const int e = e0 + 16 * wave + col;
  if (e < E) {
    float* zp = z_part + (size_t)sp * logits_partial_stride(n_rows, E) + e;
#pragma unroll
    for (int rb = 0; rb < 4; ++rb)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int r = r0 + 16 * rb + 4 * grp + i;
        if (r < n_rows) zp[(size_t)r * E] = acc[rb][i];
      }
  }
}

// Workgroups [0, n_tiles) compute logits tiles; the rest split x (one
// 32-value block per thread; FP6 for batches of tall work units, else FP8).
// Workgroup 0 also clears the three counters of the launches that follow on
// the stream: the selection's completion count and the unit claim counters of
// gate/up and down.
// The bound of two workgroups per CU (at most 256 registers per lane) keeps
// the MFMA accumulators in VGPRs; with the whole register file the compiler
// placed them in AGPRs and copied them on every chunk.
__global__ void __launch_bounds__(256, 2) prologue_kernel(const uint16_t* __restrict__ x, const float* __restrict__ w,
                                                        int n_rows, int d, int E, int S, int n_tiles,
                                                        float* __restrict__ z_part, uint8_t* __restrict__ xq,
                                                        uint8_t* __restrict__ xs, int32_t* __restrict__ done, int fp6) {
  __shared__ __attribute__((aligned(16))) uint8_t lds[2 * kLgBufBytes];
  const int b = blockIdx.x;
  if (b == 0 && threadIdx.x < kLayerCounters) done[threadIdx.x] = 0;
  if (b < n_tiles) {
    logits_tile(x, w, n_rows, d, E, S, z_part, b, lds);
  } else {
    const size_t t = (size_t)(b - n_tiles) * blockDim.x + threadIdx.x;
    if (t < (size_t)n_rows * (d / 32)) split_bf16_block(x, d, xq, xs, t, fp6 != 0);
  }
}

// Input RMSNorm (the FFN input norm), one 256-thread workgroup per row.  The
// fp32 sum of squares runs in a fixed order: each thread its 8-value chunks
// in order, a butterfly inside each wave, then the four wave sums in order;
// rs = 1/sqrt(ss/d + eps) and xn = bf16((x * rs) * g), rounded to nearest even.
__global__ void __launch_bounds__(256) rmsnorm_kernel(const uint16_t* __restrict__ x, const uint16_t* __restrict__ g,
                                                       int d, float eps, uint16_t* __restrict__ xn) {
  __shared__ float wave_sum[4];
  const int tid = threadIdx.x;
  const size_t row = (size_t)blockIdx.x * d;
  float ss = 0.f;
  for (int c = tid * 8; c < d; c += 256 * 8) {
    const u32x4 v = *(const u32x4*)(x + row + c);
#pragma unroll
    for (int h = 0; h < 4; ++h) {
      const float lo = __uint_as_float(v[h] << 16), hi = __uint_as_float(v[h] & 0xffff0000u);
      ss += lo * lo;
      ss += hi * hi;
    }
  }
#pragma unroll
  for (int m = 1; m < 64; m <<= 1) ss += __shfl_xor(ss, m, 64);
  if ((tid & 63) == 0) wave_sum[tid >> 6] = ss;
  __syncthreads();
  const float total = ((wave_sum[0] + wave_sum[1]) + wave_sum[2]) + wave_sum[3];
  const float rs = 1.0f / sqrtf(total / (float)d + eps);
  for (int c = tid * 8; c < d; c += 256 * 8) {
    const u32x4 v = *(const u32x4*)(x + row + c);
    const u32x4 w = *(const u32x4*)(g + c);
    u32x4 o;
#pragma unroll
    for (int h = 0; h < 4; ++h) {
      const float lo = (__uint_as_float(v[h] << 16) * rs) * __uint_as_float(w[h] << 16);
      const float hi = (__uint_as_float(v[h] & 0xffff0000u) * rs) * __uint_as_float(w[h] & 0xffff0000u);
      o[h] = (uint32_t)f32_to_bf16_rne(lo) | ((uint32_t)f32_to_bf16_rne(hi) << 16);
    }
    *(u32x4*)(xn + row + c) = o;
  }
}

hipError_t launch_rmsnorm(const uint16_t* x, const uint16_t* g, int n_rows, int d, float eps, uint16_t* xn,
                          hipStream_t stream) {
  hipLaunchKernelGGL(rmsnorm_kernel, dim3((unsigned)n_rows), dim3(256), 0, stream, x, g, d, eps, xn);
  return hipGetLastError();
}

hipError_t launch_prologue(const uint16_t* x, const float* w, int n_rows, int d, int E, float* z_part,
                           uint8_t* xq, uint8_t* xs, int32_t* done, bool fp6, hipStream_t stream) {
  const int S = logits_splits(n_rows, E, d);
  const int n_tiles = logits_row_tiles(n_rows) * ((E + kLgExperts - 1) / kLgExperts) * S;
  const size_t n_split = xq ? ((size_t)n_rows * (d / 32) + 255) / 256 : 0;  // no split asked for: logits only
  hipLaunchKernelGGL(prologue_kernel, dim3((unsigned)(n_tiles + n_split)), dim3(256), 0, stream, x, w, n_rows, d, E,
                     S, n_tiles, z_part, xq, xs, done, fp6 ? 1 : 0);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Scores and selection, one wave per row.  s = sqrt(softplus(z)) with
// softplus(z) = max(z,0) + log1p(exp(-|z|)).  Top-k mode takes the k largest
// scores (equal scores: lower expert id first) by k rounds of a wave maximum; hash
// mode takes tid2eid[token_ids[r]].  Selected ids are written ascending with
// gates = s / sum(s).  s increases strictly with z, so the selection runs on
// the logits and only the k selected scores are computed.

__device__ __forceinline__ float router_score(float zv) {
  return sqrtf(fmaxf(zv, 0.f) + log1pf(expf(-fabsf(zv))));
}

constexpr int kMaxExpertsPerLane = 16;  // E <= 1024
constexpr int kMaxTopK = 8;

// Order-preserving code of a logit: larger z, larger code; -0 as +0 (equal
// scores); NaN (a NaN score) above every number.  Never 0.
__device__ __forceinline__ uint32_t logit_code(float z) {
  if (z != z) return 0xFFFFFFFFu;
  uint32_t u = __float_as_uint(z);
  if (u == 0x80000000u) u = 0u;
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// Largest v over the wave (unsigned): an inclusive max scan inside each row
// of 16 lanes by DPP row shifts (1, 2, 4, 8; a lane whose source lies outside
// its row takes 0, the identity), then the four row maxima from lanes 15, 31,
// 47 and 63.
__device__ __forceinline__ uint32_t wave_max_u32(uint32_t v) {
  constexpr int kRowShr = 0x110;  // DPP row_shr:n is kRowShr + n
  v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, kRowShr + 1, 0xf, 0xf, false));
  v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, kRowShr + 2, 0xf, 0xf, false));
  v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, kRowShr + 4, 0xf, 0xf, false));
  v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, kRowShr + 8, 0xf, 0xf, false));
  const uint32_t r0 = (uint32_t)__builtin_amdgcn_readlane((int)v, 15);
  const uint32_t r1 = (uint32_t)__builtin_amdgcn_readlane((int)v, 31);
  const uint32_t r2 = (uint32_t)__builtin_amdgcn_readlane((int)v, 47);
  const uint32_t r3 = (uint32_t)__builtin_amdgcn_readlane((int)v, 63);
  return max(max(r0, r1), max(r2, r3));
}

// NC = score slots per lane the code is unrolled for (expert c*64 + lane in
// slot c); E <= 64*NC.  Instantiated for 1, 2, 4, 8 and 16 slots so that the
// selection runs over no more slots than E needs.
//
// Top-k mode, with every candidate reduced to one 32-bit order-preserving code
// (of the logit, or with a selection-only bias of the biased score; absent
// experts are 0, below every real code):
//  - k rounds, each taking the largest remaining code (a wave max) and, of
//    the candidates that hold it, the lowest id (so equal values favour the
//    lower id); a taken code becomes 0;
//  - the selected lanes write their ids, ascending (slot-major, then lane),
//    to the wave's k LDS slots.
// Hash mode: the ids tid2eid[token_ids[r]], placed by their rank in (id, table
// position) order, so a repeated id keeps table order.
// Lane j < k then holds the j-th smallest selected id, scores it, and the gate
// is score / (sum of the k scores, added in ascending id order).
template <int NC>
__device__ __forceinline__ void select_row(const float* zr /* LDS: the row's logits */, int r, int E, int k,
                                           int routing, const float* __restrict__ sel_bias,
                                           const int32_t* __restrict__ token_ids,
                                           const int32_t* __restrict__ tid2eid, int64_t vocab,
                                           int32_t* __restrict__ idx, float* __restrict__ gates,
                                           int32_t* sel_lds) {
  const int lane = threadIdx.x & 63;
  if (routing == 0) {
    uint32_t code[NC];
#pragma unroll
    for (int c = 0; c < NC; ++c) {
      const int e = c * 64 + lane;
      code[c] = e >= E ? 0u : logit_code(sel_bias ? router_score(zr[e]) + sel_bias[e] : zr[e]);
    }
    uint64_t take[NC];
#pragma unroll
    for (int c = 0; c < NC; ++c) take[c] = 0ull;
    for (int j = 0; j < k; ++j) {
      uint32_t m = code[0];
#pragma unroll
      for (int c = 1; c < NC; ++c) m = max(m, code[c]);
      const uint32_t M = wave_max_u32(m);
      bool found = false;  // wave-uniform
#pragma unroll
      for (int c = 0; c < NC; ++c) {
        const uint64_t b = __ballot(code[c] == M);
        if (!found && b != 0ull) {
          const uint64_t low = b & (~b + 1ull);
          take[c] |= low;
          if ((low >> lane) & 1ull) code[c] = 0u;
          found = true;
        }
      }
    }
    int base = 0;
#pragma unroll
    for (int c = 0; c < NC; ++c) {
      if ((take[c] >> lane) & 1ull) {
        const int below = (int)__builtin_amdgcn_mbcnt_hi((uint32_t)(take[c] >> 32),
                                                         __builtin_amdgcn_mbcnt_lo((uint32_t)take[c], 0u));
        sel_lds[base + below] = c * 64 + lane;
      }
      base += __popcll(take[c]);
    }
  } else {
    // Table entries must be valid (ids in [0, E)); an out-of-range token id
    // or expert id is clamped into range so that a bad table gives an
    // unspecified routing but never an out-of-bounds access.
    const int64_t t = min(max((int64_t)token_ids[r], (int64_t)0), vocab - 1);
    const int32_t* row = tid2eid + t * k;
    int sel[kMaxTopK];
#pragma unroll
    for (int j = 0; j < kMaxTopK; ++j) sel[j] = j < k ? min(max(row[j], 0), E - 1) : 0;
    int my = 0;
#pragma unroll
    for (int j = 0; j < kMaxTopK; ++j) my = (j < k && lane == j) ? sel[j] : my;
    int rank = 0;
#pragma unroll
    for (int i = 0; i < kMaxTopK; ++i)
      if (i < k) rank += (sel[i] < my || (sel[i] == my && i < lane)) ? 1 : 0;
    if (lane < k) sel_lds[rank] = my;
  }
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  // (clamped: the ids index the logits here and the weights later)
  const int my_id = lane < k ? min(max(sel_lds[lane], 0), E - 1) : 0;
  const float my_sv = router_score(lane < k ? zr[my_id] : 0.f);
  float sum = 0.f;
#pragma unroll
  for (int j = 0; j < kMaxTopK; ++j)
    if (j < k) sum += __uint_as_float(__builtin_amdgcn_readlane(__float_as_uint(my_sv), j));
  if (lane < k) {
    idx[(size_t)r * k + lane] = my_id;
    gates[(size_t)r * k + lane] = my_sv / sum;
  }
}

// ---------------------------------------------------------------------------
// Routing bookkeeping.  Pair q = r*k + j (row-major) of row r, selected by
// workgroup b = r/16, goes to position
//   p = offsets[e] + base[b][e] + rank(q),
// rank(q) = number of earlier pairs of expert e inside workgroup b,
// base[b][e] = number of pairs of expert e in workgroups before b.
// Inside an expert the pairs therefore follow the pair index (the row order),
// whatever the timing of the workgroups.
//  1. Every workgroup ranks its own <= 16k pairs (one wave, lanes holding the
//     same expert matched by ballots over the 10 bits of the id) and stores
//     the ranks (in inv) and its per-expert histogram row.
//  2. The last workgroup to finish scans the histogram rows per expert: sums
//     over segments of rows, a scan over the segments, then a second pass
//     that turns each row into its exclusive base (kept in LDS when the bases
//     fit there, else written over the row in global memory).  The counts,
//     their exclusive scan (offsets) and the work list of the grouped GEMMs
//     (groups of <= 16, 32 or 64 rows of one expert, and the shared expert's
//     rows) follow in one pass, then the scatter of perm/inv, whose pairs
//     each thread fetched as soon as the workgroup took over.  A launch of one
//     workgroup (<= 16 rows) takes its own histogram row as the counts, with
//     zero bases.
// Histogram rows are E rounded up to a multiple of 4 ints wide, so both scan
// passes move 16-byte columns.
constexpr int kRouteThreads = 1024;
constexpr int kMaxSplits = 16;  // the most split-K partials of the logits (logits_splits)
// Pairs up to which the last selection workgroup scatters by itself (a few per
// thread); above it the scatter is its own launch.
constexpr int kScatterPerThread = 8;
constexpr int kScatterInBlockMax = kScatterPerThread * kRouteThreads;
// Histogram bases the last workgroup keeps in LDS for its scatter (workgroups
// x experts rounded to 4; 8192 ints: the 512-row verify batch at E = 256).
constexpr int kBaseLds = 8192;
// Histogram rows per scan thread kept in registers between the two passes.
constexpr int kHistRegs = 4;
constexpr int kRouteWaves = kRouteThreads / 64;  // rows selected per workgroup
constexpr int kMaxExperts = 1024;

__device__ __forceinline__ int wave_match_rank(int e, bool act, int lane, bool* last) {
  uint64_t peers = __ballot(act);
#pragma unroll
  for (int bit = 0; bit < 10; ++bit) {
    const uint64_t m = __ballot(act && ((e >> bit) & 1));
    peers &= ((e >> bit) & 1) ? m : ~m;
  }
  const uint64_t lt_mask = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
  *last = (peers >> lane) == 1ull;  // highest lane of its peer set
  return __popcll(peers & lt_mask);
}

// Work list of groups of <= rows rows (ceil(count/rows) per expert in expert
// order, and the shared expert's rows), by the thread of expert tid: c its
// count, ng its groups, p0 its offset, g_excl the groups of the experts before
// it, total the routed groups of all experts.  The expert kernels hand each
// XCD a contiguous range of the list and each XCD runs its range in order.
// With 32-row groups (about one group per routed expert) the shared expert's
// groups, whose units carry the most rows and run longest, go first: last,
// they made the XCD holding them finish its range well after the others.  The
// 16- and 64-row lists keep them last: on 64-row lists shared-first measured
// slower (2048 hash-routed rows: the down launch 24 us longer).
__device__ __forceinline__ void write_groups(int rows, int c, int ng, int p0, int g_excl, int total, int n_rows,
                                             int P, int E, int has_shared, Group* __restrict__ groups,
                                             int32_t* __restrict__ n_groups) {
  const int nsh = has_shared ? (n_rows + rows - 1) / rows : 0;
  const bool shared_first = rows == kMediumGroupRows;
  const int tid = threadIdx.x;
  const int routed0 = shared_first ? nsh : 0, shared0 = shared_first ? 0 : total;
  if (tid < E) {
    const int g0 = routed0 + g_excl;
    for (int g = 0; g < ng; ++g) {
      Group gr;
      gr.e = tid;
      gr.p0 = p0 + g * rows;
      gr.cnt = min(rows, c - g * rows);
      gr.first = g0;
      gr.ng = ng;
      gr.seg_rows = c;
      gr.seg_p0 = p0;
      gr.rows = rows;
      groups[g0 + g] = gr;
    }
  }
  for (int g = tid; g < nsh; g += kRouteThreads) {
    Group gr;
    gr.e = E;
    gr.p0 = P + g * rows;
    gr.cnt = min(rows, n_rows - g * rows);
    gr.first = shared0;
    gr.ng = nsh;
    gr.seg_rows = n_rows;
    gr.seg_p0 = P;
    gr.rows = rows;
    groups[shared0 + g] = gr;
  }
  if (tid == 0) *n_groups = total + nsh;
}

// Each workgroup selects the experts of 16 rows (one row per wave) and ranks
// their pairs (step 1).  After its stores are released it counts itself done
// on a device-scope counter (cleared by the prologue launch); the workgroup
// that finishes last sees every workgroup's results and runs step 2.
__global__ void __launch_bounds__(kRouteThreads) select_route_kernel(
    const float* __restrict__ z, int n_split, const float* __restrict__ bias, int bias_mode, int n_rows, int E, int k, int routing, const int32_t* __restrict__ token_ids,
    const int32_t* __restrict__ tid2eid, int64_t vocab, int32_t* __restrict__ idx, float* __restrict__ gates,
    int has_shared, int32_t* __restrict__ counts, int32_t* __restrict__ offsets, int32_t* __restrict__ perm,
    int32_t* __restrict__ inv, int group_rows, Group* __restrict__ groups, int32_t* __restrict__ n_groups,
    int32_t* hist, int32_t* done, int scatter_here) {
  extern __shared__ float s_z[];  // [16][E] logits of the workgroup's rows
  __shared__ int32_t s_sel[kRouteWaves * kMaxTopK];
  __shared__ int32_t s_a[kMaxExperts];      // step 1: histogram; step 2: counts
  __shared__ int32_t s_off[kMaxExperts];    // step 2: offsets
  __shared__ int32_t s_seg[4 * kMaxExperts];  // step 2: segment sums / bases, [segment][Ep]
  __shared__ int32_t wave_tot[kRouteWaves];
  __shared__ int32_t wave_grp[kRouteWaves];
  __shared__ __attribute__((aligned(16))) int32_t s_base[kBaseLds];  // step 2: bases [workgroup][Ep]
  __shared__ int32_t is_last;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int b = blockIdx.x, nb = gridDim.x;
  const int Ep = (E + 3) & ~3;
  const int P = n_rows * k;
  const float* lbias = bias_mode == 0 ? bias : nullptr;
  const float* sbias = bias_mode == 1 ? bias : nullptr;

  // logits of the workgroup's rows into LDS: the split-K partials (stride
  // n_rows*E) added in split order, then the bias when it is a logit bias
  // (bias_mode 0; a selection-only bias enters the selection keys instead)
  {
    // the block's logits are contiguous in each partial and start on a 16-byte
    // boundary (16*b*E floats; the partial stride is padded to 4 floats)
    const int r0 = b * kRouteWaves, cnt = min(kRouteWaves, n_rows - r0) * E;
    const float* zb = z + (size_t)r0 * E;
    const size_t zstride = logits_partial_stride(n_rows, E);
    for (int i = 4 * tid; i < cnt; i += 4 * kRouteThreads) {
      if (i + 4 <= cnt) {
        // every partial is loaded before the first add (one round trip), then
        // they are added in split order
        float4 u[kMaxSplits];
#pragma unroll
        for (int sp = 0; sp < kMaxSplits; ++sp)
          if (sp < n_split) u[sp] = *(const float4*)(zb + sp * zstride + i);
        float4 v = u[0];
#pragma unroll
        for (int sp = 1; sp < kMaxSplits; ++sp)
          if (sp < n_split) {
            v.x += u[sp].x;
            v.y += u[sp].y;
            v.z += u[sp].z;
            v.w += u[sp].w;
          }
        const float vv[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
        for (int j = 0; j < 4; ++j) s_z[i + j] = lbias ? vv[j] + lbias[(i + j) % E] : vv[j];
      } else {
        for (int j = i; j < cnt; ++j) {
          float v = zb[j];
          for (int sp = 1; sp < n_split; ++sp) v += zb[sp * zstride + j];
          s_z[j] = lbias ? v + lbias[j % E] : v;
        }
      }
    }
  }
  // step 1
  for (int e = tid; e < Ep; e += kRouteThreads) s_a[e] = 0;
  __syncthreads();
  const int r = b * kRouteWaves + wave;
  if (r < n_rows) {
    const float* zr = s_z + wave * E;
    int32_t* sl = s_sel + wave * k;
    if (E <= 64)
      select_row<1>(zr, r, E, k, routing, sbias, token_ids, tid2eid, vocab, idx, gates, sl);
    else if (E <= 128)
      select_row<2>(zr, r, E, k, routing, sbias, token_ids, tid2eid, vocab, idx, gates, sl);
    else if (E <= 256)
      select_row<4>(zr, r, E, k, routing, sbias, token_ids, tid2eid, vocab, idx, gates, sl);
    else if (E <= 512)
      select_row<8>(zr, r, E, k, routing, sbias, token_ids, tid2eid, vocab, idx, gates, sl);
    else
      select_row<kMaxExpertsPerLane>(zr, r, E, k, routing, sbias, token_ids, tid2eid, vocab, idx, gates, sl);
  }
  __syncthreads();
  const int q0 = b * kRouteWaves * k;
  const int nq = min(kRouteWaves, n_rows - b * kRouteWaves) * k;
  if (wave == 0) {
    for (int i0 = 0; i0 < nq; i0 += 64) {
      const int i = i0 + lane;
      const bool act = i < nq;
      const int e = act ? s_sel[i] : -1;
      bool last;
      const int rank = wave_match_rank(e, act, lane, &last);
      const int before = act ? s_a[e] : 0;
      __builtin_amdgcn_wave_barrier();
      if (act) {
        inv[q0 + i] = before + rank;
        if (last) s_a[e] = before + rank + 1;
      }
      __builtin_amdgcn_wave_barrier();
    }
  }
  __syncthreads();
  // One workgroup (at most 16 rows) holds every pair: its own histogram row is
  // the counts and every base is 0, so it goes straight to the offsets with no
  // histogram round trip and no device-scope handshake.
  const bool single = nb == 1;
  const bool base_lds = (size_t)nb * Ep <= (size_t)kBaseLds;
  // the pairs this thread scatters in 2e (expert, rank), loaded as soon as
  // they are visible so that their latency overlaps the scans
  int q_e[kScatterPerThread], q_r[kScatterPerThread];
  auto fetch_pairs = [&]() {
#pragma unroll
    for (int i = 0; i < kScatterPerThread; ++i) {
      const int q = tid + i * kRouteThreads;
      if (scatter_here && q < P) {
        q_e[i] = idx[q];
        q_r[i] = inv[q];
      }
    }
  };
  if (single) {
    for (int e = tid; e < E; e += kRouteThreads) counts[e] = s_a[e];
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");  // idx and the ranks in inv, read back below
    __syncthreads();
    fetch_pairs();
  } else {
    for (int e = tid; e < Ep; e += kRouteThreads) hist[(size_t)b * Ep + e] = s_a[e];

    // Every wave waits until its own stores are acknowledged by the L2; after the
    // barrier, thread 0's device-scope release (part of the acq_rel atomic)
    // writes the L2 back once for the whole workgroup.  One release per
    // workgroup instead of one per wave: each costs an L2 write-back.
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
    if (tid == 0) {
      const int prev = __hip_atomic_fetch_add(done, 1, __ATOMIC_ACQ_REL, __HIP_MEMORY_SCOPE_AGENT);
      is_last = prev == nb - 1;
    }
    __syncthreads();
    if (!is_last) return;
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");  // see the other workgroups' results
    fetch_pairs();

    // step 2a: per (column of 4 experts, segment of histogram rows) sums
    const int C = Ep / 4;
    const int S = max(1, min(kRouteThreads / C, nb));  // segments
    const int L = (nb + S - 1) / S;                     // rows per segment
    const int4* h4 = (const int4*)hist;
    int4 hr[kHistRegs];  // this thread's first histogram rows, reused in 2c
    if (tid < C * S) {
      const int c = tid % C, sg = tid / C;
      const int b0 = min(sg * L, nb), b1 = min(b0 + L, nb);
      int4 acc = {0, 0, 0, 0};
#pragma unroll
      for (int j = 0; j < kHistRegs; ++j)
        if (b0 + j < b1) hr[j] = h4[(size_t)(b0 + j) * C + c];
#pragma unroll 8
      for (int bb = b0 + kHistRegs; bb < b1; ++bb) {
        const int4 v = h4[(size_t)bb * C + c];
        acc.x += v.x;
        acc.y += v.y;
        acc.z += v.z;
        acc.w += v.w;
      }
#pragma unroll
      for (int j = 0; j < kHistRegs; ++j)
        if (b0 + j < b1) {
          acc.x += hr[j].x;
          acc.y += hr[j].y;
          acc.z += hr[j].z;
          acc.w += hr[j].w;
        }
      *(int4*)(s_seg + sg * Ep + 4 * c) = acc;
    }
    __syncthreads();
    // 2b: per expert, exclusive scan over the segments; counts
    for (int e = tid; e < E; e += kRouteThreads) {
      int run = 0;
      for (int sg = 0; sg < S; ++sg) {
        const int v = s_seg[sg * Ep + e];
        s_seg[sg * Ep + e] = run;
        run += v;
      }
      s_a[e] = run;
      counts[e] = run;
    }
    __syncthreads();
    // 2c: each histogram row becomes its exclusive base (in LDS when the
    // bases fit there; in global memory when the scatter reads them there: a
    // separate scatter launch, or too many for LDS)
    if (tid < C * S) {
      const int c = tid % C, sg = tid / C;
      const int b0 = min(sg * L, nb), b1 = min(b0 + L, nb);
      const bool to_hist = !scatter_here || !base_lds;
      int4 run = *(const int4*)(s_seg + sg * Ep + 4 * c);
      int4* w4 = (int4*)hist;
      // (v by value: the caller may pass the very histogram entry this overwrites)
      auto put = [&](int bb, const int4 v) {
        if (base_lds) *(int4*)(s_base + bb * Ep + 4 * c) = run;
        if (to_hist) w4[(size_t)bb * C + c] = run;
        run.x += v.x;
        run.y += v.y;
        run.z += v.z;
        run.w += v.w;
      };
#pragma unroll
      for (int j = 0; j < kHistRegs; ++j)
        if (b0 + j < b1) put(b0 + j, hr[j]);
#pragma unroll 8
      for (int bb = b0 + kHistRegs; bb < b1; ++bb) {
        const int4 v = w4[(size_t)bb * C + c];
        put(bb, v);
      }
    }
  }  // multi-workgroup step 2a-2c
  // 2d: offsets = exclusive scan of the counts over experts, and the work
  // list's group bases = exclusive scan of the groups per expert, in one pass
  // (E <= 1024: one expert per thread); the work list is written here
  {
    const int c = (tid < E) ? s_a[tid] : 0;
    const int ng = (c + group_rows - 1) / group_rows;
    int ic = c, ig = ng;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
      const int oc = __shfl_up(ic, off, 64), og = __shfl_up(ig, off, 64);
      if (lane >= off) {
        ic += oc;
        ig += og;
      }
    }
    if (lane == 63) {
      wave_tot[wave] = ic;
      wave_grp[wave] = ig;
    }
    __syncthreads();
    int wb = 0, gb = 0, g_total = 0;
    for (int w = 0; w < kRouteWaves; ++w) {
      if (w < wave) {
        wb += wave_tot[w];
        gb += wave_grp[w];
      }
      g_total += wave_grp[w];
    }
    const int p0 = wb + ic - c;
    if (tid < E) {
      s_off[tid] = p0;
      offsets[tid] = p0;
    }
    if (tid == 0) offsets[E] = P;
    write_groups(group_rows, c, ng, p0, gb + ig - ng, g_total, n_rows, P, E, has_shared, groups, n_groups);
  }
  __syncthreads();
  // 2e: scatter of the pairs fetched above (the bases were written by this
  // workgroup in 2c); for large batches a separate launch spreads it over the
  // whole chip
  const int per_b = kRouteWaves * k;
#pragma unroll
  for (int i = 0; i < kScatterPerThread; ++i) {
    const int q = tid + i * kRouteThreads;
    if (scatter_here && q < P) {
      const int e = min(max(q_e[i], 0), E - 1);
      const int bq = q / per_b;
      const int base = single ? 0 : (base_lds ? s_base[bq * Ep + e] : hist[(size_t)bq * Ep + e]);
      const int p = s_off[e] + base + q_r[i];
      if ((unsigned)p < (unsigned)P) {  // always true for ranks from step 1; guards the scatter
        perm[p] = q;
        inv[q] = p;
      }
    }
  }
}

// Scatter of perm/inv, one pair per thread (bases and offsets come from the
// last selection workgroup of the preceding launch).
__global__ void __launch_bounds__(256) scatter_kernel(const int32_t* __restrict__ idx, const int32_t* __restrict__ hist,
                                                      const int32_t* __restrict__ offsets, int P, int k, int E,
                                                      int32_t* __restrict__ perm, int32_t* __restrict__ inv) {
  const int q = blockIdx.x * 256 + threadIdx.x;
  if (q >= P) return;
  const int Ep = (E + 3) & ~3;
  const int e = idx[q];
  const int p = offsets[e] + hist[(size_t)(q / (kRouteWaves * k)) * Ep + e] + inv[q];
  if ((unsigned)p < (unsigned)P) {
    perm[p] = q;
    inv[q] = p;
  }
}


hipError_t launch_select_route(const float* z, const float* bias, int bias_mode, int d, int n_rows, int E, int k, int routing, const int32_t* token_ids,
                               const int32_t* tid2eid, int64_t vocab, int32_t* idx, float* gates, int has_shared,
                               int32_t* counts, int32_t* offsets, int32_t* perm, int32_t* inv, int group_rows,
                               Group* groups, int32_t* n_groups, int32_t* hist, int32_t* done, hipStream_t stream) {
  if (E > kMaxExperts || k > kMaxTopK || logits_splits(n_rows, E, d) > kMaxSplits) return hipErrorInvalidValue;
  static std::atomic<uint64_t> attr{0};  // dynamic LDS up to 64 KB (E = 1024) plus the static part
  {
    hipError_t err = ensure_dynamic_lds(select_route_kernel, sizeof(float) * kRouteWaves * kMaxExperts, attr);
    if (err != hipSuccess) return err;
  }
  const int P = n_rows * k;
  const int here = P <= kScatterInBlockMax;
  const size_t lds = sizeof(float) * kRouteWaves * E;
  hipLaunchKernelGGL(select_route_kernel, dim3((unsigned)route_workgroups(n_rows)), dim3(kRouteThreads), lds, stream,
                     z, logits_splits(n_rows, E, d), bias, bias_mode, n_rows, E, k, routing, token_ids, tid2eid, vocab, idx, gates, has_shared, counts, offsets,
                     perm, inv, group_rows, groups, n_groups, hist, done, here);
  if (!here) {
    hipError_t err = hipGetLastError();
    if (err != hipSuccess) return err;
    hipLaunchKernelGGL(scatter_kernel, dim3((unsigned)((P + 255) / 256)), dim3(256), 0, stream, idx, hist, offsets, P,
                       k, E, perm, inv);
  }
  return hipGetLastError();
}

}  // namespace moe
