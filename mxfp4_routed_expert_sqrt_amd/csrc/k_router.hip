// Router and routing bookkeeping, in two launches:
//  1. prologue: fp32 router logits (MFMA) and, in the same grid, the two-term
//     FP8 split of x for the expert GEMMs;
//  2. select+route: sqrt-softplus scores with a wave-level top-k per row, and
//     the expert-major bookkeeping (histogram, scan, stable permute, work
//     list), which the last workgroup to finish its rows performs.
#include "kernels.h"
#include "split.h"

namespace moe {

// ---------------------------------------------------------------------------
// z[r][e] = sum_i x[r][i] * W[e][i] + bias[e], fp32 accumulation on
// v_mfma_f32_16x16x4_f32 (bf16 x is exact in fp32).  A workgroup computes one
// 16-row x 16-expert tile; its 4 waves take one quarter of K each and the
// partial tiles are added in wave order through LDS.  Each lane loads 8
// consecutive K values of its row and of its expert per 32-wide k-chunk (lane
// group g supplies k = k0 + 8g + i to MFMA i, for A and B alike), and 4 chunks
// are loaded before any is multiplied.
__device__ __forceinline__ void logits_tile(const uint16_t* __restrict__ x, const float* __restrict__ w,
                                            const float* __restrict__ bias, int n_rows, int d, int E,
                                            float* __restrict__ z, int r0, int e0, float (*part)[16][17]) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int col = lane & 15, grp = lane >> 4;
  const int ra = min(r0 + col, n_rows - 1);  // A operand row of this lane (clamped; result discarded)
  const int eb = min(e0 + col, E - 1);       // B operand expert of this lane
  const int kq = d / 4, kbeg = wave * kq;    // kq is a multiple of 32
  const uint16_t* xp = x + (size_t)ra * d + kbeg + 8 * grp;
  const float* wp = w + (size_t)eb * d + kbeg + 8 * grp;
  v4f acc = {0.f, 0.f, 0.f, 0.f};
  constexpr int kUnroll = 4;
  int kk = 0;
  for (; kk + 32 * kUnroll <= kq; kk += 32 * kUnroll) {
    u32x4 xa[kUnroll];
    float4 wa[kUnroll], wb[kUnroll];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      xa[u] = *(const u32x4*)(xp + kk + 32 * u);
      wa[u] = *(const float4*)(wp + kk + 32 * u);
      wb[u] = *(const float4*)(wp + kk + 32 * u + 4);
    }
    __builtin_amdgcn_sched_barrier(0);  // all 4 chunks in flight before the first multiply
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      const float wv[8] = {wa[u].x, wa[u].y, wa[u].z, wa[u].w, wb[u].x, wb[u].y, wb[u].z, wb[u].w};
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const uint32_t pair = xa[u][i >> 1];
        const float xv = __uint_as_float((i & 1) ? (pair & 0xffff0000u) : (pair << 16));
        acc = __builtin_amdgcn_mfma_f32_16x16x4f32(xv, wv[i], acc, 0, 0, 0);
      }
    }
  }
  for (; kk < kq; kk += 32) {
    const u32x4 xa = *(const u32x4*)(xp + kk);
    const float4 wa = *(const float4*)(wp + kk), wb = *(const float4*)(wp + kk + 4);
    const float wv[8] = {wa.x, wa.y, wa.z, wa.w, wb.x, wb.y, wb.z, wb.w};
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const uint32_t pair = xa[i >> 1];
      const float xv = __uint_as_float((i & 1) ? (pair & 0xffff0000u) : (pair << 16));
      acc = __builtin_amdgcn_mfma_f32_16x16x4f32(xv, wv[i], acc, 0, 0, 0);
    }
  }
  // lane holds D[row 4*grp + i][expert col]
#pragma unroll
  for (int i = 0; i < 4; ++i) part[wave][4 * grp + i][col] = acc[i];
  __syncthreads();
  const int t = threadIdx.x, rr = t >> 4, ee = t & 15;
  const int r = r0 + rr, e = e0 + ee;
  if (r < n_rows && e < E) {
    float v = part[0][rr][ee];
    v += part[1][rr][ee];
    v += part[2][rr][ee];
    v += part[3][rr][ee];
    if (bias) v += bias[e];
    z[(size_t)r * E + e] = v;
  }
}

// Workgroups [0, n_tiles) compute logits tiles; the rest split x (one
// 32-value block per thread).  Workgroup 0 also clears the completion counter
// of the select+route launch that follows on the stream.
__global__ void __launch_bounds__(256) prologue_kernel(const uint16_t* __restrict__ x, const float* __restrict__ w,
                                                        const float* __restrict__ bias, int n_rows, int d, int E,
                                                        float* __restrict__ z, uint8_t* __restrict__ xq,
                                                        uint8_t* __restrict__ xs, int32_t* __restrict__ done) {
  __shared__ float part[4][16][17];
  const int n_rt = (n_rows + 15) / 16, n_tiles = n_rt * ((E + 15) / 16);
  const int b = blockIdx.x;
  if (b == 0 && threadIdx.x == 0) *done = 0;
  if (b < n_tiles) {
    logits_tile(x, w, bias, n_rows, d, E, z, (b % n_rt) * 16, (b / n_rt) * 16, part);
  } else {
    const size_t t = (size_t)(b - n_tiles) * blockDim.x + threadIdx.x;
    if (t < (size_t)n_rows * (d / 32)) split_bf16_block(x, d, xq, xs, t);
  }
}

hipError_t launch_prologue(const uint16_t* x, const float* w, const float* bias, int n_rows, int d, int E, float* z,
                           uint8_t* xq, uint8_t* xs, int32_t* done, hipStream_t stream) {
  const int n_tiles = ((n_rows + 15) / 16) * ((E + 15) / 16);
  const size_t n_split = ((size_t)n_rows * (d / 32) + 255) / 256;
  hipLaunchKernelGGL(prologue_kernel, dim3((unsigned)(n_tiles + n_split)), dim3(256), 0, stream, x, w, bias, n_rows,
                     d, E, z, xq, xs, done);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Scores and selection, one wave per row.  s = sqrt(softplus(z)) with
// softplus(z) = max(z,0) + log1p(exp(-|z|)).  Top-k mode takes the k largest
// scores (equal scores: lower expert id first) by k rounds of a wave argmax;
// hash mode takes tid2eid[token_ids[r]].  Selected ids are written ascending
// with gates = s / sum(s) (summed in ascending id order).

__device__ __forceinline__ float router_score(float zv) {
  return sqrtf(fmaxf(zv, 0.f) + log1pf(expf(-fabsf(zv))));
}

constexpr int kMaxExpertsPerLane = 16;  // E <= 1024
constexpr int kMaxTopK = 8;
constexpr int kNoExpert = 0x7fffffff;

// (value, id) order used by the selection: larger value first, then lower id;
// an empty candidate (id kNoExpert) loses to any real one.
__device__ __forceinline__ bool better(float v, int e, float bv, int be) {
  return e != kNoExpert && (be == kNoExpert || v > bv || (v == bv && e < be));
}

// One DPP step of the (value, id) max-reduction inside each row of 16 lanes.
template <int kCtrl>
__device__ __forceinline__ void dpp_best(float& bv, int& be) {
  const float ov = __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(bv), kCtrl, 0xF, 0xF, false));
  const int oe = __builtin_amdgcn_update_dpp(kNoExpert, be, kCtrl, 0xF, 0xF, false);
  if (better(ov, oe, bv, be)) {
    bv = ov;
    be = oe;
  }
}

// Best (value, id) over the wave, returned uniform in every lane: DPP
// exchanges within rows of 16 lanes (xor 1, xor 2, rotate 4, rotate 8), then
// the four row results are read out and compared in scalar registers.
__device__ __forceinline__ void wave_best(float& bv, int& be) {
  dpp_best<0xB1>(bv, be);   // quad_perm [1,0,3,2]
  dpp_best<0x4E>(bv, be);   // quad_perm [2,3,0,1]
  dpp_best<0x124>(bv, be);  // row_ror:4
  dpp_best<0x128>(bv, be);  // row_ror:8
  float rv = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(bv), 0));
  int re = __builtin_amdgcn_readlane(be, 0);
#pragma unroll
  for (int row = 1; row < 4; ++row) {
    const float ov = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(bv), 16 * row));
    const int oe = __builtin_amdgcn_readlane(be, 16 * row);
    if (better(ov, oe, rv, re)) {
      rv = ov;
      re = oe;
    }
  }
  bv = rv;
  be = re;
}

__device__ __forceinline__ void select_row(const float* __restrict__ z, int r, int E, int k, int routing,
                                           const int32_t* __restrict__ token_ids,
                                           const int32_t* __restrict__ tid2eid, int64_t vocab,
                                           int32_t* __restrict__ idx, float* __restrict__ gates,
                                           int32_t* sel_lds) {
  const int lane = threadIdx.x & 63;
  const float* zr = z + (size_t)r * E;
  const int nc = (E + 63) / 64;  // score slots per lane in use
  int sel[kMaxTopK];
  float sv[kMaxTopK];
  if (routing == 0) {
    float s[kMaxExpertsPerLane];
#pragma unroll
    for (int c = 0; c < kMaxExpertsPerLane; ++c) {
      const int e = c * 64 + lane;
      s[c] = -INFINITY;
      if (c < nc && e < E) s[c] = router_score(zr[e]);
    }
    uint32_t taken = 0;  // bit c: expert c*64 + lane already selected
#pragma unroll
    for (int j = 0; j < kMaxTopK; ++j) {
      if (j < k) {
        // lane-local best among untaken experts; the first candidate is always
        // accepted, so some untaken id wins even if scores are NaN and the
        // selection stays a set of k distinct valid ids
        float bv = -INFINITY;
        int be = kNoExpert;
#pragma unroll
        for (int c = 0; c < kMaxExpertsPerLane; ++c) {
          const int e = c * 64 + lane;
          if (c < nc && e < E && !((taken >> c) & 1u) && better(s[c], e, bv, be)) {
            bv = s[c];
            be = e;
          }
        }
        wave_best(bv, be);
        sel[j] = be;
        sv[j] = bv;
        if ((be & 63) == lane) taken |= 1u << (be >> 6);
      }
    }
  } else {
    // Hash mode.  Table entries must be valid (distinct ids in [0, E)); an
    // invalid token id or expert id is clamped into range so that a bad table
    // gives an unspecified routing but never an out-of-bounds access.
    const int64_t t = min(max((int64_t)token_ids[r], (int64_t)0), vocab - 1);
    const int32_t* row = tid2eid + t * k;
#pragma unroll
    for (int j = 0; j < kMaxTopK; ++j) {
      if (j < k) {
        sel[j] = min(max(row[j], 0), E - 1);
        sv[j] = router_score(zr[sel[j]]);
      }
    }
  }
  // ascending expert id (k <= 8: compare-exchange passes on wave-uniform values)
#pragma unroll
  for (int pass = 0; pass < kMaxTopK; ++pass)
#pragma unroll
    for (int b = 1; b < kMaxTopK; ++b)
      if (b < k && sel[b - 1] > sel[b]) {
        const int te = sel[b];
        sel[b] = sel[b - 1];
        sel[b - 1] = te;
        const float tv = sv[b];
        sv[b] = sv[b - 1];
        sv[b - 1] = tv;
      }
  float sum = 0.f;
#pragma unroll
  for (int j = 0; j < kMaxTopK; ++j)
    if (j < k) sum += sv[j];
#pragma unroll
  for (int j = 0; j < kMaxTopK; ++j)
    if (j < k && lane == j) {
      idx[(size_t)r * k + j] = sel[j];
      gates[(size_t)r * k + j] = sv[j] / sum;
      sel_lds[j] = sel[j];
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
//     that overwrites each row with its exclusive base.  The counts, their
//     exclusive scan (offsets), the scatter of perm/inv and the work list of
//     the grouped GEMMs (groups of <= 16 rows of one expert, then the shared
//     expert's rows) follow.
// Histogram rows are E rounded up to a multiple of 4 ints wide, so both scan
// passes move 16-byte columns.
constexpr int kRouteThreads = 1024;
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

// Work list and offsets[E] once counts and offsets (in LDS) are final.
__device__ __forceinline__ void write_groups(const int32_t* s_cnt, const int32_t* s_off, int n_rows, int P, int E,
                                             int has_shared, Group* __restrict__ groups,
                                             int32_t* __restrict__ n_groups, int32_t* wave_tot) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int c = (tid < E) ? s_cnt[tid] : 0;
  const int ng = (c + kGroupRows - 1) / kGroupRows;
  int incl = ng;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const int o = __shfl_up(incl, off, 64);
    if (lane >= off) incl += o;
  }
  if (lane == 63) wave_tot[wave] = incl;
  __syncthreads();
  int wbase = 0, total = 0;
  for (int w = 0; w < kRouteWaves; ++w) {
    if (w < wave) wbase += wave_tot[w];
    total += wave_tot[w];
  }
  if (tid < E) {
    const int g0 = wbase + incl - ng;
    const int p0 = s_off[tid];
    for (int g = 0; g < ng; ++g) {
      Group gr;
      gr.e = tid;
      gr.p0 = p0 + g * kGroupRows;
      gr.cnt = min(kGroupRows, c - g * kGroupRows);
      gr.pad = 0;
      groups[g0 + g] = gr;
    }
  }
  const int nsh = has_shared ? (n_rows + kGroupRows - 1) / kGroupRows : 0;
  for (int g = tid; g < nsh; g += kRouteThreads) {
    Group gr;
    gr.e = E;
    gr.p0 = P + g * kGroupRows;
    gr.cnt = min(kGroupRows, n_rows - g * kGroupRows);
    gr.pad = 0;
    groups[total + g] = gr;
  }
  if (tid == 0) *n_groups = total + nsh;
}

// Each workgroup selects the experts of 16 rows (one row per wave) and ranks
// their pairs (step 1).  After its stores are released it counts itself done
// on a device-scope counter (cleared by the prologue launch); the workgroup
// that finishes last sees every workgroup's results and runs step 2.
__global__ void __launch_bounds__(kRouteThreads) select_route_kernel(
    const float* __restrict__ z, int n_rows, int E, int k, int routing, const int32_t* __restrict__ token_ids,
    const int32_t* __restrict__ tid2eid, int64_t vocab, int32_t* __restrict__ idx, float* __restrict__ gates,
    int has_shared, int32_t* __restrict__ counts, int32_t* __restrict__ offsets, int32_t* __restrict__ perm,
    int32_t* __restrict__ inv, Group* __restrict__ groups, int32_t* __restrict__ n_groups, int32_t* hist,
    int32_t* done, int scatter_here) {
  __shared__ int32_t s_sel[kRouteWaves * kMaxTopK];
  __shared__ int32_t s_a[kMaxExperts];      // step 1: histogram; step 2: counts
  __shared__ int32_t s_off[kMaxExperts];    // step 2: offsets
  __shared__ int32_t s_seg[4 * kMaxExperts];  // step 2: segment sums / bases, [segment][Ep]
  __shared__ int32_t wave_tot[kRouteWaves];
  __shared__ int32_t is_last;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int b = blockIdx.x, nb = gridDim.x;
  const int Ep = (E + 3) & ~3;
  const int P = n_rows * k;

  // step 1
  for (int e = tid; e < Ep; e += kRouteThreads) s_a[e] = 0;
  const int r = b * kRouteWaves + wave;
  if (r < n_rows) select_row(z, r, E, k, routing, token_ids, tid2eid, vocab, idx, gates, s_sel + wave * k);
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

  // step 2a: per (column of 4 experts, segment of histogram rows) sums
  const int C = Ep / 4;
  const int S = max(1, min(kRouteThreads / C, nb));  // segments
  const int L = (nb + S - 1) / S;                     // rows per segment
  const int4* h4 = (const int4*)hist;
  if (tid < C * S) {
    const int c = tid % C, sg = tid / C;
    const int b0 = min(sg * L, nb), b1 = min(b0 + L, nb);
    int4 acc = {0, 0, 0, 0};
#pragma unroll 8
    for (int bb = b0; bb < b1; ++bb) {
      const int4 v = h4[(size_t)bb * C + c];
      acc.x += v.x;
      acc.y += v.y;
      acc.z += v.z;
      acc.w += v.w;
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
  // 2c: each histogram row becomes its exclusive base
  if (tid < C * S) {
    const int c = tid % C, sg = tid / C;
    const int b0 = min(sg * L, nb), b1 = min(b0 + L, nb);
    int4 run = *(const int4*)(s_seg + sg * Ep + 4 * c);
    int4* w4 = (int4*)hist;
#pragma unroll 8
    for (int bb = b0; bb < b1; ++bb) {
      const int4 v = w4[(size_t)bb * C + c];
      w4[(size_t)bb * C + c] = run;
      run.x += v.x;
      run.y += v.y;
      run.z += v.z;
      run.w += v.w;
    }
  }
  // 2d: offsets = exclusive scan of the counts over experts (E <= 1024: one per thread)
  {
    const int v = (tid < E) ? s_a[tid] : 0;
    int incl = v;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
      const int o = __shfl_up(incl, off, 64);
      if (lane >= off) incl += o;
    }
    if (lane == 63) wave_tot[wave] = incl;
    __syncthreads();
    int wbase = 0;
    for (int w = 0; w < wave; ++w) wbase += wave_tot[w];
    if (tid < E) {
      s_off[tid] = wbase + incl - v;
      offsets[tid] = wbase + incl - v;
    }
    if (tid == 0) offsets[E] = P;
  }
  __syncthreads();
  // 2e: scatter (the bases were written by this workgroup in 2c); for large
  // batches a separate launch spreads it over the whole chip
  const int per_b = kRouteWaves * k;
#pragma unroll 4
  for (int q = tid; q < (scatter_here ? P : 0); q += kRouteThreads) {
    const int e = idx[q];
    const int p = s_off[e] + hist[(size_t)(q / per_b) * Ep + e] + inv[q];
    if ((unsigned)p < (unsigned)P) {  // always true for ranks from step 1; guards the scatter
      perm[p] = q;
      inv[q] = p;
    }
  }
  __syncthreads();  // wave_tot reuse
  write_groups(s_a, s_off, n_rows, P, E, has_shared, groups, n_groups, wave_tot);
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

// Pairs up to which the last selection workgroup scatters by itself (a few per
// thread); above it the scatter is its own launch.
constexpr int kScatterInBlockMax = 8 * kRouteThreads;

hipError_t launch_select_route(const float* z, int n_rows, int E, int k, int routing, const int32_t* token_ids,
                               const int32_t* tid2eid, int64_t vocab, int32_t* idx, float* gates, int has_shared,
                               int32_t* counts, int32_t* offsets, int32_t* perm, int32_t* inv, Group* groups,
                               int32_t* n_groups, int32_t* hist, int32_t* done, hipStream_t stream) {
  if (E > kMaxExperts || k > kMaxTopK) return hipErrorInvalidValue;
  const int P = n_rows * k;
  const int here = P <= kScatterInBlockMax;
  hipLaunchKernelGGL(select_route_kernel, dim3((unsigned)route_workgroups(n_rows)), dim3(kRouteThreads), 0, stream,
                     z, n_rows, E, k, routing, token_ids, tid2eid, vocab, idx, gates, has_shared, counts, offsets,
                     perm, inv, groups, n_groups, hist, done, here);
  if (!here) {
    hipError_t err = hipGetLastError();
    if (err != hipSuccess) return err;
    hipLaunchKernelGGL(scatter_kernel, dim3((unsigned)((P + 255) / 256)), dim3(256), 0, stream, idx, hist, offsets, P,
                       k, E, perm, inv);
  }
  return hipGetLastError();
}

}  // namespace moe
