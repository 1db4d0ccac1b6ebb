// Router: fp32 logits (MFMA), sqrt-softplus scores with wave-level top-k, and
// the expert-major routing bookkeeping (histogram, scan, stable permute).
#include "kernels.h"

namespace moe {

// ---------------------------------------------------------------------------
// z[r][e] = sum_i x[r][i] * W[e][i] + bias[e], fp32 accumulation on
// v_mfma_f32_16x16x4_f32 (bf16 x is exact in fp32).  A workgroup computes one
// 16-row x 16-expert tile; its 4 waves take one quarter of K each and the
// partial tiles are added in wave order through LDS.  Each lane loads 8
// consecutive K values of its row and of its expert per 32-wide k-chunk (lane
// group g supplies k = k0 + 8g + i to MFMA i, for A and B alike), and 4 chunks
// are loaded before any is multiplied.
__global__ void __launch_bounds__(256) router_logits_kernel(const uint16_t* __restrict__ x,
                                                             const float* __restrict__ w,
                                                             const float* __restrict__ bias, int n_rows, int d,
                                                             int E, float* __restrict__ z) {
  __shared__ float part[4][16][17];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int col = lane & 15, grp = lane >> 4;
  const int r0 = blockIdx.x * 16, e0 = blockIdx.y * 16;
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

hipError_t launch_router_logits(const uint16_t* x, const float* w, const float* bias, int n_rows, int d, int E,
                                float* z, hipStream_t stream) {
  dim3 grid((n_rows + 15) / 16, (E + 15) / 16);
  hipLaunchKernelGGL(router_logits_kernel, grid, dim3(256), 0, stream, x, w, bias, n_rows, d, E, z);
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

__global__ void __launch_bounds__(256) select_kernel(const float* __restrict__ z, int n_rows, int E, int k,
                                                      int routing, const int32_t* __restrict__ token_ids,
                                                      const int32_t* __restrict__ tid2eid, int64_t vocab,
                                                      int32_t* __restrict__ idx, float* __restrict__ gates) {
  const int lane = threadIdx.x & 63;
  const int r = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (r >= n_rows) return;
  const float* zr = z + (size_t)r * E;
  int sel[kMaxTopK];
  float sv[kMaxTopK];
  if (routing == 0) {
    float s[kMaxExpertsPerLane];
#pragma unroll
    for (int c = 0; c < kMaxExpertsPerLane; ++c) {
      const int e = c * 64 + lane;
      s[c] = (e < E) ? router_score(zr[e]) : -INFINITY;
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
          if (e < E && !((taken >> c) & 1u) && better(s[c], e, bv, be)) {
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
    }
}

hipError_t launch_select(const float* z, int n_rows, int E, int k, int routing, const int32_t* token_ids,
                         const int32_t* tid2eid, int64_t vocab, int32_t* idx, float* gates, hipStream_t stream) {
  hipLaunchKernelGGL(select_kernel, dim3((n_rows + 3) / 4), dim3(256), 0, stream, z, n_rows, E, k, routing,
                     token_ids, tid2eid, vocab, idx, gates);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Routing bookkeeping in one workgroup of 16 waves.  The N*k pairs (row-major,
// pair q = r*k + j) are cut into 16 contiguous ranges, one per wave.
//  1. Each wave walks its range 64 pairs at a time; a pair's rank among the
//     earlier pairs of the same expert inside the wave is the wave's running
//     count for that expert plus the number of lower lanes holding the same
//     expert in this batch.  Running counts live in an LDS row per wave.
//  2. Counts, the exclusive scan over experts, and each wave's base position
//     per expert (pairs of lower waves come first) follow by plain scans.
//  3. Position p = base[wave][e] + rank gives perm[p] = q and inv[q] = p.
// The order inside an expert is therefore by pair index, i.e. by row.  The
// work list of the grouped GEMMs (groups of <= 32 rows of one expert, then
// the shared expert's rows) is written at the end.
constexpr int kRouteThreads = 1024;
constexpr int kRouteWaves = kRouteThreads / 64;

__global__ void __launch_bounds__(kRouteThreads) route_kernel(const int32_t* __restrict__ idx, int n_rows, int k,
                                                               int E, int has_shared, int32_t* __restrict__ counts,
                                                               int32_t* __restrict__ offsets,
                                                               int32_t* __restrict__ perm, int32_t* __restrict__ inv,
                                                               Group* __restrict__ groups,
                                                               int32_t* __restrict__ n_groups) {
  extern __shared__ int32_t lds[];
  int32_t* hist = lds;                     // [kRouteWaves][E]
  int32_t* scan = lds + kRouteWaves * E;   // [E + 1]: offsets, then group bases
  __shared__ int32_t wave_tot[kRouteWaves];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int P = n_rows * k;
  for (int i = tid; i < kRouteWaves * E; i += kRouteThreads) hist[i] = 0;
  __syncthreads();

  const int chunk = (P + kRouteWaves - 1) / kRouteWaves;
  const int q_beg = min(wave * chunk, P), q_end = min(q_beg + chunk, P);
  int32_t* my_hist = hist + wave * E;
  const uint64_t lt_mask = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
  for (int base = q_beg; base < q_end; base += 64) {
    const int q = base + lane;
    const bool act = q < q_end;
    const int e = act ? idx[q] : -1;
    // lanes holding the same expert (match over the 10 bits of e < 1024)
    uint64_t peers = __ballot(act);
#pragma unroll
    for (int b = 0; b < 10; ++b) {
      const uint64_t m = __ballot(act && ((e >> b) & 1));
      peers &= ((e >> b) & 1) ? m : ~m;
    }
    int before = 0;
    if (act) before = my_hist[e];
    __builtin_amdgcn_wave_barrier();
    const int rank = __popcll(peers & lt_mask);
    if (act) {
      inv[q] = before + rank;  // local rank, completed in step 3
      const bool last = (peers >> lane) == 1ull;  // highest lane of its peer set
      if (last) my_hist[e] = before + rank + 1;
    }
    __builtin_amdgcn_wave_barrier();
  }
  __syncthreads();

  // step 2: per expert, exclusive over waves; then exclusive scan over experts
  for (int e = tid; e < E; e += kRouteThreads) {
    int run = 0;
    for (int w = 0; w < kRouteWaves; ++w) {
      const int c = hist[w * E + e];
      hist[w * E + e] = run;
      run += c;
    }
    scan[e] = run;
    counts[e] = run;
  }
  __syncthreads();
  // block-wide exclusive scan of scan[0..E) (E <= 1024: one element per thread)
  {
    const int v = (tid < E) ? scan[tid] : 0;
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
    __syncthreads();
    if (tid < E) {
      scan[tid] = wbase + incl - v;
      offsets[tid] = wbase + incl - v;
    }
    if (tid == 0) offsets[E] = P;
  }
  __syncthreads();

  // step 3
  for (int base = q_beg; base < q_end; base += 64) {
    const int q = base + lane;
    if (q < q_end) {
      const int e = idx[q];
      const int p = scan[e] + hist[wave * E + e] + inv[q];
      perm[p] = q;
      inv[q] = p;
    }
  }
  __syncthreads();

  // work list: ceil(count/32) groups per expert, then the shared expert's rows
  {
    const int c = (tid < E) ? counts[tid] : 0;
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
      const int p0 = scan[tid];
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
}

hipError_t launch_route(const int32_t* idx, int n_rows, int k, int E, int has_shared, int32_t* counts,
                        int32_t* offsets, int32_t* perm, int32_t* inv, Group* groups, int32_t* n_groups,
                        hipStream_t stream) {
  const size_t lds = sizeof(int32_t) * ((size_t)kRouteWaves * E + E + 1);
  static bool attr_set = false;  // one-time raise of the dynamic LDS limit (up to 69.6 KB at E = 1024)
  if (!attr_set) {
    hipError_t err = hipFuncSetAttribute((const void*)route_kernel, hipFuncAttributeMaxDynamicSharedMemorySize,
                                         (int)(sizeof(int32_t) * ((size_t)kRouteWaves * 1024 + 1025)));
    if (err != hipSuccess) return err;
    attr_set = true;
  }
  hipLaunchKernelGGL(route_kernel, dim3(1), dim3(kRouteThreads), lds, stream, idx, n_rows, k, E, has_shared, counts,
                     offsets, perm, inv, groups, n_groups);
  return hipGetLastError();
}

}  // namespace moe
