// Launch wrappers of the gfx950 kernels (host side).  All launches are
// asynchronous on `stream`; shapes are validated by the caller.
#pragma once
#include <atomic>
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "common.h"

namespace moe {

// Sets a kernel's dynamic LDS limit to `bytes` once per device (the limit is
// a per-device function attribute; `done` holds one bit per device id < 64,
// higher ids set it on every call).  Concurrent first calls both set it, which
// is harmless.
template <typename Kern>
inline hipError_t ensure_dynamic_lds(Kern* kernel, size_t bytes, std::atomic<uint64_t>& done) {
  int dev = 0;
  hipError_t err = hipGetDevice(&dev);
  if (err != hipSuccess) return err;
  const uint64_t bit = dev < 64 ? (1ull << dev) : 0;
  if (bit && (done.load(std::memory_order_relaxed) & bit)) return hipSuccess;
  err = hipFuncSetAttribute((const void*)kernel, hipFuncAttributeMaxDynamicSharedMemorySize, (int)bytes);
  if (err == hipSuccess) done.fetch_or(bit, std::memory_order_relaxed);
  return err;
}

// Packed-layout sizes of one MXFP4 matrix [rows][K] (rows % 16 == 0, K % 128 == 0).
__host__ __device__ inline size_t packed_q_bytes(int rows, int K) { return (size_t)rows * (size_t)(K / 2); }
__host__ __device__ inline size_t packed_s_bytes(int rows, int K) {
  const int nks = K / 128, n_sg = (nks + 3) / 4;
  return (size_t)(rows / 16) * (size_t)n_sg * 256;
}
// Two-term FP8 split of activation rows of length K.
__host__ __device__ inline size_t split_q_row_bytes(int K) { return (size_t)K * 2; }
// Byte of the scale of 32-block blk, term `term`, in an activation split's
// scale row ([term][n_sg][4][4]: lane group g of a k-step reads the scales of
// its block for 4 consecutive k-steps as one dword).
__host__ __device__ inline size_t split_scale_offset(int term, int blk, int n_sg) {
  const int ks = blk >> 2;
  return (size_t)(((term * n_sg + (ks >> 2)) * 4 + (blk & 3)) * 4 + (ks & 3));
}

// FP6 split rows (tall units) use 192 bytes per 128-wide k-step of the same row, 96 per term.
constexpr int kFp6StepBytes = 192, kFp6TermBytes = 96;
__host__ __device__ inline size_t split_s_row_bytes(int K) {
  const int nks = K / 128, n_sg = (nks + 3) / 4;
  return (size_t)2 * n_sg * 16;
}

hipError_t launch_pack_mxfp4(const uint8_t* q, const uint8_t* s, int n_mat, int rows, int K, uint8_t* q_out,
                             uint8_t* s_out, hipStream_t stream);

// Counters of one layer call, zeroed by the prologue launch: the selection's
// completion count, the claim pools of gate/up and down, and the per-XCD
// claim counters of the tall gate/up and down kernels.
constexpr int kLayerCounters = 3 + 2 * kXcds;

// Router logits partials and (xq != NULL) the two-term split of x; clears the
// kLayerCounters counters at done.
hipError_t launch_prologue(const uint16_t* x, const float* w, int n_rows, int d, int E, float* z_part, uint8_t* xq,
                           uint8_t* xs, int32_t* done, bool fp6, hipStream_t stream);

// xn[r] = bf16((x[r][i] * rs[r]) * g[i]), rs[r] = 1/sqrt(mean_i x[r][i]^2 + eps), fp32 (d % 128 == 0).
hipError_t launch_rmsnorm(const uint16_t* x, const uint16_t* g, int n_rows, int d, float eps, uint16_t* xn,
                          hipStream_t stream);

// Rows of one work group (and work unit) of the expert GEMMs for a batch of
// n_pairs routed pairs:
//  - 64 (tall units, activations split into two FP6 terms) once the batch has
//    at least 32 routed rows per expert on average (prefill-like);
//  - 32 (medium units, FP8 terms) from kWideUnitPairs pairs on: nearly every
//    expert then fits one group, so its weights are read once;
//  - 16 otherwise (small batches, or widths the wider units do not divide).
// The wider units need gate/up I % 256 and down d % 512.
constexpr int kWideUnitPairs = 1024;

inline int unit_rows(int n_pairs, int E, int d, int I) {
  if (I % 256 != 0 || d % 512 != 0) return kGroupRows;
  if (n_pairs >= 32 * E) return kTallGroupRows;
  if (n_pairs >= kWideUnitPairs) return kMediumGroupRows;
  return kGroupRows;
}

// Split-K factor of the router logits: enough 64x64 tiles for >= 256
// workgroups (>= 768, three per CU, from 64 tiles on: a tile's K loop runs at
// the latency of its chunk steps, so large batches gain from more tiles in
// flight per CU), at most 16 partials and at least two 64-wide K chunks each.
__host__ __device__ inline int logits_splits(int n_rows, int E, int d) {
  const int tiles = ((n_rows + 63) / 64) * ((E + 63) / 64);
  const int target = tiles >= 64 ? 768 : 256;
  int S = (target + tiles - 1) / tiles;
  S = S < 16 ? S : 16;
  S = S < d / 128 ? S : d / 128;
  return S > 1 ? S : 1;
}
// Floats between consecutive logits partials (n_rows*E rounded up to 4).
__host__ __device__ inline size_t logits_partial_stride(int n_rows, int E) {
  return ((size_t)n_rows * E + 3) & ~(size_t)3;
}

// bias_mode 0: bias added to the logits; 1: added to the scores for the selection only
hipError_t launch_select_route(const float* z, const float* bias, int bias_mode, int d, int n_rows, int E, int k, int routing, const int32_t* token_ids,
                               const int32_t* tid2eid, int64_t vocab, int32_t* idx, float* gates, int has_shared,
                               int32_t* counts, int32_t* offsets, int32_t* perm, int32_t* inv, int group_rows,
                               Group* groups, int32_t* n_groups, int32_t* hist, int32_t* done, hipStream_t stream);

// Selection workgroups (16 rows each) and the size of their per-expert
// histogram rows (E rounded up to 4 int32).
inline int route_workgroups(int n_rows) { return (n_rows + 15) / 16; }
inline size_t route_hist_bytes(int n_rows, int E) {
  return (size_t)route_workgroups(n_rows) * (size_t)((E + 3) & ~3) * 4;
}

struct ExpertArgs {
  // weights of the routed experts (E matrices) and of the shared expert
  const uint8_t *q0, *s0, *q1, *s1;      // gate/up: q0/s0 gate, q1/s1 up; down: q0/s0
  const uint8_t *sq0, *ss0, *sq1, *ss1;  // shared expert, same roles
  const uint8_t* aq;                     // activation split bytes (x for gate/up, h for down)
  const uint8_t* as;                     // activation split scales
  const int32_t* perm;                   // expert-major pair -> r*k + j
  const Group* groups;                   // work list of <= rows-row groups
  const int32_t* n_groups;
  int K, R;                              // contraction length, rows of each weight matrix
  int E, k, P;                           // experts, top-k, routed pairs (N*k)
  float limit;                           // swiglu limit (<= 0: none)
  uint8_t* hq;                           // gate/up output: split h bytes
  uint8_t* hs;                           // gate/up output: split h scales
  float* y;                              // down output [pairs][R]
  int tail_units;                        // units per XCD processed as two halves at the end
  int32_t* pool;                         // claim counter of xcd_unit_claim (medium and tall units)
  int32_t* xcd_ctr;                      // tall units: per-XCD claim counters [kXcds]
  int rows;                              // rows of the work list's groups (unit_rows); 64: FP6 activations
};

// Workgroups of a unit-dealt launch: enough for every unit of max_groups
// groups x n_fb feature blocks to be taken in halves (see xcd_unit_split).
inline unsigned unit_grid(int max_groups, int n_fb) {
  const size_t halves = 2 * (size_t)max_groups * n_fb;
  size_t per = (halves + kXcds - 1) / kXcds;
  per += per & 1;
  return (unsigned)(kXcds * per);
}

// max_groups: capacity of the work list (max_work_groups for a.rows)
hipError_t launch_gateup(const ExpertArgs& a, int max_groups, hipStream_t stream);
hipError_t launch_down(const ExpertArgs& a, int max_groups, hipStream_t stream);

// residual: bf16 [N][d] added before the rounding, or NULL (may equal out)
hipError_t launch_combine(const float* y, const int32_t* inv, const float* gates, int n_rows, int d, int k,
                          int P, int has_shared, float route_scale, const uint16_t* residual, uint16_t* out,
                          hipStream_t stream);

// Shared expert with bf16 weights: h = silu(min(Wg x, L)) * clamp(Wu x) as bf16
// [N][I]; y_sh [N][d] = Wd h in fp32 (the shared rows of y).  d and I
// multiples of 64.
hipError_t launch_shared_bf16_gateup(const uint16_t* x, int n_rows, int d, int I, const uint16_t* wg,
                                     const uint16_t* wu, float limit, uint16_t* h, hipStream_t stream);
hipError_t launch_shared_bf16_down(const uint16_t* h, int n_rows, int d, int I, const uint16_t* wd, float* y_sh,
                                   hipStream_t stream);

// The same two GEMMs on weights packed by launch_pack_bf16 (bf16-MFMA
// fragments), streamed per wave instead of tiled through LDS: faster for
// large batches.  d and I multiples of 512.
constexpr int kSharedStreamRows = 2048;  // batches from this size take the streamed kernels
hipError_t launch_shared_stream_gateup(const uint16_t* x, int n_rows, int d, int I, const uint8_t* wg_p,
                                       const uint8_t* wu_p, float limit, uint16_t* h, hipStream_t stream);
hipError_t launch_shared_stream_down(const uint16_t* h, int n_rows, int d, int I, const uint8_t* wd_p, float* y_sh,
                                     hipStream_t stream);

// bf16 matrices [rows][K] (rows % 16 == 0, K % 32 == 0) into bf16-MFMA
// fragments: fragment (rt, ks) at byte (rt * K/32 + ks) * 1024, lane l holding
// row 16 rt + l % 16, values 32 ks + 8 (l / 16) .. +7.
hipError_t launch_pack_bf16(const uint8_t* w, int n_mat, int rows, int K, uint8_t* out, hipStream_t stream);

// ---------------------------------------------------------------------------
// Routed experts in Q2_K (k_q2k.hip).  Packed matrix [R][K] (R % 16 == 0,
// K % 256 == 0): 16-row tile rt, super-block b at byte (rt * K/256 + b) * 1344.
constexpr int kQ2kBlockBytes = 84;   // one 256-value super-block of one row
constexpr int kQ2kTileBytes = 1344;  // 16 rows of one super-block, packed
__host__ __device__ inline size_t q2k_matrix_bytes(int rows, int K) {
  return (size_t)rows * (size_t)(K / 256) * kQ2kBlockBytes;
}

hipError_t launch_pack_q2k(const uint8_t* q, int n_mat, int rows, int K, uint8_t* out, hipStream_t stream);

// Per activation row of length K (bf16, or fp16 when f16): pairs
// [rows][K/256][16] (hi | lo << 16 in the same type, of each 16-value
// sub-block sum) and X [rows][K/256] (fp32 super-block sums).
hipError_t launch_q2k_sums(const uint16_t* act, int rows, int K, bool f16, uint32_t* pairs, float* X,
                           hipStream_t stream);

struct Q2kArgs {
  const uint8_t *w0, *w1;  // packed Q2_K experts: gate and up (gate/up), or down (w0)
  const uint16_t* act;     // bf16 activation rows [*][K]: x (reached through perm) or h (pair order)
  const uint32_t* pairs;   // sub-block sums of the activation rows (launch_q2k_sums)
  const float* X;
  const int32_t* perm;
  const Group* groups;
  const int32_t* n_groups;
  int K, R, k, rows;       // contraction, output width, top-k, rows of the work list's groups
  int P;                   // routed pairs (N * k)
  float limit;             // swiglu limit (<= 0: none)
  uint16_t* h;             // gate/up output: [P][R], fp16 when h_f16, else bf16
  int h_f16;               // h in fp16 (gate/up writes it, down reads it); needs |h| < 65504
  float* y;                // down output: fp32 [P][R]
  int32_t* pool;           // claim counter (zeroed before the launch)
};

hipError_t launch_q2k_gateup(const Q2kArgs& a, int max_groups, hipStream_t stream);
hipError_t launch_q2k_down(const Q2kArgs& a, int max_groups, hipStream_t stream);

// LDS of a Q2_K work unit whose 16 activation rows of length K stay resident
// for the whole contraction (rows + sub-block pairs + X, padded rows).
__host__ __device__ inline size_t q2k_resident_lds_bytes(int K) {
  return 16 * (size_t)(2 * K + 16) + 16 * (size_t)(K / 4 + 16) + (size_t)(K / 256) * 64;
}
constexpr size_t kQ2kResidentMaxLds = 160 * 1024 - 256;  // 160 KB of LDS less room for the static claim slot

// Rows of the Q2_K work list's groups: 64 once the batch has at least 32
// routed rows per expert on average (prefill-like); else 16, whose units keep
// their activations resident in LDS (both GEMMs' K = d and I fit at d, I <=
// 4096), or, where they do not fit, 32 from kWideUnitPairs pairs on.
inline int q2k_unit_rows(int n_pairs, int E, int d, int I) {
  if (n_pairs >= 32 * E) return kTallGroupRows;
  const int K = d > I ? d : I;
  if (q2k_resident_lds_bytes(K) <= kQ2kResidentMaxLds) return kGroupRows;
  if (n_pairs >= kWideUnitPairs) return kMediumGroupRows;
  return kGroupRows;
}

// Worst-case number of work groups of <= rows rows each for n_rows rows:
// sum_e ceil(c_e/rows) <= ceil(P/rows) + E, plus the shared rows.
inline int max_work_groups(int n_rows, int k, int E, int has_shared, int rows = kGroupRows) {
  const long P = (long)n_rows * k;
  return (int)((P + rows - 1) / rows + E + (has_shared ? (n_rows + rows - 1) / rows : 0));
}

}  // namespace moe
