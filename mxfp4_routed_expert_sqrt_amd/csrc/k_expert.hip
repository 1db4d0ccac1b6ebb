// Grouped expert GEMMs on v_mfma_scale_f32_16x16x128_f8f6f4.
//
// A operand = the expert's MXFP4 weight rows (E2M1, with their E8M0 scales
// fed to the MFMA directly, so there is no dequantisation step); B operand =
// activations as two FP8 (E4M3) terms with per-32 E8M0 scales (x ~= q1*2^e1 +
// q2*2^e2), or two FP6 (E2M3) terms on tall work units, so every product is
// weight * (q1 + q2) accumulated in fp32.
//
// One workgroup = one work unit = (group of <= 16, 32 or 64 rows of one expert
// = NB MFMA column tiles, a block of output features).  4 or 8 waves per
// workgroup, each with several 16-row weight tiles.
// Weight fragments go straight from HBM into a 4-deep register ring per wave:
// the packed layout makes each wave's 16-byte-per-lane load one contiguous
// kilobyte, and every weight byte is used by exactly one wave.  The
// activations, which all waves of the workgroup share, are staged once per
// workgroup through LDS in chunks of 4 k-steps (double-buffered), so the
// waves' vector-memory queues carry weight bytes only.
//
// Lane layout of the 16x16x128 scaled MFMA (measured on gfx950; the probe test
// pins it): lane l supplies row/column l%16; a 4-bit operand holds K values
// 32*(l/16)..+31 (low nibble first), an 8-bit operand holds K values
// 16*(l/16)..+15 and 64+16*(l/16)..+15, a 6-bit operand holds K values
// 32*(l/16)..+31 as a 192-bit little-endian string (value i at bits 6i, dwords
// 0-5 of the 8-dword operand); the E8M0 scale of 32-block b of
// row/column n is byte `opsel` of lane n+16b's scale register; the fp32 result
// has D[4*(l/16) + i][l%16] in element i of lane l.
#include "kernels.h"

namespace moe {

template <int J, bool FP6 = false>
__device__ __forceinline__ v4f mfma_fp4_fp8(const u32x4& a, const v8i& b, const v4f& c, uint32_t sa, uint32_t sb) {
  const v8i av = {(int)a[0], (int)a[1], (int)a[2], (int)a[3], 0, 0, 0, 0};
  return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(av, b, c, 4 /* A: E2M1 */, FP6 ? 2 /* B: E2M3 */ : 0 /* E4M3 */,
                                                          J, (int)sa, J, (int)sb);
}

// v, hidden from the optimiser: the constant indices of the loads that start
// the next unit go through it, so the address arithmetic that depends on them
// is done where they are issued instead of being hoisted out of the loop over
// units and held in registers for the whole kernel.
__device__ __forceinline__ int opaque(int v) {
  asm volatile("" : "+s"(v));
  return v;
}

// threadIdx.x, hidden from the optimiser in the same way: the lane arithmetic
// of the code that runs once per unit (row lookup, epilogue addresses) and of
// the activation staging is done where it runs instead of being held in
// registers across the K loop.
__device__ __forceinline__ int opaque_tid() {
  int t = threadIdx.x;
  asm volatile("" : "+v"(t));
  return t;
}

// Pointers into global memory (activation rows, and the weight tiles below):
// loads and stores through them are global, never flat, however the pointer
// was obtained.
typedef const __attribute__((address_space(1))) uint8_t* gptr;
template <class T>
__device__ __forceinline__ __attribute__((address_space(1))) T* to_global(T* p) {
  return (__attribute__((address_space(1))) T*)p;
}

// ---------------------------------------------------------------------------
// Activation chunk in LDS: 4 k-steps of the 16 * NB token rows of a unit,
// row-major.  Row r of the unit (tile r / 16, column r % 16) holds its chunk
// bytes as they lie in the split row (FP8: 4 k-steps x 256, each [lane group
// g][term][two 16-byte runs]; FP6: 4 k-steps x 2 terms x 96, operand dwords
// 0-3 of lane groups 0..3 then dwords 4-5) at r * kRowStride, followed by the
// B scales of the NB tiles (per tile [term][group][col] as dwords, 512 B).
// Each wave stages whole rows: one load per lane (16 bytes, FP6 12) covers a
// row's chunk bytes, contiguous, and is stored at the same offsets, so a
// load touches 8 (FP6 6) cache lines instead of one per 32-64 bytes used.
// Strides: FP8 1040 bytes (16 mod 128), so the 8 lanes of a 16-byte fragment
// read cycle fall in distinct banks; FP6 776 bytes (8 mod 128), whose
// fragment reads are done as 8-byte pieces, 16 lanes a cycle.
constexpr int kRing = 4;           // weight ring slots per wave (4 or 8)
constexpr int kDownUnitMax = 512;  // widest down work unit (features)

template <bool FP6>
struct RowLayout {
  static constexpr int kStepBytes = FP6 ? 192 : 256;  // one k-step of a split row
  static constexpr int kLoadBytes = kStepBytes / 16;  // per lane: a row chunk is 64 loads
  static constexpr int kStride = FP6 ? 776 : 1040;
};

// Bytes of one chunk buffer, and the offset of tile tt's B scales in it.
template <int NB, bool FP6>
__host__ __device__ constexpr int chunk_buf_bytes() {
  return 16 * NB * RowLayout<FP6>::kStride + NB * 512;
}
template <int NB, bool FP6>
__device__ __forceinline__ constexpr int scale_off(int tt) {
  return 16 * NB * RowLayout<FP6>::kStride + tt * 512;
}

// Rows a wave stages per chunk: the unit's 16 * NB rows over THREADS / 64 waves.
template <int THREADS, int NB>
__host__ __device__ constexpr int rows_per_wave() {
  return 16 * NB * 64 / THREADS;
}

// This thread's share of one chunk (global -> registers -> LDS).  Wave w
// stages rows rows_per_wave * w + i; brow_q holds their pointers, lane i for
// row i (the other lanes repeat them), read out to a wave-uniform address per
// load.  The chunk's 128*NB scale dwords are carried as dword tid + THREADS*i
// (tile (tid + THREADS*i) >> 7), from the scale row brow_s[i].
template <int THREADS, int NB, bool FP6 = false>
struct ChunkStage {
  static constexpr int kRows = rows_per_wave<THREADS, NB>();
  static_assert(kRows >= 1 && kRows <= 16 && (kRows & (kRows - 1)) == 0, "chunk staging shape");
  static constexpr int kScales = (128 * NB + THREADS - 1) / THREADS;
  typedef RowLayout<FP6> L;
  typedef uint32_t u32x3 __attribute__((ext_vector_type(3)));
  typedef typename std::conditional<FP6, u32x3, u32x4>::type Piece;
  Piece q[kRows];
  uint32_t s[kScales];

  __device__ __forceinline__ void load(gptr brow_q, const gptr (&brow_s)[kScales], int sg, int nks, int n_sg) {
    const int tid = opaque_tid();
    // lane l: kLoadBytes at row chunk offset l * kLoadBytes = k-step l / 16
    // (clamped: past the end any valid step, never multiplied), byte (l % 16) * kLoadBytes
    const int l = tid & 63;
    const uint32_t off = (uint32_t)min(4 * sg + (l >> 4), nks - 1) * L::kStepBytes + L::kLoadBytes * (l & 15);
    const uint64_t rp = (uint64_t)brow_q;
    const uint32_t lo = (uint32_t)rp, hi = (uint32_t)(rp >> 32);
#pragma unroll
    for (int i = 0; i < kRows; ++i) {
      // (each half as uint32_t: a signed low word would sign-extend into the high one)
      const uint32_t rlo = (uint32_t)__builtin_amdgcn_readlane((int)lo, i);
      const uint32_t rhi = (uint32_t)__builtin_amdgcn_readlane((int)hi, i);
      const gptr row = (gptr)(((uint64_t)rhi << 32) | rlo);
      q[i] = *(const __attribute__((address_space(1))) Piece*)(row + off);
    }
#pragma unroll
    for (int i = 0; i < kScales; ++i) {
      const int u = tid + THREADS * i;
      if (u < 128 * NB) {
        const int t = (u >> 6) & 1, g = (u >> 4) & 3;
        s[i] = *(const __attribute__((address_space(1))) uint32_t*)(brow_s[i] + (size_t)(t * n_sg + sg) * 16 + g * 4);
      }
    }
  }

  __device__ __forceinline__ void store(uint8_t* buf) const {
    const int tid = threadIdx.x, wave = tid >> 6, l = tid & 63;
#pragma unroll
    for (int i = 0; i < kRows; ++i) {
      uint8_t* dst = buf + (kRows * wave + i) * L::kStride + L::kLoadBytes * l;
      if constexpr (FP6) {
        ((uint32_t*)dst)[0] = q[i][0];
        ((uint32_t*)dst)[1] = q[i][1];
        ((uint32_t*)dst)[2] = q[i][2];
      } else {
        *(u32x4*)dst = q[i];
      }
    }
#pragma unroll
    for (int i = 0; i < kScales; ++i) {
      const int u = tid + THREADS * i;
      if (u < 128 * NB) *(uint32_t*)(buf + scale_off<NB, FP6>(u >> 7) + (u & 127) * 4) = s[i];
    }
  }
};

template <int NA>
struct WFrag {
  u32x4 A[NA];
};

// Wave-uniform pointer into global memory: kept in scalar registers, so each
// weight load is "scalar base + one shared per-lane offset".

__device__ __forceinline__ gptr uniform_gptr(const uint8_t* p) {
  const uint64_t v = (uint64_t)p;
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)v);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(v >> 32));
  return (gptr)(((uint64_t)hi << 32) | lo);
}

// Weight fragment of k-step ks of each tile.  NT: non-temporal loads.
template <bool NT, int NA>
__device__ __forceinline__ void load_w(WFrag<NA>& f, const gptr (&wq)[NA], int ks) {
  const uint32_t off = (threadIdx.x & 63) * 16 + (uint32_t)ks * 1024;
#pragma unroll
  for (int a = 0; a < NA; ++a) {
    const __attribute__((address_space(1))) u32x4* p = (const __attribute__((address_space(1))) u32x4*)(wq[a] + off);
    f.A[a] = NT ? __builtin_nontemporal_load(p) : *p;
  }
}

template <int NA>
__device__ __forceinline__ void load_wscales(uint32_t (&sa)[NA], const gptr (&ws)[NA], int sg) {
  const uint32_t off = (threadIdx.x & 63) * 4 + (uint32_t)sg * 256;
#pragma unroll
  for (int a = 0; a < NA; ++a) sa[a] = *(const __attribute__((address_space(1))) uint32_t*)(ws[a] + off);
}

// k-step J of the current chunk: B (NB column tiles) from LDS, weights from a
// ring slot; every weight fragment meets every column tile.  The 2*NB B
// fragments are taken term-major (i = t*NB + tt), so the two terms of one
// accumulator are NA*NB MFMAs apart, and double-buffered: fragment i+1 is read
// from LDS before fragment i's MFMAs are issued, so the LDS latency is
// covered by MFMA work.
template <int J, int NB, bool FP6>
__device__ __forceinline__ v8i read_b(const uint8_t* chunk, int i) {
  const int lane = threadIdx.x & 63, tt = i % NB, t = i / NB, col = lane & 15, g = lane >> 4;
  if constexpr (FP6) {
    const uint8_t* c = chunk + (16 * tt + col) * RowLayout<true>::kStride + J * 192 + t * 96;
    const u32x2 w0 = *(const u32x2*)(c + g * 16);
    const u32x2 w1 = *(const u32x2*)(c + g * 16 + 8);
    const u32x2 w2 = *(const u32x2*)(c + 64 + g * 8);
    return v8i{(int)w0[0], (int)w0[1], (int)w1[0], (int)w1[1], (int)w2[0], (int)w2[1], 0, 0};
  } else {
    const uint8_t* c = chunk + (16 * tt + col) * RowLayout<false>::kStride + J * 256 + g * 64 + t * 32;
    const u32x4 lo = *(const u32x4*)c;
    const u32x4 hi = *(const u32x4*)(c + 16);
    return v8i{(int)lo[0], (int)lo[1], (int)lo[2], (int)lo[3], (int)hi[0], (int)hi[1], (int)hi[2], (int)hi[3]};
  }
}

// nbu (wave-uniform): column tiles multiplied; the MFMAs of tiles past it
// (padding rows of a unit whose rows fit in fewer tiles) are branched over.
template <int J, int NA, int NB, bool FP6>
__device__ __forceinline__ void mma_step(const WFrag<NA>& f, const uint8_t* chunk, const uint32_t (&sa)[NA],
                                         const uint32_t (&sb)[NB][2], v4f (&acc)[NA][NB], int nbu = NB) {
  constexpr int NF = 2 * NB;
  v8i b0 = read_b<J, NB, FP6>(chunk, 0), b1;
#pragma unroll
  for (int i = 0; i < NF; ++i) {
    v8i& cur = (i & 1) ? b1 : b0;
    v8i& nxt = (i & 1) ? b0 : b1;
    const int tt = i % NB, t = i / NB;
    if (i + 1 < NF) nxt = read_b<J, NB, FP6>(chunk, i + 1);
    if (NF > 2) __builtin_amdgcn_sched_barrier(0);  // keep the read ahead of these MFMAs
    if (tt < 2 || tt < nbu) {  // (tiles 0 and 1 always: no branch for them)
#pragma unroll
      for (int a = 0; a < NA; ++a) acc[a][tt] = mfma_fp4_fp8<J, FP6>(f.A[a], cur, acc[a][tt], sa[a], sb[tt][t]);
    }
    if (NF > 2) __builtin_amdgcn_sched_barrier(0);
  }
}

// Weight tiles and activation rows a unit's loads come from (brow_q: the
// staged rows, brow_s: the scale rows, as ChunkStage takes them).
template <int NA, int NB, int NS, bool FP6 = false>
struct UnitSrc {
  gptr aq[NA], as[NA];
  gptr brow_q;
  gptr brow_s[NS];
};

// One group of 4 k-steps: chunk sg of the activations is in LDS at `chunk`,
// and chunk sg+1 is written to `next_buf` at the end.  Weights: ring slot of
// step ks is ks % RING; while step ks is multiplied the fragments of
// ks+1 .. ks+RING-1 are in flight.  GI = position of this group inside a ring
// cycle (RING/4 groups per cycle), so every slot index and scale byte is a
// compile-time constant.
// Loads past the end of the unit (the chunk after the last, weight steps
// past the last) re-read the last chunk and step (valid addresses, never
// multiplied).
// The chunk loaded during the group is chunk cc of cs (in a unit's K loop:
// chunk sg+1 of the unit, clamped).
template <int GI, int RING, int NA, int THREADS, int NB, bool NT, bool FP6>
__device__ __forceinline__ void k_group(WFrag<NA> (&f)[RING], ChunkStage<THREADS, NB, FP6>& stage,
                                        uint32_t (&sa)[NA], uint32_t (&sa_n)[NA],
                                        const UnitSrc<NA, NB, ChunkStage<THREADS, NB>::kScales, FP6>& cur, int sg,
                                        int nks, int n_sg, v4f (&acc)[NA][NB], const uint8_t* chunk,
                                        uint8_t* next_buf,
                                        const UnitSrc<NA, NB, ChunkStage<THREADS, NB>::kScales, FP6>& cs, int cc,
                                        int nbu = NB) {
  const int lane = threadIdx.x & 63, last = nks - 1, k0 = 4 * sg;
  uint32_t sb[NB][2];
#pragma unroll
  for (int tt = 0; tt < NB; ++tt) {
    sb[tt][0] = *(const uint32_t*)(chunk + scale_off<NB, FP6>(tt) + lane * 4);
    sb[tt][1] = *(const uint32_t*)(chunk + scale_off<NB, FP6>(tt) + 256 + lane * 4);
  }
  // weight step loaded at position j of the group (RING-1+j steps ahead)
  auto load_step = [&](WFrag<NA>& slot, int j) { load_w<NT>(slot, cur.aq, min(k0 + RING - 1 + j, last)); };
  stage.load(cs.brow_q, cs.brow_s, cc, nks, n_sg);
  load_wscales(sa_n, cur.as, min(sg + 1, n_sg - 1));
  load_step(f[(4 * GI + RING - 1) % RING], 0);
  __builtin_amdgcn_sched_barrier(0);
  mma_step<0, NA, NB, FP6>(f[(4 * GI) % RING], chunk, sa, sb, acc, nbu);
  __builtin_amdgcn_sched_barrier(0);
  load_step(f[(4 * GI + RING) % RING], 1);
  __builtin_amdgcn_sched_barrier(0);
  if (k0 + 1 < nks) mma_step<1, NA, NB, FP6>(f[(4 * GI + 1) % RING], chunk, sa, sb, acc, nbu);
  __builtin_amdgcn_sched_barrier(0);
  load_step(f[(4 * GI + RING + 1) % RING], 2);
  __builtin_amdgcn_sched_barrier(0);
  if (k0 + 2 < nks) mma_step<2, NA, NB, FP6>(f[(4 * GI + 2) % RING], chunk, sa, sb, acc, nbu);
  __builtin_amdgcn_sched_barrier(0);
  load_step(f[(4 * GI + RING + 2) % RING], 3);
  __builtin_amdgcn_sched_barrier(0);
  if (k0 + 3 < nks) mma_step<3, NA, NB, FP6>(f[(4 * GI + 3) % RING], chunk, sa, sb, acc, nbu);
  __builtin_amdgcn_sched_barrier(0);
  stage.store(next_buf);
  __syncthreads();
#pragma unroll
  for (int a = 0; a < NA; ++a) sa[a] = sa_n[a];
}

// The loads that start a unit's K loop: chunk 0 into LDS at buf, the weight
// scales of chunk 0 and the first RING-1 weight steps.
template <int RING, int NA, int THREADS, int NB, bool NT, bool FP6>
__device__ __forceinline__ void k_start(WFrag<NA> (&f)[RING], ChunkStage<THREADS, NB, FP6>& stage, uint32_t (&sa)[NA],
                                        const UnitSrc<NA, NB, ChunkStage<THREADS, NB>::kScales, FP6>& cur, int nks,
                                        uint8_t* buf) {
  const int n_sg = (nks + 3) / 4, last = nks - 1;
  stage.load(cur.brow_q, cur.brow_s, 0, nks, n_sg);
  load_wscales(sa, cur.as, 0);
#pragma unroll
  for (int i = 0; i < RING - 1; ++i) load_w<NT>(f[i], cur.aq, min(i, last));
  stage.store(buf);
  __syncthreads();
}

// K loop of one unit.  Weights: a register ring of RING k-step fragments
// (RING-1 steps in flight ahead of the one being multiplied; weight scales
// one group of 4 k-steps ahead).  Activations: chunk sg+1 is fetched into
// registers at the start of group sg and written to the other LDS buffer at
// its end, then one workgroup barrier per group (it waits on LDS traffic
// only, not on the weight loads in flight).  Loads are unconditional (clamped
// indices) and the sched_barrier(0) points keep their issue order, so each
// wait on the in-order vector-memory counter covers only what is about to be
// used.  RING = 8 needs the group count to be even.
template <int RING, int NA, int THREADS, int NB, bool NT, bool FP6>
__device__ __forceinline__ void mainloop(const UnitSrc<NA, NB, ChunkStage<THREADS, NB>::kScales, FP6>& src, int nks,
                                         v4f (&acc)[NA][NB], uint8_t* lds) {
  static_assert(RING == 4 || RING == 8, "ring of 1 or 2 groups");
  constexpr int kBuf = chunk_buf_bytes<NB, FP6>();
  const int n_sg = (nks + 3) / 4;
  ChunkStage<THREADS, NB, FP6> stage;
  WFrag<NA> f[RING];
  uint32_t sa[NA], sa_n[NA];
  k_start<RING, NA, THREADS, NB, NT, FP6>(f, stage, sa, src, nks, lds);
  for (int sg = 0; sg < n_sg; sg += RING / 4) {
    k_group<0, RING, NA, THREADS, NB, NT, FP6>(f, stage, sa, sa_n, src, sg, nks, n_sg, acc,
                                               lds + (sg & 1) * kBuf, lds + ((sg + 1) & 1) * kBuf, src,
                                               min(sg + 1, n_sg - 1));
    if (RING == 8)
      k_group<1, RING, NA, THREADS, NB, NT, FP6>(f, stage, sa, sa_n, src, sg + 1, nks, n_sg, acc,
                                                 lds + ((sg + 1) & 1) * kBuf, lds + (sg & 1) * kBuf, src,
                                                 min(sg + 2, n_sg - 1));
  }
}

// Rows staged by this thread, as positions in the unit's group (padding
// positions past its rows reuse the group's first row): slot 0 is the row
// rows_per_wave * wave + lane % rows_per_wave (lane i < rows_per_wave holds
// the row of the wave's i-th load), slots 1.. the row of each scale dword.
template <int THREADS, int NB>
__host__ __device__ constexpr int row_slots() {
  return 1 + (128 * NB + THREADS - 1) / THREADS;
}

template <int THREADS, int NB>
__device__ __forceinline__ int slot_pos(int k) {
  constexpr int R = rows_per_wave<THREADS, NB>();
  const int tid = opaque_tid();
  if (k == 0) return R * (tid >> 6) + (tid & (R - 1));
  return 16 * min((tid + THREADS * (k - 1)) >> 7, NB - 1) + (tid & 15);
}

__device__ __forceinline__ int group_pair(const Group& g, int c) { return g.p0 + (c < g.cnt ? c : 0); }

// Row pointers from the rows (token rows of x, or pair rows of h) of the slots.
template <int THREADS, int NB, int NA, bool FP6>
__device__ __forceinline__ void row_ptrs(const ExpertArgs& a, const int (&row)[row_slots<THREADS, NB>()], int K,
                                         UnitSrc<NA, NB, ChunkStage<THREADS, NB>::kScales, FP6>& src) {
  src.brow_q = to_global(a.aq) + (size_t)row[0] * split_q_row_bytes(K);
#pragma unroll
  for (int i = 0; i < ChunkStage<THREADS, NB>::kScales; ++i)
    src.brow_s[i] = to_global(a.as) + (size_t)row[1 + i] * split_s_row_bytes(K);
}

// pair_rows: the activation rows are in pair order (h for down); otherwise
// they are token rows of x reached through perm (the shared expert's rows
// follow the routed pairs in natural order).
template <int THREADS, int NB, int NA, bool FP6>
__device__ __forceinline__ void stage_rows(const ExpertArgs& a, const Group g, int K, bool shared, bool pair_rows,
                                           UnitSrc<NA, NB, ChunkStage<THREADS, NB>::kScales, FP6>& src) {
  constexpr int NR = row_slots<THREADS, NB>();
  int row[NR];
#pragma unroll
  for (int k = 0; k < NR; ++k) {
    const int p = group_pair(g, slot_pos<THREADS, NB>(k));
    // (perm entries clamped into [0, P): a bad entry gives a wrong row, never an access out of bounds)
    row[k] = pair_rows ? p : (shared ? p - a.P : min(max(to_global(a.perm)[p], 0), a.P - 1) / a.k);
  }
  row_ptrs<THREADS, NB, NA, FP6>(a, row, K, src);
}

// Weight tile pointers of this wave: gate/up takes TPM 16-row tiles of gate
// and the same rows of up from feature f0 (NA = 2 TPM), down NA tiles.
template <int NA, bool GU>
__device__ __forceinline__ void weight_ptrs(const ExpertArgs& a, const Group& g, int f0, gptr (&aq)[NA],
                                            gptr (&as)[NA]) {
  const int K = a.K, R = a.R, nks = K / 128, n_sg = (nks + 3) / 4, rt0 = f0 / 16;
  const bool shared = g.e == a.E;
  const size_t mq = packed_q_bytes(R, K), ms = packed_s_bytes(R, K);
  const size_t tq = (size_t)nks * 1024, ts = (size_t)n_sg * 256;  // one 16-row tile
  const uint8_t* q0 = shared ? a.sq0 : a.q0 + (size_t)g.e * mq;
  const uint8_t* s0 = shared ? a.ss0 : a.s0 + (size_t)g.e * ms;
  if constexpr (GU) {
    constexpr int TPM = NA / 2;
    const uint8_t* q1 = shared ? a.sq1 : a.q1 + (size_t)g.e * mq;
    const uint8_t* s1 = shared ? a.ss1 : a.s1 + (size_t)g.e * ms;
#pragma unroll
    for (int i = 0; i < TPM; ++i) {
      aq[i] = uniform_gptr(q0 + (rt0 + i) * tq);
      aq[TPM + i] = uniform_gptr(q1 + (rt0 + i) * tq);
      as[i] = uniform_gptr(s0 + (rt0 + i) * ts);
      as[TPM + i] = uniform_gptr(s1 + (rt0 + i) * ts);
    }
  } else {
#pragma unroll
    for (int i = 0; i < NA; ++i) {
      aq[i] = uniform_gptr(q0 + (rt0 + i) * tq);
      as[i] = uniform_gptr(s0 + (rt0 + i) * ts);
    }
  }
}

// ---------------------------------------------------------------------------
// gate/up: h = silu(min(gate, L)) * clamp(up, -L, L), written as the two-term
// split that the down GEMM consumes (FP8, or FP6 on tall units; the layout of
// the x split with K = I).
// Each of the WAVES waves takes TPM 16-row tiles of the gate matrix and the
// same rows of the up matrix: 16*TPM features per wave, 16*TPM*WAVES per work
// unit.

// Tall gate/up epilogue (4 column tiles, FP6 h): for each 32-feature block of
// the wave, lane (col, grp) first forms h of token 16c + col for every column
// tile c (8 values: features 4grp..4grp+3 and 16+4grp..+3 of the block).  A
// 4 x 4 exchange over the lane rows (two rounds of permlane swaps) then gives
// lane (col, r) the whole block of token 16r + col: slot q holds what row q
// had for tile r.  Each lane splits its block into two E2M3 terms with the
// hardware conversions (split_fp6_32) and stores them as its operand dwords
// (the x split's FP6 layout, K = I).
template <int TPM>
__device__ __forceinline__ void gateup_epilogue_tall(const ExpertArgs& a, const Group g, int f0,
                                                     const v4f (&acc)[2 * TPM][4]) {
  const int lane = opaque_tid() & 63, col = lane & 15, r = lane >> 4;
  const int n_sg_h = (a.R / 128 + 3) / 4;
  const float L = a.limit;
#pragma unroll
  for (int b = 0; b < TPM / 2; ++b) {
    const int blk_h = f0 / 32 + b;
    float h[4][8];
#pragma unroll
    for (int c = 0; c < 4; ++c)
#pragma unroll
      for (int tt = 0; tt < 2; ++tt)
#pragma unroll
        for (int ii = 0; ii < 4; ++ii) {
          float gv = acc[2 * b + tt][c][ii], uv = acc[TPM + 2 * b + tt][c][ii];
          if (L > 0.f) {
            gv = fminf(gv, L);
            uv = fminf(fmaxf(uv, -L), L);
          }
          h[c][tt * 4 + ii] = gv * __builtin_amdgcn_rcpf(1.f + __expf(-gv)) * uv;  // silu with a 1-ulp reciprocal
        }
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      swap32(h[0][k], h[2][k]);
      swap32(h[1][k], h[3][k]);
    }
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      swap16(h[0][k], h[1][k]);
      swap16(h[2][k], h[3][k]);
    }
    // h[q][k]: feature 4q + k (k < 4) or 16 + 4q + k - 4 (k >= 4) of the block
    v16f ev, od;
#pragma unroll
    for (int q = 0; q < 4; ++q)
#pragma unroll
      for (int k = 0; k < 8; ++k) {
        const int j = k < 4 ? 4 * q + k : 12 + 4 * q + k;
        if (j & 1)
          od[j >> 1] = h[q][k];
        else
          ev[j >> 1] = h[q][k];
      }
    u32x6 t1, t2;
    int e1, e2;
    split_fp6_32(ev, od, &t1, &t2, &e1, &e2);
    if (16 * r + col < g.cnt) {
      const size_t p = (size_t)g.p0 + 16 * r + col;
      __attribute__((address_space(1))) uint8_t* dst =
          to_global(a.hq) + p * split_q_row_bytes(a.R) + (size_t)(blk_h >> 2) * kFp6StepBytes;
      const int gb = blk_h & 3;
      *(__attribute__((address_space(1))) u32x4*)(dst + 16 * gb) = u32x4{t1[0], t1[1], t1[2], t1[3]};
      *(__attribute__((address_space(1))) u32x2*)(dst + 64 + 8 * gb) = u32x2{t1[4], t1[5]};
      *(__attribute__((address_space(1))) u32x4*)(dst + kFp6TermBytes + 16 * gb) = u32x4{t2[0], t2[1], t2[2], t2[3]};
      *(__attribute__((address_space(1))) u32x2*)(dst + kFp6TermBytes + 64 + 8 * gb) = u32x2{t2[4], t2[5]};
      __attribute__((address_space(1))) uint8_t* srow = to_global(a.hs) + p * split_s_row_bytes(a.R);
      srow[split_scale_offset(0, blk_h, n_sg_h)] = (uint8_t)(e1 + 127);
      srow[split_scale_offset(1, blk_h, n_sg_h)] = (uint8_t)(e2 + 127);
    }
  }
}

// gate/up epilogue: h of this wave's features [f0, f0 + 16 TPM) for the rows
// of group g, from the gate (acc[0..TPM)) and up (acc[TPM..2TPM)) sums.
template <int TPM, int NB, bool FP6>
__device__ __forceinline__ void gateup_epilogue(const ExpertArgs& a, const Group g, int f0,
                                                const v4f (&acc)[2 * TPM][NB]) {
  const int lane = opaque_tid() & 63, col = lane & 15, grp = lane >> 4;
  const int R = a.R;
  const int n_sg_h = (R / 128 + 3) / 4;
  const float L = a.limit;
  // each pair of tiles (32 features) is one 32-block of h: 4 lanes (grp 0..3) x 8 values per token
#pragma unroll
  for (int c = 0; c < NB; ++c)
#pragma unroll
  for (int b = 0; b < TPM / 2; ++b) {
    const int blk_h = f0 / 32 + b;
    float h[8];
#pragma unroll
    for (int tt = 0; tt < 2; ++tt)
#pragma unroll
      for (int ii = 0; ii < 4; ++ii) {
        float gv = acc[2 * b + tt][c][ii], uv = acc[TPM + 2 * b + tt][c][ii];
        if (L > 0.f) {
          gv = fminf(gv, L);
          uv = fminf(fmaxf(uv, -L), L);
        }
        h[tt * 4 + ii] = gv * __builtin_amdgcn_rcpf(1.f + __expf(-gv)) * uv;  // silu with a 1-ulp reciprocal
      }
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
    if (16 * c + col < g.cnt) {
      const size_t p = (size_t)g.p0 + 16 * c + col;
      // feature 16tt + 4grp + ii of block blk_h = 4ks + bb: group 2*(bb%2) + tt, byte 16*(bb/2) + 4grp + ii
      const int bb = blk_h & 3;
      __attribute__((address_space(1))) uint8_t* dst =
          to_global(a.hq) + p * split_q_row_bytes(R) + (size_t)(blk_h >> 2) * 256 + 16 * (bb >> 1) + 4 * grp;
#pragma unroll
      for (int tt = 0; tt < 2; ++tt) {
        __attribute__((address_space(1))) uint8_t* gdst = dst + (2 * (bb & 1) + tt) * 64;
        *(__attribute__((address_space(1))) uint32_t*)(gdst) = w1[tt];
        *(__attribute__((address_space(1))) uint32_t*)(gdst + 32) = w2[tt];
      }
      if (grp == 0) {
        __attribute__((address_space(1))) uint8_t* srow = to_global(a.hs) + p * split_s_row_bytes(R);
        srow[split_scale_offset(0, blk_h, n_sg_h)] = (uint8_t)(e1 + 127);
        srow[split_scale_offset(1, blk_h, n_sg_h)] = (uint8_t)(e2 + 127);
      }
    }
  }
}


// One work unit: features [fu0, fu0 + WAVES*16*TPM) of gate and up for the
// rows of group g.
template <int TPM, int WAVES, int NB, int RING, bool NT, bool FP6>
__device__ __forceinline__ void gateup_unit(const ExpertArgs& a, const Group g, int fu0, uint8_t* lds) {
  constexpr int NA = 2 * TPM, kThreads = 64 * WAVES;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int nks = a.K / 128, f0 = fu0 + wave * 16 * TPM;
  UnitSrc<NA, NB, ChunkStage<kThreads, NB>::kScales, FP6> src;
  weight_ptrs<NA, true>(a, g, f0, src.aq, src.as);
  stage_rows<kThreads, NB, NA, FP6>(a, g, a.K, g.e == a.E, false, src);
  v4f acc[NA][NB];
#pragma unroll
  for (int i = 0; i < NA; ++i)
#pragma unroll
    for (int c = 0; c < NB; ++c) acc[i][c] = v4f{0.f, 0.f, 0.f, 0.f};
  if (RING == 8 && (nks % 8) == 0)
    mainloop<8, NA, kThreads, NB, NT, FP6>(src, nks, acc, lds);
  else
    mainloop<4, NA, kThreads, NB, NT, FP6>(src, nks, acc, lds);
  gateup_epilogue<TPM, NB, FP6>(a, g, f0, acc);
}

// POOL: units dealt by xcd_unit_claim (static ranges with a shared tail),
// else by xcd_unit_split (static ranges, optional tail halves).
template <int TPM, int WAVES, int NB, int RING, bool NT, bool FP6, bool POOL>
__global__ void __launch_bounds__(64 * WAVES) gateup_kernel(ExpertArgs a) {
  constexpr int kFeatUnit = WAVES * 16 * TPM;
  extern __shared__ __attribute__((aligned(16))) uint8_t lds[];  // 2 * chunk_buf_bytes<NB, FP6>()
  const int n_fb = a.R / kFeatUnit;
  int half_idx;
  bool is_half = false;
  if constexpr (POOL) {
    __shared__ int s_claim;
    half_idx = xcd_unit_claim(*a.n_groups * n_fb, a.pool, &s_claim);
    if (half_idx < 0) return;
  } else if (!xcd_unit_split(*a.n_groups * n_fb, TPM >= 4 ? a.tail_units : 0, &half_idx, &is_half)) {
    return;
  }
  int fb;
  const Group g = unit_group<FP6>(a.groups, half_idx >> 1, n_fb, &fb);
  const int fu0 = fb * kFeatUnit + (half_idx & 1) * (kFeatUnit / 2);
  if constexpr (TPM >= 4) {
    if (is_half) {
      gateup_unit<TPM / 2, WAVES, NB, RING, NT, FP6>(a, g, fu0, lds);
      return;
    }
  }
  if constexpr (NB == 2) {
    if (g.cnt <= 16) {  // one column tile holds the group: half the staging and MFMAs
      gateup_unit<TPM, WAVES, 1, RING, NT, FP6>(a, g, fu0, lds);
      return;
    }
  }
  gateup_unit<TPM, WAVES, NB, RING, NT, FP6>(a, g, fu0, lds);
}

// ---------------------------------------------------------------------------
// down: y[p][f] = sum_n W_down[e][f][n] h[p][n], fp32 rows in expert-major
// pair order (routed) followed by the shared expert's rows.  Each of the
// WAVES waves takes NA 16-row tiles: 16*NA features per wave, 16*NA*WAVES per
// unit.

// down epilogue: this wave's features [f0, f0 + 16 NA) of the y rows of group g.
template <int NA, int NB>
__device__ __forceinline__ void down_epilogue(const ExpertArgs& a, const Group g, int f0, const v4f (&acc)[NA][NB]) {
  const int lane = opaque_tid() & 63, col = lane & 15, grp = lane >> 4;
#pragma unroll
  for (int c = 0; c < NB; ++c)
    if (16 * c + col < g.cnt) {
      __attribute__((address_space(1))) float* dst = to_global(a.y) + ((size_t)g.p0 + 16 * c + col) * a.R + f0 + 4 * grp;
#pragma unroll
      for (int tt = 0; tt < NA; ++tt)
        __builtin_nontemporal_store(acc[tt][c], (__attribute__((address_space(1))) v4f*)(dst + 16 * tt));
    }
}

template <int NA, int WAVES, int NB, int RING, bool NT, bool FP6>
__device__ __forceinline__ void down_unit(const ExpertArgs& a, const Group g, int fu0, uint8_t* lds) {
  constexpr int kThreads = 64 * WAVES;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int nks = a.K / 128, f0 = fu0 + wave * 16 * NA;
  UnitSrc<NA, NB, ChunkStage<kThreads, NB>::kScales, FP6> src;
  weight_ptrs<NA, false>(a, g, f0, src.aq, src.as);
  stage_rows<kThreads, NB, NA, FP6>(a, g, a.K, g.e == a.E, true, src);
  v4f acc[NA][NB];
#pragma unroll
  for (int i = 0; i < NA; ++i)
#pragma unroll
    for (int c = 0; c < NB; ++c) acc[i][c] = v4f{0.f, 0.f, 0.f, 0.f};
  if (RING == 8 && (nks % 8) == 0)
    mainloop<8, NA, kThreads, NB, NT, FP6>(src, nks, acc, lds);
  else
    mainloop<4, NA, kThreads, NB, NT, FP6>(src, nks, acc, lds);
  down_epilogue<NA, NB>(a, g, f0, acc);
}

template <int NA, int WAVES, int NB, int RING, bool NT, bool FP6, bool POOL>
__global__ void __launch_bounds__(64 * WAVES) down_kernel(ExpertArgs a) {
  constexpr int kFeatUnit = WAVES * 16 * NA;
  extern __shared__ __attribute__((aligned(16))) uint8_t lds[];  // 2 * chunk_buf_bytes<NB, FP6>()
  const int n_fb = a.R / kFeatUnit;
  int half_idx;
  bool is_half = false;
  if constexpr (POOL) {
    __shared__ int s_claim;
    half_idx = xcd_unit_claim(*a.n_groups * n_fb, a.pool, &s_claim);
    if (half_idx < 0) return;
  } else if (!xcd_unit_split(*a.n_groups * n_fb, NA >= 2 ? a.tail_units : 0, &half_idx, &is_half)) {
    return;
  }
  int fb;
  const Group g = unit_group<FP6>(a.groups, half_idx >> 1, n_fb, &fb);
  const int fu0 = fb * kFeatUnit + (half_idx & 1) * (kFeatUnit / 2);
  if constexpr (NA >= 2) {
    if (is_half) {
      down_unit<NA / 2, WAVES, NB, RING, NT, FP6>(a, g, fu0, lds);
      return;
    }
  }
  if constexpr (NB == 2) {
    if (g.cnt <= 16) {  // one column tile holds the group: half the staging and MFMAs
      down_unit<NA, WAVES, 1, RING, NT, FP6>(a, g, fu0, lds);
      return;
    }
  }
  down_unit<NA, WAVES, NB, RING, NT, FP6>(a, g, fu0, lds);
}

// ---------------------------------------------------------------------------
// Tall units in persistent workgroups (one per CU).  Each workgroup runs units
// one after another and always holds the next one it will run, claimed a unit
// ahead: at the start of a unit's K loop the next unit's rows (perm) are
// fetched; the next unit's first activation chunk is loaded by this unit's
// last group in place of its own (clamped) one (down, whose rows are pair
// rows) or issued before this unit's epilogue (gate/up, whose rows come from
// perm), as are the next unit's weight scales and first RING-1 weight steps,
// so the next K loop starts with its data in place
// (a new workgroup per unit waits for the chain work list -> perm ->
// activations and weights instead).
// Claims: the next unit of the workgroup's XCD range in order (an atomic on
// the XCD's counter: consecutive units, which share weights under
// feature-block-major order, run side by side, and faster CUs take more
// units), past the range's static part (all but its last kPoolUnits units) a
// unit of the shared pool of the ranges' tails.
constexpr int kTallWorkgroups = 256;

// The launch's arguments, read again from the kernel-argument segment (the
// kernel's only argument is the ExpertArgs, at its start) through a pointer
// the optimiser cannot see through: the loop over units then fetches each
// field where it is used instead of holding every argument in scalar
// registers across all units.
__device__ __forceinline__ ExpertArgs reload_args() {
  static_assert(sizeof(ExpertArgs) % 4 == 0, "whole dwords");
  typedef const __attribute__((address_space(4))) uint32_t* kernarg_words;
  kernarg_words p = (kernarg_words)__builtin_amdgcn_kernarg_segment_ptr();
  asm volatile("" : "+s"(p));
  ExpertArgs r;
  uint32_t w[sizeof(ExpertArgs) / 4];
#pragma unroll
  for (size_t i = 0; i < sizeof(ExpertArgs) / 4; ++i) w[i] = p[i];
  __builtin_memcpy(&r, w, sizeof(r));
  return r;
}

// Word (threadIdx.x % 8) of work-list entry i, as a global load whose result
// is read out (entry_from_words) only where it is needed.
__device__ __forceinline__ int entry_word(const Group* groups, int i) {
  return ((const __attribute__((address_space(1))) int32_t*)(groups + i))[opaque_tid() & 7];
}

__device__ __forceinline__ Group entry_from_words(int w) {
  Group g;
  g.e = __builtin_amdgcn_readlane(w, 0), g.p0 = __builtin_amdgcn_readlane(w, 1);
  g.cnt = __builtin_amdgcn_readlane(w, 2), g.first = __builtin_amdgcn_readlane(w, 3);
  g.ng = __builtin_amdgcn_readlane(w, 4), g.seg_rows = __builtin_amdgcn_readlane(w, 5);
  g.seg_p0 = __builtin_amdgcn_readlane(w, 6), g.rows = __builtin_amdgcn_readlane(w, 7);
  return g;
}

template <int NA, int WAVES, bool GU>
__global__ void __launch_bounds__(64 * WAVES) tall_kernel(ExpertArgs a) {
  constexpr int NB = 4, RING = 4, kThreads = 64 * WAVES, NS = ChunkStage<kThreads, NB>::kScales;
  constexpr int kFeatWave = 16 * (GU ? NA / 2 : NA), kFeatUnit = WAVES * kFeatWave;
  constexpr int kBuf = chunk_buf_bytes<NB, true>(), NR = row_slots<kThreads, NB>();
  extern __shared__ __attribute__((aligned(16))) uint8_t lds[];  // 2 * kBuf
  __shared__ int s_claim[2];
  const int n_fb = a.R / kFeatUnit, n_units = *a.n_groups * n_fb;
  const int nks = a.K / 128, n_sg = (nks + 3) / 4;
  const int tid = threadIdx.x, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int xcd = blockIdx.x % kXcds;
  const int H = 2 * n_units;
  int per = (H + kXcds - 1) / kXcds;
  per += per & 1;
  const int nx = min(per, max(0, H - xcd * per)) / 2;
  const int n_static = nx - min(kPoolUnits, nx), u_base = xcd * per / 2;
  __attribute__((address_space(1))) int32_t* xctr = to_global(a.xcd_ctr) + xcd;
  // the unit of counter value t (thread 0 only): in order through the
  // static part, then from the pool (-1: none left)
  auto resolve = [&](int t, int32_t* pool) -> int {
    if (t < n_static) return u_base + t;
    const int h = pool_claim_one(n_units, pool);
    return h < 0 ? -1 : h >> 1;
  };
  if (tid == 0) {
    const int t0 = __hip_atomic_fetch_add(xctr, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    const int u0 = resolve(t0, a.pool);
    int u1 = -1;
    if (u0 >= 0) u1 = resolve(__hip_atomic_fetch_add(xctr, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT), a.pool);
    s_claim[0] = u0;
    s_claim[1] = u1;
  }
  __syncthreads();
  int u = s_claim[0], q = s_claim[1];
  if (u < 0) return;

  ChunkStage<kThreads, NB, true> stage;
  WFrag<NA> f[RING];
  uint32_t sa[NA], sa_n[NA];
  v4f acc[NA][NB];
  int fb;
  Group g = unit_group<true>(a.groups, u, n_fb, &fb);
  int f0 = fb * kFeatUnit + wave * kFeatWave;
  UnitSrc<NA, NB, NS, true> cur;
  weight_ptrs<NA, GU>(a, g, f0, cur.aq, cur.as);
  stage_rows<kThreads, NB, NA, true>(a, g, a.K, g.e == a.E, !GU, cur);
  k_start<RING, NA, kThreads, NB, false, true>(f, stage, sa, cur, nks, lds);
  // the queued unit (a workgroup's last unit queues itself: valid addresses,
  // never used): its group and feature block
  int uq = q >= 0 ? q : u;
  int fbq;
  Group gq = unit_group_of(entry_from_words(entry_word(a.groups, uq / n_fb)), uq, n_fb, &fbq);
  int bp = 0;  // LDS buffer of the unit's chunk 0
  while (true) {
    // claim the unit after the queued one; fetch the queued unit's rows
    // (the address goes through the opaque lane index, so the compiler does not
    // turn this one-thread atomic into a wave-wide one that waits for its
    // result, and with it every load in flight, right here)
    int t = 0;
    if (tid == 0 && q >= 0)
      t = __hip_atomic_fetch_add(xctr + min(opaque_tid(), 0), 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    int row[NR];
#pragma unroll
    for (int k = 0; k < NR; ++k) {
      const int p = group_pair(gq, slot_pos<kThreads, NB>(k));
      row[k] = GU ? min(max(to_global(a.perm)[min(p, a.P - 1)], 0), a.P - 1) : p;  // (clamped as in stage_rows)
    }
#pragma unroll
    for (int i = 0; i < NA; ++i)
#pragma unroll
      for (int c = 0; c < NB; ++c) acc[i][c] = v4f{0.f, 0.f, 0.f, 0.f};
    // K loop: chunk sg of the unit is in LDS buffer (bp + sg) & 1.  The last
    // group loads and stages the queued unit's first chunk.
    UnitSrc<NA, NB, NS, true> nxt;
    if constexpr (!GU) row_ptrs<kThreads, NB, NA, true>(a, row, a.K, nxt);
    // column tiles that hold the group's rows (the others would multiply padding rows)
    const int nbu = __builtin_amdgcn_readfirstlane((g.cnt + 15) / 16);
    for (int sg = 0; sg + 1 < n_sg; ++sg)
      k_group<0, RING, NA, kThreads, NB, false, true>(f, stage, sa, sa_n, cur, sg, nks, n_sg, acc,
                                                      lds + ((bp + sg) & 1) * kBuf, lds + ((bp + sg + 1) & 1) * kBuf,
                                                      cur, sg + 1, nbu);
    const int f0q = fbq * kFeatUnit + wave * kFeatWave;
    {
      const ExpertArgs B = reload_args();
      if constexpr (GU) {
        // the queued unit's token rows, from the perm entries fetched at the top
        const bool sh = gq.e == B.E;
#pragma unroll
        for (int k = 0; k < NR; ++k) row[k] = sh ? group_pair(gq, slot_pos<kThreads, NB>(k)) - B.P : row[k] / B.k;
        row_ptrs<kThreads, NB, NA, true>(B, row, B.K, nxt);
      }
    }
    k_group<0, RING, NA, kThreads, NB, false, true>(f, stage, sa, sa_n, cur, n_sg - 1, nks, n_sg, acc,
                                                    lds + ((bp + n_sg - 1) & 1) * kBuf,
                                                    lds + ((bp + n_sg) & 1) * kBuf, nxt, 0, nbu);
    bp = (bp + n_sg) & 1;
    const ExpertArgs A = reload_args();
    if (tid == 0) s_claim[0] = q >= 0 ? resolve(t, A.pool) : -1;
    __syncthreads();
    const int q2 = s_claim[0];
    // the unit after the queued one: its work-list entry (one dword per lane,
    // lane i % 8 holds word i), first of the loads issued here and read out at
    // the end of the iteration, so that its wait leaves the loads issued after
    // it (the queued unit's weights and chunk, the epilogue's stores) in flight
    const int uq2 = q2 >= 0 ? q2 : uq;
    const int gword = entry_word(A.groups, uq2 / n_fb);
    // the queued unit's scales and first weight steps
    weight_ptrs<NA, GU>(A, gq, f0q, nxt.aq, nxt.as);
    load_wscales(sa, nxt.as, opaque(0));
#pragma unroll
    for (int i = 0; i < RING - 1; ++i) load_w<false>(f[i], nxt.aq, min(opaque(i), nks - 1));
    if constexpr (GU)
      gateup_epilogue_tall<NA / 2>(A, g, f0, acc);
    else
      down_epilogue<NA, NB>(A, g, f0, acc);
    if (q < 0) break;
    u = q;
    g = gq;
    f0 = f0q;
    cur = nxt;
    q = q2;
    uq = uq2;
    gq = unit_group_of(entry_from_words(gword), uq, n_fb, &fbq);
  }
}

template <int NA, int WAVES, bool GU>
static hipError_t tall_launch(const ExpertArgs& a, hipStream_t stream) {
  static std::atomic<uint64_t> attr{0};
  const size_t lds = 2 * (size_t)chunk_buf_bytes<4, true>();
  hipError_t err = ensure_dynamic_lds(tall_kernel<NA, WAVES, GU>, lds, attr);
  if (err != hipSuccess) return err;
  hipLaunchKernelGGL((tall_kernel<NA, WAVES, GU>), dim3(kTallWorkgroups), dim3(64 * WAVES), lds, stream, a);
  return hipGetLastError();
}


// Narrow (16-row) units: the widest unit that divides the output width;
// wider units stage each activation chunk for more weight bytes (less
// activation traffic per weight byte).

// Dynamic LDS of one kernel instantiation: two chunk buffers of NB column
// tiles (above 64 KB the per-device limit is raised on first use).
template <int TPM, int WAVES, int NB, bool NT = false, bool FP6 = false, bool POOL = false, int RING = kRing>
static hipError_t gateup_launch(const ExpertArgs& a, int max_groups, hipStream_t stream) {
  static std::atomic<uint64_t> attr{0};
  const size_t lds = 2 * (size_t)chunk_buf_bytes<NB, FP6>();
  hipError_t err = ensure_dynamic_lds(gateup_kernel<TPM, WAVES, NB, RING, NT, FP6, POOL>, lds, attr);
  if (err != hipSuccess) return err;
  hipLaunchKernelGGL((gateup_kernel<TPM, WAVES, NB, RING, NT, FP6, POOL>), dim3(unit_grid(max_groups, a.R / (16 * TPM * WAVES))),
                     dim3(64 * WAVES), lds, stream, a);
  return hipGetLastError();
}

template <int NA, int WAVES, int NB, bool NT = false, bool FP6 = false, bool POOL = false, int RING = kRing>
static hipError_t down_launch(const ExpertArgs& a, int max_groups, hipStream_t stream) {
  static std::atomic<uint64_t> attr{0};
  const size_t lds = 2 * (size_t)chunk_buf_bytes<NB, FP6>();
  hipError_t err = ensure_dynamic_lds(down_kernel<NA, WAVES, NB, RING, NT, FP6, POOL>, lds, attr);
  if (err != hipSuccess) return err;
  hipLaunchKernelGGL((down_kernel<NA, WAVES, NB, RING, NT, FP6, POOL>), dim3(unit_grid(max_groups, a.R / (16 * NA * WAVES))),
                     dim3(64 * WAVES), lds, stream, a);
  return hipGetLastError();
}

// Small batches (fewer than kWideUnitPairs routed pairs, e.g. 8 rows: about
// one round of units) take the last kSmallTailUnits units of each XCD range in
// halves, which puts twice as many CUs to work; on larger batches halves
// measured slightly slower (more activation staging per weight byte).
constexpr int kSmallTailUnits = 64;

// Work units by the rows of the work list (unit_rows):
//  - 64 (tall, prefill-like): 4 column tiles per unit, so each weight fragment
//    feeds 4x as many MFMAs, on the two-term FP6 activation split (twice the
//    FP8 MFMA rate);
//  - 32 (medium, e.g. 512-row verify batches): 2 column tiles; nearly every
//    expert is one group, so its weights are read once and stream with
//    non-temporal loads;
//  - 16 (small batches): one column tile, non-temporal weight loads and tail
//    halves; 16-row lists of larger batches (widths the wider units do not
//    divide) use the widest unit that fits.
hipError_t launch_gateup(const ExpertArgs& a0, int max_groups, hipStream_t stream) {
  ExpertArgs a = a0;
  a.tail_units = 0;
  if (a.rows == kTallGroupRows) {
    return tall_launch<4, 8, true>(a, stream);
  }
  if (a.rows == kMediumGroupRows) return gateup_launch<2, 8, 2, true, false, true>(a, max_groups, stream);
  if (a.P < kWideUnitPairs) {
    a.tail_units = kSmallTailUnits;
    if (a.R % 256 == 0) return gateup_launch<4, 4, 1, true>(a, max_groups, stream);
    return gateup_launch<2, 4, 1, true>(a, max_groups, stream);
  }
  if (a.R % 512 == 0) return gateup_launch<4, 8, 1>(a, max_groups, stream);
  if (a.R % 256 == 0) return gateup_launch<4, 4, 1>(a, max_groups, stream);
  return gateup_launch<2, 4, 1>(a, max_groups, stream);
}

// (8-wave down units measured slower with 16-row units: those keep 4 waves.)
hipError_t launch_down(const ExpertArgs& a0, int max_groups, hipStream_t stream) {
  ExpertArgs a = a0;
  a.tail_units = 0;
  if (a.rows == kTallGroupRows) {
    return tall_launch<4, 8, false>(a, stream);
  }
  if (a.rows == kMediumGroupRows) return down_launch<4, 8, 2, true, false, true>(a, max_groups, stream);
  if (a.P < kWideUnitPairs) {
    a.tail_units = kSmallTailUnits;
    if (a.R % kDownUnitMax == 0) return down_launch<kDownUnitMax / 64, 4, 1, true>(a, max_groups, stream);
    if (a.R % 256 == 0) return down_launch<4, 4, 1, true>(a, max_groups, stream);
    return down_launch<2, 4, 1, true>(a, max_groups, stream);
  }
  if (a.R % kDownUnitMax == 0) return down_launch<kDownUnitMax / 64, 4, 1>(a, max_groups, stream);
  if (a.R % 256 == 0) return down_launch<4, 4, 1>(a, max_groups, stream);
  return down_launch<2, 4, 1>(a, max_groups, stream);
}

// ---------------------------------------------------------------------------
// out[r] = y_shared[r] + route_scale * sum_j g[r][j] * y[inv[r][j]] (+ residual[r]),
// fp32 in ascending slot order, rounded once to bf16 (nearest even).  y is written
// once by the down GEMM and read once here: both sides use non-temporal
// accesses.

__global__ void __launch_bounds__(256) combine_kernel(const float* __restrict__ y, const int32_t* __restrict__ inv,
                                                       const float* __restrict__ gates, int d, int k, int P,
                                                       int has_shared, float route_scale, const uint16_t* residual,
                                                       uint16_t* out) {
  constexpr int kMaxK = 8;
  const int r = blockIdx.x;
  const float* src[kMaxK];
  float gw[kMaxK];
#pragma unroll
  for (int j = 0; j < kMaxK; ++j) {
    src[j] = (j < k) ? y + (size_t)min(max(inv[(size_t)r * k + j], 0), P - 1) * d : y;  // (clamped into [0, P))
    gw[j] = (j < k) ? gates[(size_t)r * k + j] : 0.f;
  }
  const float* ysh = has_shared ? y + ((size_t)P + r) * d : nullptr;
  // kU chunks of 4 features per thread: all of their loads are issued first
  constexpr int kU = 4;
  const int step = blockDim.x * 4;
  for (int c0 = threadIdx.x * 4; c0 < d; c0 += kU * step) {
    v4f v[kU][kMaxK + 1];
#pragma unroll
    for (int u = 0; u < kU; ++u) {
      const int c = min(c0 + u * step, d - 4);  // past the end: re-read the last chunk (not stored)
#pragma unroll
      for (int j = 0; j < kMaxK; ++j)
        if (j < k) v[u][j] = __builtin_nontemporal_load((const v4f*)(src[j] + c));
      v[u][kMaxK] = ysh ? __builtin_nontemporal_load((const v4f*)(ysh + c)) : v4f{0.f, 0.f, 0.f, 0.f};
    }
#pragma unroll
    for (int u = 0; u < kU; ++u) {
      const int c = c0 + u * step;
      if (c >= d) break;
      v4f acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int j = 0; j < kMaxK; ++j)
        if (j < k) {
#pragma unroll
          for (int i = 0; i < 4; ++i) acc[i] = fmaf(gw[j], v[u][j][i], acc[i]);
        }
      const v4f sh = v[u][kMaxK];
      float o[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) o[i] = fmaf(route_scale, acc[i], sh[i]);
      if (residual) {  // read before the store: residual may be out itself
        const uint2 rb = *(const uint2*)(residual + (size_t)r * d + c);
        o[0] += __uint_as_float(rb.x << 16);
        o[1] += __uint_as_float(rb.x & 0xffff0000u);
        o[2] += __uint_as_float(rb.y << 16);
        o[3] += __uint_as_float(rb.y & 0xffff0000u);
      }
      uint2 packed;
      packed.x = (uint32_t)f32_to_bf16_rne(o[0]) | ((uint32_t)f32_to_bf16_rne(o[1]) << 16);
      packed.y = (uint32_t)f32_to_bf16_rne(o[2]) | ((uint32_t)f32_to_bf16_rne(o[3]) << 16);
      *(uint2*)(out + (size_t)r * d + c) = packed;
    }
  }
}

hipError_t launch_combine(const float* y, const int32_t* inv, const float* gates, int n_rows, int d, int k, int P,
                          int has_shared, float route_scale, const uint16_t* residual, uint16_t* out,
                          hipStream_t stream) {
  hipLaunchKernelGGL(combine_kernel, dim3(n_rows), dim3(256), 0, stream, y, inv, gates, d, k, P, has_shared,
                     route_scale, residual, out);
  return hipGetLastError();
}

}  // namespace moe
