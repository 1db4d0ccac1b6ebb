// Routed experts in Q2_K, the drafter's expert type (TensorSharp "Getting a
// drafter", --expert-type q2_k; the block layout is GGUF's Q2_K): weight
// packing, activation sub-block sums and the grouped gate/up and down GEMMs on
// bf16 MFMA (v_mfma_f32_16x16x32_bf16, fp32 accumulation).
//
// A Q2_K super-block holds 256 values of one weight row: 2-bit quants q, a
// 4-bit scale sc and min mn per 16-value sub-block m, and fp16 factors d and
// dmin; a value is d * sc * q - dmin * mn.  For weight row n and activation
// row r, the dot product over super-block b is
//     d * (T1 - 128 X) - dmin * T2,
//     T1 = sum_t (128 + sc[t/16] q[t]) x[r][t]        8 MFMA k-steps
//     T2 = sum_m mn[m] (xh[r][m] + xl[r][m])           1 MFMA k-step
//     X  = sum_t x[r][t],   xh + xl = the sum of x over sub-block m (bf16 hi/lo)
// 128 + sc * q (at most 173) is an integer, so it is exact in bf16, and it is
// built by byte shuffles alone (a byte p under the high byte 0x43 is the bf16
// number 128 + p); bf16 x times an integer is exact in fp32.  The down GEMM
// runs the same way on fp16 (1024 + sc * q: high byte 0x64) when h is kept in
// fp16: with the swiglu clamp at 0 < L <= 255, |h| <= L^2 < 65504, and fp16
// carries 3 more bits of h than bf16; without such a clamp h stays bf16.
// What rounds: the fp32 sums, xh + xl (16 or 22 bits of each sub-block sum),
// the fold, and h, once, to fp16 or bf16.
//
// A workgroup = one work unit = (group of <= 16*NB rows of one expert, a
// block of output features).  Each wave owns TPM 16-row weight tiles (of gate
// and of up, for gate/up), their per-lane fragments loaded straight from HBM
// into a register ring; the activation rows, their sub-block pairs and X are
// staged once per workgroup through LDS (double-buffered).
// MFMA operands: A = 16 activation rows, B = 16 weight rows; lane (col, g)
// supplies row col, K values 8g..8g+7 of each 32-wide k-step, and holds
// D[activation row 4g+i][weight row col], so each lane's four results share
// one weight row and its d and dmin.
#include "kernels.h"

namespace moe {

typedef __bf16 v8bf __attribute__((ext_vector_type(8)));
typedef _Float16 v8h __attribute__((ext_vector_type(8)));
typedef unsigned short u16x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));

// Packed tile (16 rows x one super-block): [0, 1024) quants, lane l = 16 bytes
// of row l%16 (natural bytes 16+8g..+7 and 48+8g..+7, g = l/16); [1024, 1280)
// the 16 scale/min bytes of each row; [1280, 1344) d and dmin of each row.
constexpr int kQkScales = 1024, kQkFactors = 1280;

// Natural [n_mat][rows][K/256][84] -> packed, one dword per thread.
__global__ void pack_q2k_kernel(const uint8_t* __restrict__ q, size_t n_words, int K, uint8_t* __restrict__ out) {
  const size_t t = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (t >= n_words) return;
  const int nb = K / 256;
  const size_t tile = t / 336;
  const int w = (int)(t % 336);
  const size_t mat_rt = tile / nb;  // matrix * rows/16 + row tile
  const int b = (int)(tile % nb);
  int row, off;
  if (w < 256) {
    const int l = w >> 2, part = w & 3;
    row = l & 15;
    off = (part < 2 ? 16 : 48) + 8 * (l >> 4) + 4 * (part & 1);
  } else if (w < 320) {
    row = (w - 256) >> 2;
    off = 4 * ((w - 256) & 3);
  } else {
    row = w - 320;
    off = 80;
  }
  const uint8_t* src = q + ((mat_rt * 16 + row) * nb + b) * (size_t)kQ2kBlockBytes + off;
  *(uint32_t*)(out + tile * kQ2kTileBytes + 4 * (size_t)w) = *(const uint32_t*)src;
}

hipError_t launch_pack_q2k(const uint8_t* q, int n_mat, int rows, int K, uint8_t* out, hipStream_t stream) {
  const size_t n_words = (size_t)n_mat * (rows / 16) * (K / 256) * 336;
  if (n_words == 0) return hipSuccess;
  hipLaunchKernelGGL(pack_q2k_kernel, dim3((unsigned)((n_words + 255) / 256)), dim3(256), 0, stream, q, n_words, K,
                     out);
  return hipGetLastError();
}

// One thread per (row, 16-value sub-block): the fp32 sum in ascending order,
// stored as hi | lo << 16 in the activations' type: bf16 hi (truncated) and lo
// (the rest, nearest even), or fp16 hi and lo (both nearest even); the 16
// sub-blocks of a super-block are 16 consecutive lanes, whose butterfly sum
// (a fixed order) is X.
__device__ __forceinline__ float qk_lo_value(uint32_t v, bool f16) {
  return f16 ? (float)__builtin_bit_cast(f16x2, v)[0] : __uint_as_float(v << 16);
}
__device__ __forceinline__ float qk_hi_value(uint32_t v, bool f16) {
  return f16 ? (float)__builtin_bit_cast(f16x2, v)[1] : __uint_as_float(v & 0xffff0000u);
}

template <bool F16>
__global__ void q2k_sums_kernel(const uint16_t* __restrict__ act, size_t total, uint32_t* __restrict__ pairs,
                                float* __restrict__ X) {
  const size_t t = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
  float s = 0.f;
  if (t < total) {
    const uint16_t* src = act + t * 16;
    const u32x4 v0 = *(const u32x4*)src, v1 = *(const u32x4*)(src + 8);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      s += qk_lo_value(v0[i], F16);
      s += qk_hi_value(v0[i], F16);
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      s += qk_lo_value(v1[i], F16);
      s += qk_hi_value(v1[i], F16);
    }
  }
  float x = s;
  x += __shfl_xor(x, 1, kWave);
  x += __shfl_xor(x, 2, kWave);
  x += __shfl_xor(x, 4, kWave);
  x += __shfl_xor(x, 8, kWave);
  if (t < total) {
    if constexpr (F16) {
      const _Float16 hi = (_Float16)s, lo = (_Float16)(s - (float)hi);
      pairs[t] = (uint32_t)__builtin_bit_cast(uint16_t, hi) | ((uint32_t)__builtin_bit_cast(uint16_t, lo) << 16);
    } else {
      const uint32_t hi = __float_as_uint(s) & 0xffff0000u;
      pairs[t] = (hi >> 16) | ((uint32_t)f32_to_bf16_rne(s - __uint_as_float(hi)) << 16);
    }
    if ((t & 15) == 0) X[t >> 4] = x;
  }
}

hipError_t launch_q2k_sums(const uint16_t* act, int rows, int K, bool f16, uint32_t* pairs, float* X,
                           hipStream_t stream) {
  const size_t total = (size_t)rows * (K / 16);  // a multiple of 16: whole super-blocks per lane group
  if (total == 0) return hipSuccess;
  const dim3 grid((unsigned)((total + 255) / 256));
  if (f16)
    hipLaunchKernelGGL(q2k_sums_kernel<true>, grid, dim3(256), 0, stream, act, total, pairs, X);
  else
    hipLaunchKernelGGL(q2k_sums_kernel<false>, grid, dim3(256), 0, stream, act, total, pairs, X);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// LDS buffer of one super-block of the unit's 16*NB activation rows: the rows
// (256 bf16 + 16 bytes of padding, so the 16 rows of a fragment read fall in
// distinct banks), their 16 sub-block pairs (+16 bytes) and their X values.
constexpr int kQkXStride = 528, kQkPStride = 80;

template <int NB>
struct QkBuf {
  static constexpr int kRows = 16 * NB;
  static constexpr int kPairs = kRows * kQkXStride;
  static constexpr int kSums = kPairs + kRows * kQkPStride;
  static constexpr int kBytes = kSums + kRows * 4;
};

// This thread's share of one super-block of activations (global -> registers
// -> LDS).  Activation piece p (16 bytes) = row p/32, bytes 16*(p%32); pair
// piece tid < 4*rows = row tid/4, pairs 4*(tid%4)..; X of row tid < rows.
template <int THREADS, int NB>
struct QkStage {
  static constexpr int kRows = 16 * NB;
  static constexpr int kPieces = kRows * 32 / THREADS;
  static_assert(kRows * 32 % THREADS == 0 && 4 * kRows <= THREADS, "staging shape");
  u32x4 x[kPieces];
  u32x4 pr;
  float xs;
};

// Activation rows of this thread's pieces.
template <int THREADS, int NB>
struct QkRows {
  int x[QkStage<THREADS, NB>::kPieces], p, s;
};

// Every thread issues every load (threads past the pair and X pieces read a
// clamped valid row), so the loads of a step are unconditional and the waits
// on the in-order vector-memory counter cover only what is about to be used.
template <int THREADS, int NB>
__device__ __forceinline__ void qk_stage_load(QkStage<THREADS, NB>& st, const QkRows<THREADS, NB>& rows,
                                              const Q2kArgs& a, int b) {
  const int tid = threadIdx.x, nb = a.K / 256;
#pragma unroll
  for (int m = 0; m < QkStage<THREADS, NB>::kPieces; ++m)
    st.x[m] = *(const u32x4*)(a.act + (size_t)rows.x[m] * a.K + 256 * b + 8 * ((tid + THREADS * m) & 31));
  st.pr = *(const u32x4*)(a.pairs + ((size_t)rows.p * nb + b) * 16 + 4 * (tid & 3));
  st.xs = a.X[(size_t)rows.s * nb + b];
}

template <int THREADS, int NB>
__device__ __forceinline__ void qk_stage_store(const QkStage<THREADS, NB>& st, uint8_t* buf) {
  constexpr int kRows = 16 * NB;
  const int tid = threadIdx.x;
#pragma unroll
  for (int m = 0; m < QkStage<THREADS, NB>::kPieces; ++m) {
    const int p = tid + THREADS * m;
    *(u32x4*)(buf + (p >> 5) * kQkXStride + 16 * (p & 31)) = st.x[m];
  }
  if (tid < 4 * kRows) *(u32x4*)(buf + QkBuf<NB>::kPairs + (tid >> 2) * kQkPStride + 16 * (tid & 3)) = st.pr;
  if (tid < kRows) *(float*)(buf + QkBuf<NB>::kSums + 4 * tid) = st.xs;
}

// Per-lane fragments of NA weight tiles for one super-block.
template <int NA>
struct QkW {
  u32x4 qs[NA], sc[NA];
  uint32_t dd[NA];
};

typedef const __attribute__((address_space(1))) uint8_t* qk_gptr;

__device__ __forceinline__ qk_gptr qk_uniform(const uint8_t* p) {
  const uint64_t v = (uint64_t)p;
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)v);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(v >> 32));
  return (qk_gptr)(((uint64_t)hi << 32) | lo);
}

template <int NA>
__device__ __forceinline__ void qk_load_w(QkW<NA>& f, const qk_gptr (&w)[NA], int b) {
  typedef const __attribute__((address_space(1))) u32x4* p4;
  typedef const __attribute__((address_space(1))) uint32_t* p1;
  const int lane = threadIdx.x & 63, col = lane & 15;
  const uint32_t off = (uint32_t)b * kQ2kTileBytes;
#pragma unroll
  for (int i = 0; i < NA; ++i) {
    f.qs[i] = __builtin_nontemporal_load((p4)(w[i] + off + 16 * lane));
    f.sc[i] = *(p4)(w[i] + off + kQkScales + 16 * col);
    f.dd[i] = *(p1)(w[i] + off + kQkFactors + 4 * col);
  }
}

// The MFMA input type: bf16 (magic high byte 0x43: 128 + byte) or fp16
// (0x64: 1024 + byte).
template <bool F16>
struct QkType {
  typedef v8bf vec;
  static constexpr uint32_t kMagic = 0x43434343u;
  static constexpr float kBase = 128.f;
  static __device__ __forceinline__ v4f mfma(const vec& a, const vec& b, const v4f& c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
  }
  static __device__ __forceinline__ uint32_t small_int_bits(uint32_t n) { return __float_as_uint((float)n) >> 16; }
};
template <>
struct QkType<true> {
  typedef v8h vec;
  static constexpr uint32_t kMagic = 0x64646464u;
  static constexpr float kBase = 1024.f;
  static __device__ __forceinline__ v4f mfma(const vec& a, const vec& b, const v4f& c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
  }
  static __device__ __forceinline__ uint32_t small_int_bits(uint32_t n) {
    return __builtin_bit_cast(uint16_t, (_Float16)(float)n);
  }
};

// Pairs base + byte: bytes 0,1 (lo) or 2,3 (hi) of p under the magic high
// byte, one byte permute each (selector bytes 0-3 take p's bytes, 4 takes the
// magic byte: perm(0x43434343, 0xDDCCBBAA, 0x04010400) = 0x43BB43AA).
__device__ __forceinline__ uint32_t qk_pair_lo(uint32_t p, uint32_t magic) {
  return __builtin_amdgcn_perm(magic, p, 0x04010400u);
}
__device__ __forceinline__ uint32_t qk_pair_hi(uint32_t p, uint32_t magic) {
  return __builtin_amdgcn_perm(magic, p, 0x04030402u);
}

// B fragment of k-step S (values 32S + 8g .. +7 of the super-block) as the
// bf16 numbers 128 + sc*q.  Those values sit in half S/4 at bits 2*(S%4) of
// the lane's 8 quant bytes of that half, in sub-block 2S + g/2, whose scale is
// nibble 0 of scale byte 2S + g/2 (gsh = 8*(g/2)).
template <int S, bool F16>
__device__ __forceinline__ typename QkType<F16>::vec qk_frag(const u32x4& qs, const u32x4& sc, uint32_t gsh) {
  constexpr uint32_t M = QkType<F16>::kMagic;
  constexpr int H = S >> 2, J = S & 3;
  const uint32_t scv = __builtin_amdgcn_ubfe(sc[S >> 1], 16 * (S & 1) + gsh, 4);
  const u16x2 m = {(unsigned short)scv, (unsigned short)scv};
  const uint32_t q0 = (qs[2 * H] >> (2 * J)) & 0x03030303u, q1 = (qs[2 * H + 1] >> (2 * J)) & 0x03030303u;
  // sc * q per byte (at most 45, so the two bytes of a 16-bit lane never carry)
  const uint32_t p0 = __builtin_bit_cast(uint32_t, __builtin_bit_cast(u16x2, q0) * m);
  const uint32_t p1 = __builtin_bit_cast(uint32_t, __builtin_bit_cast(u16x2, q1) * m);
  const u32x4 r = {qk_pair_lo(p0, M), qk_pair_hi(p0, M), qk_pair_lo(p1, M), qk_pair_hi(p1, M)};
  return __builtin_bit_cast(typename QkType<F16>::vec, r);
}

// B fragment of the min k-step: k = 2m + t (t = 0 hi, 1 lo) holds mn[m] of
// sub-blocks m = 4g..4g+3 (high nibbles of scale dword g), exact.
template <bool F16>
__device__ __forceinline__ typename QkType<F16>::vec qk_min_frag(const u32x4& sc, int g) {
  // dword g of sc by bit selects (no divergent branches): odd/even, then upper/lower pair
  const uint32_t odd = 0u - (uint32_t)(g & 1), upper = 0u - (uint32_t)(g >> 1);
  const uint32_t lo = (sc[1] & odd) | (sc[0] & ~odd), hi = (sc[3] & odd) | (sc[2] & ~odd);
  const uint32_t sg = (hi & upper) | (lo & ~upper);
  u32x4 r;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const uint32_t b = QkType<F16>::small_int_bits((sg >> (8 * i + 4)) & 15u);
    r[i] = b | (b << 16);
  }
  return __builtin_bit_cast(typename QkType<F16>::vec, r);
}

// One super-block: T1 over 8 k-steps, the fold d * (T1 - 128 X), then T2 and
// the fold - dmin * T2, into acc[tile][row block].
// Where one super-block's activations sit in LDS: row r's 256 values at
// x + r*xs, its 16 sub-block pairs at p + r*ps, the rows' X values at sums
// (4 bytes per row, rows consecutive).
struct QkView {
  const uint8_t *x, *p, *sums;
  int xs, ps;
};

// Row blocks tt >= ntt (all padding rows) are skipped (ntt is uniform).
template <int NA, int NB, bool F16>
__device__ __forceinline__ void qk_superblock(const QkW<NA>& f, const QkView& v, v4f (&acc)[NA][NB], int ntt) {
  typedef QkType<F16> T;
  typedef typename T::vec vec;
  const int lane = threadIdx.x & 63, col = lane & 15, g = lane >> 4;
  const uint32_t gsh = 8 * (g >> 1);
  const v4f zero = {0.f, 0.f, 0.f, 0.f};
  v4f t[NA][NB];
#define QK_STEP(S)                                                                                    \
  {                                                                                                   \
    vec bw[NA];                                                                                       \
    _Pragma("unroll") for (int i = 0; i < NA; ++i) bw[i] = qk_frag<S, F16>(f.qs[i], f.sc[i], gsh);    \
    _Pragma("unroll") for (int tt = 0; tt < NB; ++tt) {                                               \
      if (tt > 0 && tt >= ntt) break;                                                                 \
      const vec av = *(const vec*)(v.x + (16 * tt + col) * v.xs + 64 * (S) + 16 * g);                 \
      _Pragma("unroll") for (int i = 0; i < NA; ++i) t[i][tt] =                                       \
          T::mfma(av, bw[i], (S) == 0 ? zero : t[i][tt]);                                             \
    }                                                                                                 \
  }
  QK_STEP(0)
  QK_STEP(1)
  QK_STEP(2)
  QK_STEP(3)
  QK_STEP(4)
  QK_STEP(5)
  QK_STEP(6)
  QK_STEP(7)
#undef QK_STEP
  v4f xv[NB];
#pragma unroll
  for (int tt = 0; tt < NB; ++tt) xv[tt] = *(const v4f*)(v.sums + 4 * (16 * tt + 4 * g));
  float dmin[NA];
#pragma unroll
  for (int i = 0; i < NA; ++i) {
    const f16x2 dd = __builtin_bit_cast(f16x2, f.dd[i]);
    const float dv = (float)dd[0];
    dmin[i] = (float)dd[1];
#pragma unroll
    for (int tt = 0; tt < NB; ++tt) {
      if (tt > 0 && tt >= ntt) break;
#pragma unroll
      for (int e = 0; e < 4; ++e) acc[i][tt][e] = fmaf(dv, fmaf(-T::kBase, xv[tt][e], t[i][tt][e]), acc[i][tt][e]);
    }
  }
  vec pv[NB];
#pragma unroll
  for (int tt = 0; tt < NB; ++tt)
    pv[tt] = *(const vec*)(v.p + (16 * tt + col) * v.ps + 16 * g);
#pragma unroll
  for (int i = 0; i < NA; ++i) {
    const vec bm = qk_min_frag<F16>(f.sc[i], g);
#pragma unroll
    for (int tt = 0; tt < NB; ++tt) {
      if (tt > 0 && tt >= ntt) break;
      const v4f t2 = T::mfma(pv[tt], bm, zero);
#pragma unroll
      for (int e = 0; e < 4; ++e) acc[i][tt][e] = fmaf(-dmin[i], t2[e], acc[i][tt][e]);
    }
  }
}

// Unit outputs: lane (col, g) holds rows 16tt + 4g + e of features
// f0 + 16i + col.  GU: h = silu(min(gate, L)) * clamp(up, -L, L); else y.
template <int TPM, int NB, bool GU>
__device__ __forceinline__ void qk_epilogue(const Q2kArgs& a, const Group g, int f0,
                                            const v4f (&acc)[GU ? 2 * TPM : TPM][NB]) {
  const int lane = threadIdx.x & 63, col = lane & 15, grp = lane >> 4;
  const float L = a.limit;
#pragma unroll
  for (int i = 0; i < TPM; ++i)
#pragma unroll
    for (int tt = 0; tt < NB; ++tt)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int c = 16 * tt + 4 * grp + e;
        if (c >= g.cnt) continue;
        const size_t o = (size_t)(g.p0 + c) * a.R + f0 + 16 * i + col;
        if constexpr (GU) {
          float gv = acc[i][tt][e], uv = acc[TPM + i][tt][e];
          if (L > 0.f) {
            gv = fminf(gv, L);
            uv = fminf(fmaxf(uv, -L), L);
          }
          const float hv = gv * __builtin_amdgcn_rcpf(1.f + __expf(-gv)) * uv;
          a.h[o] = a.h_f16 ? __builtin_bit_cast(uint16_t, (_Float16)hv) : f32_to_bf16_rne(hv);
        } else {
          a.y[o] = acc[i][tt][e];
        }
      }
}

// One work unit: output features [fu0, fu0 + WAVES*16*TPM) of group g; GU:
// gate and up, written as h (fp16 when a.h_f16, else bf16); else down, on
// fp16 (F16) or bf16 activations h, written as y.
template <int TPM, int WAVES, int NB, int RING, bool GU, bool F16>
__device__ __forceinline__ void qk_unit(const Q2kArgs& a, const Group g, int fu0, uint8_t* lds) {
  constexpr int NA = GU ? 2 * TPM : TPM, kThreads = 64 * WAVES, kRows = 16 * NB;
  constexpr int kBuf = QkBuf<NB>::kBytes;
  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int K = a.K, R = a.R, nb = K / 256;
  const int f0 = fu0 + wave * 16 * TPM;
  const size_t mat = q2k_matrix_bytes(R, K), tile = (size_t)nb * kQ2kTileBytes;
  qk_gptr w[NA];
#pragma unroll
  for (int i = 0; i < TPM; ++i) {
    w[i] = qk_uniform(a.w0 + (size_t)g.e * mat + (size_t)(f0 / 16 + i) * tile);
    if constexpr (GU) w[TPM + i] = qk_uniform(a.w1 + (size_t)g.e * mat + (size_t)(f0 / 16 + i) * tile);
  }
  // activation row of unit row c (padding rows repeat the group's first row)
  auto act_row = [&](int c) -> int {
    const int p = g.p0 + (c < g.cnt ? c : 0);
    return GU ? min(max(a.perm[p], 0), a.P - 1) / a.k : p;  // (perm entries clamped into [0, P))
  };
  QkRows<kThreads, NB> rows;
#pragma unroll
  for (int m = 0; m < QkStage<kThreads, NB>::kPieces; ++m) rows.x[m] = act_row((tid + kThreads * m) >> 5);
  rows.p = act_row(min(tid >> 2, kRows - 1));
  rows.s = act_row(min(tid, kRows - 1));

  v4f acc[NA][NB];
#pragma unroll
  for (int i = 0; i < NA; ++i)
#pragma unroll
    for (int tt = 0; tt < NB; ++tt) acc[i][tt] = v4f{0.f, 0.f, 0.f, 0.f};
  const int ntt = (g.cnt + 15) / 16;
  // Weights: a ring of RING super-blocks (RING-1 in flight while one is
  // multiplied).  Activations: one register set; super-block b+1 (loaded at
  // the end of step b-1) is stored to the other LDS buffer at the end of step
  // b, then b+2 is loaded, then the barrier.  Loads past the last super-block
  // repeat the last one (clamped, never used), so every step issues the same
  // loads in the same order (kept by the scheduling barriers) and each wait on
  // the in-order vector-memory counter covers only the data about to be used.
  // The loop is unrolled RING steps so every register index is a constant.
  const int last = nb - 1;
  QkW<NA> f[RING];
  QkStage<kThreads, NB> st;
#pragma unroll
  for (int r = 0; r < RING - 1; ++r) qk_load_w(f[r], w, min(r, last));
  qk_stage_load(st, rows, a, 0);
  qk_stage_store(st, lds);
  qk_stage_load(st, rows, a, min(1, last));
  __syncthreads();
  for (int b0 = 0; b0 < nb; b0 += RING) {
#pragma unroll
    for (int r = 0; r < RING; ++r) {
      const int b = b0 + r;
      if (b >= nb) break;
      __builtin_amdgcn_sched_barrier(0);
      qk_load_w(f[(r + RING - 1) % RING], w, min(b + RING - 1, last));
      __builtin_amdgcn_sched_barrier(0);
      const uint8_t* buf = lds + (b & 1) * kBuf;
      qk_superblock<NA, NB, F16>(f[r], QkView{buf, buf + QkBuf<NB>::kPairs, buf + QkBuf<NB>::kSums, kQkXStride,
                                               kQkPStride}, acc, ntt);
      __builtin_amdgcn_sched_barrier(0);
      qk_stage_store(st, lds + ((b + 1) & 1) * kBuf);
      qk_stage_load(st, rows, a, min(b + 2, last));
      __syncthreads();
    }
  }

  qk_epilogue<TPM, NB, GU>(a, g, f0, acc);
}

// LDS of a unit whose 16 activation rows stay resident for the whole
// contraction K: rows (2K bytes + 16 of padding, so that the 16 rows of a
// fragment read fall in distinct banks), their pairs (K/4 + 16 bytes) and X
// ([K/256][16] floats).
__host__ __device__ inline int qk_res_xs(int K) { return 2 * K + 16; }
__host__ __device__ inline int qk_res_ps(int K) { return K / 4 + 16; }

// One work unit of a group of <= 16 rows with its activations resident in
// LDS: all of the group's rows, pairs and X are staged once, then the
// super-blocks are multiplied with no barrier, the weight ring RING-1 deep.
template <int TPM, int WAVES, int RING, bool GU, bool F16>
__device__ __forceinline__ void qk_unit_resident(const Q2kArgs& a, const Group g, int fu0, uint8_t* lds) {
  constexpr int NA = GU ? 2 * TPM : TPM, kThreads = 64 * WAVES;
  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int K = a.K, R = a.R, nb = K / 256, last = nb - 1;
  const int xs = qk_res_xs(K), ps = qk_res_ps(K);
  uint8_t* lds_p = lds + 16 * (size_t)xs;
  uint8_t* lds_s = lds_p + 16 * (size_t)ps;
  const int f0 = fu0 + wave * 16 * TPM;
  const size_t mat = q2k_matrix_bytes(R, K), tile = (size_t)nb * kQ2kTileBytes;
  qk_gptr w[NA];
#pragma unroll
  for (int i = 0; i < TPM; ++i) {
    w[i] = qk_uniform(a.w0 + (size_t)g.e * mat + (size_t)(f0 / 16 + i) * tile);
    if constexpr (GU) w[TPM + i] = qk_uniform(a.w1 + (size_t)g.e * mat + (size_t)(f0 / 16 + i) * tile);
  }
  QkW<NA> f[RING];
#pragma unroll
  for (int r = 0; r < RING - 1; ++r) qk_load_w(f[r], w, min(r, last));
  // the group's rows (padding rows repeat its first row): 16-byte pieces,
  // K/8 per row, then 16-byte pair pieces, K/64 per row, then X
  auto act_row = [&](int c) -> size_t {
    const int p = g.p0 + (c < g.cnt ? c : 0);
    return (size_t)(GU ? min(max(a.perm[p], 0), a.P - 1) / a.k : p);  // (perm entries clamped into [0, P))
  };
  const int xpr = K / 8, ppr = K / 64;
  for (int q = tid; q < 16 * xpr; q += kThreads) {
    const int c = q / xpr, j = q % xpr;
    *(u32x4*)(lds + c * xs + 16 * j) = *(const u32x4*)(a.act + act_row(c) * K + 8 * j);
  }
  for (int q = tid; q < 16 * ppr; q += kThreads) {
    const int c = q / ppr, j = q % ppr;
    *(u32x4*)(lds_p + c * ps + 16 * j) = *(const u32x4*)(a.pairs + act_row(c) * (K / 16) + 4 * j);
  }
  for (int q = tid; q < 16 * nb; q += kThreads) {
    const int c = q & 15, b = q >> 4;
    *(float*)(lds_s + 4 * q) = a.X[act_row(c) * nb + b];
  }
  __syncthreads();
  v4f acc[NA][1];
#pragma unroll
  for (int i = 0; i < NA; ++i) acc[i][0] = v4f{0.f, 0.f, 0.f, 0.f};
  for (int b0 = 0; b0 < nb; b0 += RING) {
#pragma unroll
    for (int r = 0; r < RING; ++r) {
      const int b = b0 + r;
      if (b >= nb) break;
      __builtin_amdgcn_sched_barrier(0);
      qk_load_w(f[(r + RING - 1) % RING], w, min(b + RING - 1, last));
      __builtin_amdgcn_sched_barrier(0);
      qk_superblock<NA, 1, F16>(f[r], QkView{lds + 512 * b, lds_p + 64 * b, lds_s + 64 * b, xs, ps}, acc, 1);
    }
  }
  qk_epilogue<TPM, 1, GU>(a, g, f0, acc);
}

// Units dealt by xcd_unit_claim; tall units feature-block-major (unit_group).
template <int TPM, int WAVES, int NB, int RING, bool GU, bool F16>
__global__ void __launch_bounds__(64 * WAVES) q2k_kernel(Q2kArgs a) {
  constexpr int kFeatUnit = WAVES * 16 * TPM;
  extern __shared__ __attribute__((aligned(16))) uint8_t lds[];  // 2 * QkBuf<NB>::kBytes
  const int n_fb = a.R / kFeatUnit;
  __shared__ int s_claim;
  const int half_idx = xcd_unit_claim(*a.n_groups * n_fb, a.pool, &s_claim);
  if (half_idx < 0) return;
  int fb;
  const Group g = unit_group<NB == 4>(a.groups, half_idx >> 1, n_fb, &fb);
  qk_unit<TPM, WAVES, NB, RING, GU, F16>(a, g, fb * kFeatUnit, lds);
}

// 16-row groups with resident activations, dealt feature-block-major within
// an expert (an expert's groups of one feature block run side by side, so
// its weights come from HBM once and from L2 for the other groups).
template <int TPM, int WAVES, int RING, bool GU, bool F16>
__global__ void __launch_bounds__(64 * WAVES) q2k_res_kernel(Q2kArgs a) {
  constexpr int kFeatUnit = WAVES * 16 * TPM;
  extern __shared__ __attribute__((aligned(16))) uint8_t lds[];  // q2k_resident_lds_bytes(K)
  const int n_fb = a.R / kFeatUnit;
  __shared__ int s_claim;
  const int half_idx = xcd_unit_claim(*a.n_groups * n_fb, a.pool, &s_claim);
  if (half_idx < 0) return;
  int fb;
  const Group g = unit_group<true>(a.groups, half_idx >> 1, n_fb, &fb);
  qk_unit_resident<TPM, WAVES, RING, GU, F16>(a, g, fb * kFeatUnit, lds);
}

template <int TPM, int WAVES, int RING, bool GU, bool F16 = false>
static hipError_t q2k_res_launch(const Q2kArgs& a, int max_groups, hipStream_t stream) {
  static std::atomic<uint64_t> attr{0};
  constexpr int kFeatUnit = WAVES * 16 * TPM;
  if (a.R % kFeatUnit || a.K % 256) return hipErrorInvalidValue;
  const size_t lds = q2k_resident_lds_bytes(a.K);
  if (lds > kQ2kResidentMaxLds) return hipErrorInvalidValue;
  hipError_t err = ensure_dynamic_lds(q2k_res_kernel<TPM, WAVES, RING, GU, F16>, kQ2kResidentMaxLds, attr);
  if (err != hipSuccess) return err;
  hipLaunchKernelGGL((q2k_res_kernel<TPM, WAVES, RING, GU, F16>), dim3(unit_grid(max_groups, a.R / kFeatUnit)),
                     dim3(64 * WAVES), lds, stream, a);
  return hipGetLastError();
}

template <int TPM, int WAVES, int NB, int RING, bool GU, bool F16 = false>
static hipError_t q2k_launch(const Q2kArgs& a, int max_groups, hipStream_t stream) {
  static std::atomic<uint64_t> attr{0};
  constexpr int kFeatUnit = WAVES * 16 * TPM;
  if (a.R % kFeatUnit || a.K % 256) return hipErrorInvalidValue;
  const size_t lds = 2 * (size_t)QkBuf<NB>::kBytes;
  hipError_t err = ensure_dynamic_lds(q2k_kernel<TPM, WAVES, NB, RING, GU, F16>, lds, attr);
  if (err != hipSuccess) return err;
  hipLaunchKernelGGL((q2k_kernel<TPM, WAVES, NB, RING, GU, F16>), dim3(unit_grid(max_groups, a.R / kFeatUnit)),
                     dim3(64 * WAVES), lds, stream, a);
  return hipGetLastError();
}

// Launch shapes (TPM tiles per wave and matrix, waves, 16-row column tiles,
// weight ring depth) per group size; 16-row groups keep their activations
// resident (TPM, waves, ring depth).
#define QK_GU_TALL 1, 8, 4, 2
#define QK_GU_MED 1, 8, 2, 3
#define QK_GU_SMALL 1, 8, 1, 2
#define QK_GU_RES 2, 8, 3
#define QK_DN_TALL 2, 8, 4, 2
#define QK_DN_MED 1, 8, 2, 2
#define QK_DN_SMALL 1, 8, 1, 2
#define QK_DN_RES 2, 8, 3

template <bool F16>
static hipError_t q2k_down_launch(const Q2kArgs& a, int max_groups, hipStream_t stream) {
  if (a.rows == kTallGroupRows) return q2k_launch<QK_DN_TALL, false, F16>(a, max_groups, stream);
  if (a.rows == kMediumGroupRows) return q2k_launch<QK_DN_MED, false, F16>(a, max_groups, stream);
  if (q2k_resident_lds_bytes(a.K) <= kQ2kResidentMaxLds)
    return q2k_res_launch<QK_DN_RES, false, F16>(a, max_groups, stream);
  return q2k_launch<QK_DN_SMALL, false, F16>(a, max_groups, stream);
}

hipError_t launch_q2k_gateup(const Q2kArgs& a, int max_groups, hipStream_t stream) {
  if (a.rows == kTallGroupRows) return q2k_launch<QK_GU_TALL, true>(a, max_groups, stream);
  if (a.rows == kMediumGroupRows) return q2k_launch<QK_GU_MED, true>(a, max_groups, stream);
  if (q2k_resident_lds_bytes(a.K) <= kQ2kResidentMaxLds)
    return q2k_res_launch<QK_GU_RES, true, false>(a, max_groups, stream);
  return q2k_launch<QK_GU_SMALL, true>(a, max_groups, stream);
}

hipError_t launch_q2k_down(const Q2kArgs& a, int max_groups, hipStream_t stream) {
  return a.h_f16 ? q2k_down_launch<true>(a, max_groups, stream) : q2k_down_launch<false>(a, max_groups, stream);
}

}  // namespace moe
