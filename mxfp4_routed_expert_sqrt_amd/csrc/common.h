// Device helpers shared by the gfx950 kernels of the routed MoE layer.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace moe {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr int kWave = 64;
constexpr int kGroupRows = 16;       // token rows of a narrow work unit (one MFMA column tile)
constexpr int kMediumGroupRows = 32;  // token rows of a medium work unit (2 column tiles)
constexpr int kTallGroupRows = 64;    // token rows of a tall work unit (4 column tiles)
constexpr int kXcds = 8;         // gfx950: workgroups are dealt round-robin to 8 XCDs

// One work group of the grouped GEMMs: rows [p0, p0 + cnt) of expert e; the
// expert's groups are entries [first, first + ng) of the work list and cut its
// segment of seg_rows rows from seg_p0 into pieces of `rows`, so any one entry
// describes all of them.
struct Group {
  int32_t e, p0, cnt, first, ng, seg_rows, seg_p0, rows;
};

// Maps this workgroup to a work unit so that each XCD receives a contiguous
// range of units (units of one group share activations in that XCD's L2),
// counted in half units: each XCD's range is taken whole, except its last
// `tail_units`, which are taken one half at a time (two workgroups each).
// Returns false for workgroups beyond the device-side unit count.
// Sets *half_idx = 2*unit + half (half = 0 for a whole unit) and *is_half.
__device__ __forceinline__ bool xcd_unit_split(int n_units, int tail_units, int* half_idx, bool* is_half) {
  const int bid = blockIdx.x;
  const int xcd = bid % kXcds, slot = bid / kXcds;
  const int H = 2 * n_units;
  int per = (H + kXcds - 1) / kXcds;
  per += per & 1;  // whole units never straddle two XCDs
  const int h0 = xcd * per;
  const int hx = min(per, max(0, H - h0));
  const int tail = min(hx, 2 * tail_units);
  const int n_whole = (hx - tail) / 2;
  if (slot < n_whole) {
    *half_idx = h0 + 2 * slot;
    *is_half = false;
    return true;
  }
  if (slot < n_whole + tail) {
    *half_idx = h0 + 2 * n_whole + (slot - n_whole);
    *is_half = true;
    return true;
  }
  return false;
}

// Units per XCD range that are dealt dynamically by xcd_unit_claim.
constexpr int kPoolUnits = 16;

// The pool part of xcd_unit_claim, by one thread: claims the next unit of the
// shared pool of the eight XCD ranges' last kPoolUnits units.  Returns the
// half index (2 * unit) or -1 when the pool is used up.
__device__ __forceinline__ int pool_claim_one(int n_units, int32_t* ctr) {
  const int H = 2 * n_units;
  int per = (H + kXcds - 1) / kXcds;
  per += per & 1;
  constexpr int kPool = kXcds * kPoolUnits;
  __attribute__((address_space(1))) int32_t* gctr = (__attribute__((address_space(1))) int32_t*)ctr;
  while (__hip_atomic_load(gctr, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) < kPool) {
    const int u = __hip_atomic_fetch_add(gctr, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    if (u >= kPool) break;
    const int x = u % kXcds, t = u / kXcds;
    const int n = min(per, max(0, H - x * per)) / 2;
    const int tn = min(kPoolUnits, n);
    if (t < tn) return x * per + 2 * (n - tn + t);
  }
  return -1;
}

// pool_claim_one for the workgroup: every thread must call it.
__device__ __forceinline__ int pool_claim(int n_units, int32_t* ctr, int* s_claim) {
  if (threadIdx.x == 0) *s_claim = pool_claim_one(n_units, ctr);
  __syncthreads();
  return *s_claim;
}

// Dealing with a shared tail: XCD x's range (as in xcd_unit_split, whole
// units) is taken statically in slot order except for its last kPoolUnits
// units.  Those tails of all eight ranges form one pool, ordered tail unit 0
// of XCD 0..7, then tail unit 1, ...; a workgroup past its XCD's static part
// claims the next pool entry with an atomic on *ctr (zeroed before the
// launch), so XCDs that run faster take over the end of slower ones' ranges.
// The claim loop ends once the counter passes the pool size.  Returns the
// half index (2 * unit) or -1 when nothing is left; s_claim is a
// workgroup-shared int.  Every thread of the workgroup must call it.
__device__ __forceinline__ int xcd_unit_claim(int n_units, int32_t* ctr, int* s_claim) {
  const int bid = blockIdx.x, xcd = bid % kXcds, slot = bid / kXcds;
  const int H = 2 * n_units;
  int per = (H + kXcds - 1) / kXcds;
  per += per & 1;
  const int nx = min(per, max(0, H - xcd * per)) / 2;
  const int tx = min(kPoolUnits, nx);
  if (slot < nx - tx) return xcd * per + 2 * slot;
  return pool_claim(n_units, ctr, s_claim);
}

// Work group and feature block of unit `unit`.  Units run through the work
// list expert by expert.  Group-major (FBMAJOR false): the n_fb feature blocks
// of one group are consecutive, so they share that group's activations in L2.
// Feature-block-major (the tall units): within an expert, the expert's ng
// groups of one feature block are consecutive, so they share that block's
// weights in L2 while they run side by side on one XCD (at 8192 rows this
// took the gate/up weight fetch from 6.31 to 3.68 GB per launch and down from
// 2.41 to 1.69 GB).
// A work-list entry, read as a global load however the pointer was obtained.
__device__ __forceinline__ Group load_group(const Group* p) {
  typedef const __attribute__((address_space(1))) int32_t* gw;
  const gw w = (gw)p;
  Group g;
  g.e = w[0], g.p0 = w[1], g.cnt = w[2], g.first = w[3];
  g.ng = w[4], g.seg_rows = w[5], g.seg_p0 = w[6], g.rows = w[7];
  return g;
}

// Group j of the expert of g (the work-list entry g.first + j), from g alone.
__device__ __forceinline__ Group group_piece(Group g, int j) {
  g.p0 = g.seg_p0 + j * g.rows;
  g.cnt = min(g.rows, g.seg_rows - j * g.rows);
  return g;
}

// Feature-block-major: group and feature block of unit `unit`, given the
// work-list entry unit / n_fb.
__device__ __forceinline__ Group unit_group_of(const Group& g, int unit, int n_fb, int* fb) {
  const int l = unit - g.first * n_fb, j = l % g.ng;
  *fb = l / g.ng;
  return group_piece(g, j);
}

template <bool FBMAJOR>
__device__ __forceinline__ Group unit_group(const Group* groups, int unit, int n_fb, int* fb) {
  const Group g = load_group(groups + unit / n_fb);
  if constexpr (!FBMAJOR) {
    *fb = unit % n_fb;
    return g;
  } else {
    return unit_group_of(g, unit, n_fb, fb);
  }
}

__device__ __forceinline__ float bf16_to_f32(uint16_t b) { return __uint_as_float((uint32_t)b << 16); }

__device__ __forceinline__ uint16_t f32_to_bf16_rne(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return (uint16_t)((u >> 16) | 0x40);  // quiet NaN
  u += 0x7fffu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

// Shared exponent for a two-term FP8 (E4M3) split of a block whose largest
// magnitude is amax: amax / 2^e lands in [128, 256), inside E4M3's normal range
// (max 448), so no element saturates.  Clamped to the E8M0 range.
__device__ __forceinline__ int split_exponent(float amax) {
  if (!(amax > 0.f)) return 0;
  int ex;
  frexpf(amax, &ex);  // amax = m * 2^ex, m in [0.5, 1)
  int e = ex - 1 - 7;
  e = e < -127 ? -127 : e;
  e = e > 127 ? 127 : e;
  return e;
}

// 4 floats -> 4 E4M3 bytes (round to nearest even), packed little-endian.
__device__ __forceinline__ uint32_t pack4_fp8(float a, float b, float c, float d) {
  int v = __builtin_amdgcn_cvt_pk_fp8_f32(a, b, 0, false);
  v = __builtin_amdgcn_cvt_pk_fp8_f32(c, d, v, true);
  return (uint32_t)v;
}

__device__ __forceinline__ float fp8_byte_to_f32(uint32_t word, int byte) {
  switch (byte) {
    case 0: return __builtin_amdgcn_cvt_f32_fp8((int)word, 0);
    case 1: return __builtin_amdgcn_cvt_f32_fp8((int)word, 1);
    case 2: return __builtin_amdgcn_cvt_f32_fp8((int)word, 2);
    default: return __builtin_amdgcn_cvt_f32_fp8((int)word, 3);
  }
}

// ---------------------------------------------------------------------------
// FP6 E2M3: sign, 2 exponent bits (bias 1), 3 mantissa bits; subnormals m/8,
// normals 2^(e-1) * (1 + m/8), largest 7.5.  The scaled MFMA's 6-bit operand
// holds K values 32*(l/16)..+31 of lane l as a little-endian bitstream over
// the lane's first 6 dwords, value i at bits 6i..6i+5 (measured on gfx950;
// the probe test pins it).

// Shared exponent of a block whose largest magnitude is amax, so that
// amax / 2^e <= 7.5 (inside E2M3, no saturation); clamped to the E8M0 range.
__device__ __forceinline__ int fp6_exponent(float amax) {
  if (!(amax > 0.f)) return 0;
  int ex;
  frexpf(amax, &ex);  // amax in [2^(ex-1), 2^ex): amax / 2^(ex-3) in [4, 8)
  int e = ex - 3;
  if (amax > ldexpf(7.5f, e)) ++e;
  e = e < -127 ? -127 : e;
  e = e > 127 ? 127 : e;
  return e;
}

typedef float v16f __attribute__((ext_vector_type(16)));
typedef float v32f __attribute__((ext_vector_type(32)));
typedef uint32_t u32x6 __attribute__((ext_vector_type(6)));

// gfx950's FP6 conversions of one 32-value block at a power-of-two scale.
// fp6_pack32: code j = E2M3 of v_j / scale, rounded to nearest with ties to
// the even code and saturating at 7.5 (measured on the instruction over a
// sweep of [-16, 16] at scales 1/2, 1 and 2: every code was the
// round-to-nearest-even one); position j takes ev[j / 2] for even j and
// od[j / 2] for odd j, value j at bits 6j of the 6 result dwords (the scaled
// MFMA's 6-bit operand).  The result is marked early-clobber: the
// instruction writes its destination before it has read all 32 source
// registers, so the two must not overlap (a destination placed over the last
// two source registers converted stale values).
__device__ __forceinline__ u32x6 fp6_pack32(const v16f& ev, const v16f& od, float scale) {
  u32x6 r;
  asm("v_cvt_scalef32_2xpk16_fp6_f32 %0, %1, %2, %3" : "=&v"(r) : "v"(ev), "v"(od), "v"(scale));
  return r;
}

// fp6_unpack32: the value of code j times scale, in element j (exact).
__device__ __forceinline__ v32f fp6_unpack32(const u32x6& codes, float scale) {
  v32f d;
  asm("v_cvt_scalef32_pk32_f32_fp6 %0, %1, %2" : "=&v"(d) : "v"(codes), "v"(scale));
  return d;
}

// Two-term E2M3 split of one 32-value block (values at even positions in ev,
// odd in od): term 1 = fp6_pack32 at scale 2^e1 with the block maximum inside
// E2M3's range, term 2 = the exact residual v - term 1, split the same way.
// The exponents are clamped below at -126, so each scale is a normal fp32.
// On return ev/od hold the residuals.
__device__ __forceinline__ void split_fp6_32(v16f& ev, v16f& od, u32x6* t1, u32x6* t2, int* e1, int* e2) {
  float amax = 0.f;
#pragma unroll
  for (int i = 0; i < 16; ++i) amax = fmaxf(amax, fmaxf(fabsf(ev[i]), fabsf(od[i])));
  *e1 = max(fp6_exponent(amax), -126);
  const float s1 = ldexpf(1.f, *e1);
  *t1 = fp6_pack32(ev, od, s1);
  const v32f d1 = fp6_unpack32(*t1, s1);
  float amax2 = 0.f;
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    ev[i] -= d1[2 * i];
    od[i] -= d1[2 * i + 1];
    amax2 = fmaxf(amax2, fmaxf(fabsf(ev[i]), fabsf(od[i])));
  }
  *e2 = max(fp6_exponent(amax2), -126);
  *t2 = fp6_pack32(ev, od, ldexpf(1.f, *e2));
}

// Swaps of 32-bit values between lane groups of 16 ("rows"), gfx950's
// permlane swaps: after swap32, rows 2-3 of x and rows 0-1 of y are
// exchanged; after swap16, rows 1 and 3 of x and rows 0 and 2 of y.
__device__ __forceinline__ void swap32(float& x, float& y) {
  const auto s = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(y), false, false);
  x = __uint_as_float(s[0]);
  y = __uint_as_float(s[1]);
}
__device__ __forceinline__ void swap16(float& x, float& y) {
  const auto s = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(y), false, false);
  x = __uint_as_float(s[0]);
  y = __uint_as_float(s[1]);
}

template <int kOff>
__device__ __forceinline__ float shfl_xor_max(float v) {
  return fmaxf(v, __shfl_xor(v, kOff, kWave));
}

}  // namespace moe
