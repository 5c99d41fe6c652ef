// Device helpers shared by the gfx950 attention kernels: vector types, bf16
// conversion, MFMA wrappers, document bounds, the element-wise NeoX rotation
// and the lane layout of the per-row passes.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "kernels.hpp"

namespace neox {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

// bfloat16 bit patterns (low / high half of a dword) to float.
__device__ __forceinline__ float bf2f(uint32_t bits16) { return __uint_as_float(bits16 << 16); }
__device__ __forceinline__ float bf_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// The 16-bit storage element of the matrix kernels.  Their sources are compiled
// once per type: bfloat16 by default, IEEE half when the translation unit
// defines NEOX_ELEM_F16 to 1 before including this header.  elem8 is the MFMA
// operand of 8 elements; el_lo / el_hi / el2f widen to float, pack2 / pack8
// round to nearest even.
#ifndef NEOX_ELEM_F16
#define NEOX_ELEM_F16 0
#endif
#if NEOX_ELEM_F16
typedef f16x8 elem8;
typedef f16x2 elem2;
typedef _Float16 elem1;
__device__ __forceinline__ float el2f(uint32_t bits16) {
  return (float)__builtin_bit_cast(_Float16, (uint16_t)bits16);
}
__device__ __forceinline__ f32x16 mfma32x32x16(elem8 a, elem8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c, 0, 0, 0);
}
#else
typedef bf16x8 elem8;
typedef bf16x2 elem2;
typedef __bf16 elem1;
__device__ __forceinline__ float el2f(uint32_t bits16) { return bf2f(bits16); }
__device__ __forceinline__ f32x16 mfma32x32x16(elem8 a, elem8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}
#endif
// Name of a launcher compiled for the element type (name_bf16 or name_f16), and
// the namespace holding that type's kernels (their symbols differ per type).
#if NEOX_ELEM_F16
#define NEOX_ELEM_FN(name) name##_f16
#define NEOX_ELEM_NS f16
#else
#define NEOX_ELEM_FN(name) name##_bf16
#define NEOX_ELEM_NS bf16
#endif
__device__ __forceinline__ float el_lo(uint32_t w) { return el2f(w & 0xffffu); }
__device__ __forceinline__ float el_hi(uint32_t w) { return el2f(w >> 16); }

// Two floats -> two elements in one dword.
__device__ __forceinline__ uint32_t pack2(float a, float b) {
  elem2 v;
  v[0] = (elem1)a;
  v[1] = (elem1)b;
  return __builtin_bit_cast(uint32_t, v);
}

__device__ __forceinline__ elem8 pack8(const float* x) {
  u32x4 w;
  w[0] = pack2(x[0], x[1]);
  w[1] = pack2(x[2], x[3]);
  w[2] = pack2(x[4], x[5]);
  w[3] = pack2(x[6], x[7]);
  return __builtin_bit_cast(elem8, w);
}

__device__ __forceinline__ elem8 lds_read8(const uint16_t* p) {
  return __builtin_bit_cast(elem8, *reinterpret_cast<const u32x4*>(p));
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// Direct global -> LDS tile loads (16 bytes per lane) through a raw buffer
// resource over a wave-uniform base, with a per-lane byte offset.  The
// compiler's wait-count bookkeeping treats this buffer form as a vector-memory
// load only, whereas it counts the global form against the LDS counter as
// well; with a global-form tile load in flight every LDS operand wait then
// becomes a full lgkmcnt(0), which leaves no LDS read in flight behind a
// matrix product.  Word 3 of the resource selects 32-bit data (the gfx9 raw
// buffer setting); offsets stay below 2^31 (bounded row strides, whole tiles).
typedef __amdgpu_buffer_rsrc_t buf_rsrc;
__device__ __forceinline__ buf_rsrc raw_rsrc(const void* base) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, 0x7fffffff,
                                           0x00020000);
}
__device__ __forceinline__ void dma16(buf_rsrc r, uint32_t byte_off, void* lds_block) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(
      r, (__attribute__((address_space(3))) void*)(reinterpret_cast<uintptr_t>(lds_block)), 16,
      (int)byte_off, 0, 0, 0);
}

// Start and end (exclusive) of the document holding token t of one batch row.
// off[0..n] lists document starts (off[0] = 0, off[n] = S, non-decreasing).
// Results are clamped so that start <= t < end <= S even for malformed rows.
__device__ __forceinline__ void doc_bounds(const int32_t* off, int n, int S, int t, int& start,
                                           int& end) {
  // first idx in [1, n] with off[idx] > t (n if none)
  int lo = 1, hi = n;
  while (lo < hi) {
    int mid = (lo + hi) >> 1;
    if (off[mid] > t) hi = mid; else lo = mid + 1;
  }
  int s = off[lo - 1], e = off[lo];
  s = s < 0 ? 0 : (s > t ? t : s);
  e = e > S ? S : (e <= t ? t + 1 : e);
  start = s;
  end = e;
}

// ALiBi slope of head h in the log2 domain (slope * log2 e).
__device__ __forceinline__ float alibi_slope_log2(const AttnShape& a, int h) {
  float s = a.slopes ? a.slopes[h] : exp2f(-8.0f * (float)(h + 1) / (float)a.H);
  return s * kLog2e;
}

// Rotation of 8 consecutive dims d0..d0+7 of one row (position pos), reading
// each partner element (d +- rd/2) from global memory.  Works for any even rd.
// Every partner and table load is issued (at a valid address: the element
// itself and pair 0 outside the rotary dims) before any is used, with no
// branch in between, so the loads overlap instead of waiting one by one.
// Requires rd > 0 (rope non-null).
__device__ __forceinline__ void rotate8_scalar(const uint16_t* row, int d0, float* x, int pos,
                                               int rd, const float2* rope) {
  const int half = rd >> 1;
  float xp[8];
  float2 cs[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    const int d = d0 + e;
    const bool in = d < rd, first = d < half;
    xp[e] = el2f(row[in ? (first ? d + half : d - half) : d]);
    cs[e] = rope[(int64_t)pos * half + (in ? (first ? d : d - half) : 0)];
  }
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    const int d = d0 + e;
    const float sn = d < half ? -cs[e].y : cs[e].y;
    if (d < rd) x[e] = fmaf(xp[e], sn, x[e] * cs[e].x);
  }
}

// Transpose of the rotate-half rotation for dim d of a row, in integer and bit
// operations only (no compares, so nothing is held in lane masks when a
// caller unrolls many dims): the offset of d's rotary partner (+half below
// half, -half below rd, 0 past rd) and the factors on x_d and on the partner
// (cos and +-sin inside the rotary dims, 1 and 0 past them) given the table
// entry cs of d (any finite value past rd).
__device__ __forceinline__ int rot_partner_step(int d, int half, int rd) {
  const int lt_half = (d - half) >> 31, lt_rd = (d - rd) >> 31;  // -1 when below
  return ((half ^ ~lt_half) - ~lt_half) & lt_rd;
}
// The (cos, sin) table entries of dims d0 .. d0 + 7 (d0 a multiple of 8) from
// the table row `rrow` (half entries): column d mod half for d < rd; dims past
// rd get some valid entry (callers use cos 1, sin 0 there).  With half even a
// pair of dims (d, d + 1), d even, never straddles half and its two entries
// are 16-byte aligned, so four loads suffice; else eight.
__device__ __forceinline__ void rope_entries8(const float2* rrow, int d0, int half, int rd,
                                              float2* cs) {
  if ((half & 1) == 0) {
#pragma unroll
    for (int e2 = 0; e2 < 4; ++e2) {
      const int d = d0 + 2 * e2;
      const int lt_half = (d - half) >> 31, lt_rd = (d - rd) >> 31;  // -1 when below
      const int col = (d - (half & ~lt_half)) & lt_rd;                // 0 past rd
      const f32x4 v = *reinterpret_cast<const f32x4*>(rrow + col);
      cs[2 * e2] = float2{v[0], v[1]};
      cs[2 * e2 + 1] = float2{v[2], v[3]};
    }
  } else {
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const int dc = min(d0 + e, rd - 1);
      cs[e] = rrow[dc - (half & ~((dc - half) >> 31))];
    }
  }
}
__device__ __forceinline__ void rot_t_factors(float2 cs, int d, int half, int rd, float& cn,
                                              float& sn) {
  const uint32_t lt_half = (uint32_t)((d - half) >> 31), lt_rd = (uint32_t)((d - rd) >> 31);
  cn = __uint_as_float((__float_as_uint(cs.x) & lt_rd) | (0x3f800000u & ~lt_rd));
  sn = __uint_as_float((__float_as_uint(cs.y) ^ (0x80000000u & ~lt_half)) & lt_rd);
}

// Workgroup order for kernels that stream one head's K/V (or Q/dO) tiles
// from many workgroups (one per row tile).  Workgroups go to the 8 XCDs
// round-robin (workgroup i on XCD i % 8), each XCD with its own 4 MB L2.
// When B*H is a multiple of 8 every workgroup of head bh runs on XCD bh % 8,
// and each XCD takes its heads in groups small enough that the group's
// streamed tiles (stream_bytes per head) stay L2-resident while all row tiles
// of the group are in flight, heaviest tile first.  Otherwise heads run
// fastest, heaviest tile level first.  Returns (tile, bh); tile 0 is the
// heaviest.
__device__ __forceinline__ void xcd_order(int ntile, int BH, int64_t stream_bytes, int& tile,
                                          int& bh) {
  const int i = (int)blockIdx.x;
  if ((BH & 7) == 0) {
    const int x = i & 7, jj = i >> 3;
    const int hpx = BH >> 3;  // heads per XCD
    int G = (int)(((int64_t)5 << 19) / (stream_bytes > 0 ? stream_bytes : 1));  // 2.5 MB
    G = G < 1 ? 1 : (G > hpx ? hpx : G);
    const int g = jj / (ntile * G);
    const int gs = (hpx - g * G) < G ? hpx - g * G : G;
    const int rem = jj - g * ntile * G;
    tile = rem / gs;
    bh = 8 * (g * G + rem % gs) + x;
  } else {
    tile = i / BH;
    bh = i % BH;
  }
}

// Per-row passes (q/k rotation, backward prep and finalize) give each row a
// group of G lanes, G = D/8 rounded up to a power of two, 16 B per lane, so
// one wave covers 64/G rows and every memory instruction is full width.  Each
// lane issues all of its loads before it uses any, and rotary partners (dims
// +- rd/2, which need not fall on 8-dim chunk boundaries) are exchanged
// through LDS behind an LDS-only wait, so outstanding stores never stall the
// exchange.
template <int D>
struct RowGroups {
  static constexpr int C = D / 8;
  static constexpr int G = C <= 8 ? 8 : 16;
  static constexpr int RPW = 64 / G;  // rows per wave
  static constexpr int RPB = 4 * RPW; // rows per 256-thread workgroup
};

// s_waitcnt immediate (gfx9 encoding): at most n vector memory loads still
// outstanding, all LDS operations done, expcnt not waited on.
constexpr int waitcnt_vm_lgkm0(int n) { return (n & 15) | (7 << 4) | ((n >> 4) << 14); }

// Waits for this wave's LDS operations only (lgkmcnt(0); vmcnt and expcnt
// left at their maxima in the gfx9 s_waitcnt encoding).
__device__ __forceinline__ void lds_wave_sync() {
  __builtin_amdgcn_s_waitcnt(0xC07F);
  __builtin_amdgcn_wave_barrier();
}

}  // namespace neox
