// Device helpers shared by the gfx950 attention kernels: vector types, bf16
// conversion, MFMA wrappers, document bounds, and the tile loaders that apply
// the NeoX rotary rotation while staging rows into LDS.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "kernels.hpp"

namespace neox {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

__device__ __forceinline__ float bf2f(uint32_t bits16) { return __uint_as_float(bits16 << 16); }
__device__ __forceinline__ float bf_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// Two floats -> two bf16 (round to nearest even, v_cvt_pk_bf16_f32) in one dword.
__device__ __forceinline__ uint32_t pack2(float a, float b) {
  bf16x2 v;
  v[0] = (__bf16)a;
  v[1] = (__bf16)b;
  return __builtin_bit_cast(uint32_t, v);
}

__device__ __forceinline__ bf16x8 pack8(const float* x) {
  u32x4 w;
  w[0] = pack2(x[0], x[1]);
  w[1] = pack2(x[2], x[3]);
  w[2] = pack2(x[4], x[5]);
  w[3] = pack2(x[6], x[7]);
  return __builtin_bit_cast(bf16x8, w);
}

__device__ __forceinline__ f32x16 mfma32x32x16(bf16x8 a, bf16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ bf16x8 lds_read8(const uint16_t* p) {
  return __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(p));
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

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
__device__ __forceinline__ void rotate8_scalar(const uint16_t* row, int d0, float* x, int pos,
                                               int rd, const float2* rope) {
  const int half = rd >> 1;
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    const int d = d0 + e;
    if (d < rd) {
      const bool first = d < half;
      const int p = first ? d : d - half;
      const float xp = bf2f(row[first ? d + half : d - half]);
      const float2 cs = rope[(int64_t)pos * half + p];
      x[e] = first ? (x[e] * cs.x - xp * cs.y) : (x[e] * cs.x + xp * cs.y);
    }
  }
}

// Column of tile row `r` (a multiple of 4) in a transposed LDS tile.  With
// PERM, rows are reordered inside each group of 16 as [0-3][8-11][4-7][12-15]
// so that an MFMA accumulator column (rows (r/4)*8 + 4*half + r%4) can feed
// the next MFMA's B operand (8 consecutive k per lane) without a shuffle.
template <bool PERM>
__device__ __forceinline__ int tcol(int r) {
  if (!PERM) return r;
  const int g = (r >> 2) & 3;
  const int pg = (g == 1) ? 2 : (g == 2 ? 1 : g);
  return (r & ~15) + 4 * pg;
}

// Stages rows [r0, r0 + R) of one head's [S, D] bf16 matrix (row stride ss
// elements) into LDS.  With ROT == 1 (rd % 8 == 0) or ROT == 2 (any even rd)
// the first rd dims are rotated by the rotary angle of each row's position;
// ROT == 0 copies.  Rows at or beyond S are stored as zeros.  ROWMAJOR writes
// dst_row[row * RS + dim]; TRANS writes dst_t[dim * TS + tcol<PERM>(row)].
// Work items are (group of 4 rows, slot of 8 dims); for ROT == 1 the first
// rd/8 slots are "pair slots" holding dims p0..p0+3 and half+p0..half+p0+3.
template <int D, int ROT, int R, int NT, bool ROWMAJOR, bool TRANS, bool PERM>
__device__ __forceinline__ void load_tile(const uint16_t* __restrict__ base, int64_t ss, int r0,
                                          int S, int rd, const float2* __restrict__ rope,
                                          uint16_t* dst_row, int RS, uint16_t* dst_t, int TS,
                                          int tid) {
  constexpr int NSLOT = D / 8;
  constexpr int NITEM = (R / 4) * NSLOT;
  const int half = rd >> 1;
  const int npair = (ROT == 1) ? (rd >> 3) : 0;
#pragma unroll
  for (int it0 = 0; it0 < NITEM; it0 += NT) {
    const int it = it0 + tid;
    if (NITEM % NT != 0 && it >= NITEM) break;
    const int slot = it % NSLOT;
    const int g = it / NSLOT;
    const bool pair = slot < npair;
    const int p0 = slot * 4;  // pair slot: first-half dims p0..p0+3
    const int d0 = slot * 8;  // plain slot: dims d0..d0+7
    float x[4][8];
#pragma unroll
    for (int rr = 0; rr < 4; ++rr) {
      const int row = r0 + 4 * g + rr;
      if (row < S) {
        const uint16_t* src = base + (int64_t)row * ss;
        if (pair) {
          const u32x2 a = *reinterpret_cast<const u32x2*>(src + p0);
          const u32x2 b = *reinterpret_cast<const u32x2*>(src + half + p0);
          const float x1[4] = {bf_lo(a[0]), bf_hi(a[0]), bf_lo(a[1]), bf_hi(a[1])};
          const float x2[4] = {bf_lo(b[0]), bf_hi(b[0]), bf_lo(b[1]), bf_hi(b[1])};
          const f32x4* cs4 = reinterpret_cast<const f32x4*>(rope + (int64_t)row * half + p0);
          const f32x4 c01 = cs4[0], c23 = cs4[1];
          const float cs[4] = {c01[0], c01[2], c23[0], c23[2]};
          const float sn[4] = {c01[1], c01[3], c23[1], c23[3]};
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            x[rr][e] = x1[e] * cs[e] - x2[e] * sn[e];
            x[rr][4 + e] = x2[e] * cs[e] + x1[e] * sn[e];
          }
        } else {
          const u32x4 w = *reinterpret_cast<const u32x4*>(src + d0);
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            x[rr][2 * e] = bf_lo(w[e]);
            x[rr][2 * e + 1] = bf_hi(w[e]);
          }
          if (ROT == 2) rotate8_scalar(src, d0, x[rr], row, rd, rope);
        }
      } else {
#pragma unroll
        for (int e = 0; e < 8; ++e) x[rr][e] = 0.0f;
      }
    }
    if (ROWMAJOR) {
#pragma unroll
      for (int rr = 0; rr < 4; ++rr) {
        uint16_t* dst = dst_row + (4 * g + rr) * RS;
        if (pair) {
          u32x2 lo, hi;
          lo[0] = pack2(x[rr][0], x[rr][1]);
          lo[1] = pack2(x[rr][2], x[rr][3]);
          hi[0] = pack2(x[rr][4], x[rr][5]);
          hi[1] = pack2(x[rr][6], x[rr][7]);
          *reinterpret_cast<u32x2*>(dst + p0) = lo;
          *reinterpret_cast<u32x2*>(dst + half + p0) = hi;
        } else {
          u32x4 w;
#pragma unroll
          for (int e = 0; e < 4; ++e) w[e] = pack2(x[rr][2 * e], x[rr][2 * e + 1]);
          *reinterpret_cast<u32x4*>(dst + d0) = w;
        }
      }
    }
    if (TRANS) {
      const int col = tcol<PERM>(4 * g);
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int dim = pair ? (e < 4 ? p0 + e : half + p0 + e - 4) : d0 + e;
        u32x2 w;
        w[0] = pack2(x[0][e], x[1][e]);
        w[1] = pack2(x[2][e], x[3][e]);
        *reinterpret_cast<u32x2*>(dst_t + dim * TS + col) = w;
      }
    }
  }
}

}  // namespace neox
