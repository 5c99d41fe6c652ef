// Autoregressive decoding step on gfx950: one new token per (batch, head)
// against a key/value cache ("FasterTransformer GPT-NeoX 推理指南", section
// "背景": the decoder that generates one token at a time).
//
//   split:   the cache rows of each (batch, head) are cut into chunks (a
//            multiple of 256 rows, chosen per call from the head count so that
//            the grid fills the chip); the new token sits at position
//            t = cache_lens[b] and the chunks up to the one holding t each get
//            a workgroup.  Every workgroup rotates the query itself
//            (q~ = R_t q, NeoX rotate-half); the workgroup whose chunk holds t
//            also rotates the key, writes k~ and v into cache row t and takes
//            that key from registers, so no workgroup reads a row written in
//            the same launch.  The cached rows (< t) stream through the 4
//            waves: one key row per group of D/8 lanes, 16 bytes per lane,
//            nontemporal loads (the cache is read once per step), in batches
//            issued before any is used, the next batch in flight while the
//            current one is consumed; rows past the chunk end and idle lanes
//            are clamped to valid addresses and masked, so the loads carry no
//            branches.  Each wave keeps an online softmax (running max, sum and
//            the weighted value sum of its dims); the waves merge through LDS
//            into one partial (m, l, o) per chunk, in the exp2 domain.  With a
//            single chunk per head the workgroup writes o and lse itself.
//   combine: (more than one chunk per head) one wave per (batch, head) merges
//            the chunk partials: o = sum 2^(m_i - M) o_i / sum 2^(m_i - M) l_i,
//            lse = (M + log2 L) ln 2; lane i weighs chunk i, and the o loads
//            of different chunks are independent.
//
// The step reads every cached key and value once, so it is bound by HBM
// bandwidth: 2 t D element reads per (batch, head).
#include <mutex>
#include <type_traits>
#include <vector>

#include "../../include/neoxattn.h"
#include "device_common.hpp"

// Chunk partials of neox_rope_attn_decode_noalloc: one fixed array in every
// device's copy of the code object, held until the process ends.  In host code
// this name is only a stand-in for the device address; decode_scratch() looks
// the real one up per device, and only that pointer reaches kernels.
static __device__ __align__(256) float scratch[NEOX_DECODE_SCRATCH_BYTES / sizeof(float)];

namespace neox {
namespace {

// Tuning: steps per load batch (bf16; fp32 takes half), double-buffered
// batches, first batch issued before the query rotation, nontemporal cache
// loads, and (for measurements) a fixed chunk size instead of the per-call
// choice.
#ifndef NEOX_DEC_NB
#define NEOX_DEC_NB 8
#endif
#ifndef NEOX_DEC_PIPE
#define NEOX_DEC_PIPE 1
#endif
#ifndef NEOX_DEC_EARLY
#define NEOX_DEC_EARLY 1
#endif
#ifndef NEOX_DEC_NTLOAD
#define NEOX_DEC_NTLOAD 1
#endif
#ifndef NEOX_DEC_FORCE_CHUNK
#define NEOX_DEC_FORCE_CHUNK 0
#endif
#ifndef NEOX_DEC_MIN_GROUPS
#define NEOX_DEC_MIN_GROUPS 512
#endif
constexpr int DEC_TILE = 256;  // chunks are multiples of this many rows
constexpr int DEC_NT = 256;    // threads per split workgroup (4 waves)

// 16-byte load of streamed cache data.
__device__ __forceinline__ u32x4 ld16(const void* p) {
#if NEOX_DEC_NTLOAD
  return __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
#else
  return *reinterpret_cast<const u32x4*>(p);
#endif
}

template <typename T>
struct Elem;
template <>
struct Elem<uint16_t> {  // bf16 storage
  static constexpr int W = 4;  // dwords per 8 elements
  static __device__ __forceinline__ void load8(const uint16_t* p, uint32_t* w) {
    const u32x4 x = ld16(p);
#pragma unroll
    for (int e = 0; e < 4; ++e) w[e] = x[e];
  }
  static __device__ __forceinline__ float get(const uint32_t* w, int e) {
    return (e & 1) ? bf_hi(w[e >> 1]) : bf_lo(w[e >> 1]);
  }
  static __device__ __forceinline__ float load1(const uint16_t* p) { return bf2f(*p); }
  static __device__ __forceinline__ void store1(uint16_t* p, float x) {
    *p = __builtin_bit_cast(uint16_t, (__bf16)x);  // round to nearest even
  }
};
struct half_t {  // IEEE half storage
  uint16_t bits;
};
template <>
struct Elem<half_t> {
  static constexpr int W = 4;
  static __device__ __forceinline__ void load8(const half_t* p, uint32_t* w) {
    const u32x4 x = ld16(p);
#pragma unroll
    for (int e = 0; e < 4; ++e) w[e] = x[e];
  }
  static __device__ __forceinline__ float h2f(uint32_t bits16) {
    return (float)__builtin_bit_cast(_Float16, (uint16_t)bits16);
  }
  static __device__ __forceinline__ float get(const uint32_t* w, int e) {
    return h2f((e & 1) ? (w[e >> 1] >> 16) : (w[e >> 1] & 0xffffu));
  }
  static __device__ __forceinline__ float load1(const half_t* p) { return h2f(p->bits); }
  static __device__ __forceinline__ void store1(half_t* p, float x) {
    p->bits = __builtin_bit_cast(uint16_t, (_Float16)x);  // round to nearest even
  }
};
template <>
struct Elem<float> {  // fp32 storage
  static constexpr int W = 8;
  static __device__ __forceinline__ void load8(const float* p, uint32_t* w) {
    const u32x4 a = ld16(p);
    const u32x4 b = ld16(p + 4);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      w[e] = a[e];
      w[4 + e] = b[e];
    }
  }
  static __device__ __forceinline__ float get(const uint32_t* w, int e) {
    return __uint_as_float(w[e]);
  }
  static __device__ __forceinline__ float load1(const float* p) { return *p; }
  static __device__ __forceinline__ void store1(float* p, float x) { *p = x; }
};

__device__ __forceinline__ int decode_pos(const DecodeParams& p, int b) {
  const int t = p.lens[b];
  return t < 0 ? 0 : (t >= p.cap ? p.cap - 1 : t);  // malformed lengths: no stray access
}

// NeoX rotate-half of element d of a row at position t (fp32).
template <typename T>
__device__ __forceinline__ float rope_elem(const T* row, int d, int t, int rd, const float2* rope) {
  const float x = Elem<T>::load1(row + d);
  if (d >= rd) return x;
  const int half = rd >> 1;
  const bool first = d < half;
  const float xp = Elem<T>::load1(row + (first ? d + half : d - half));
  const float2 cs = rope[(int64_t)t * half + (first ? d : d - half)];
  return fmaf(xp, first ? -cs.y : cs.y, x * cs.x);
}

// Sum over aligned groups of G = 8 or 16 lanes, result in every lane, by DPP
// lane swaps within a row of 16: quad [1,0,3,2], quad [2,3,0,1], reverse
// within 8 (each quad meets the other), reverse within 16 (each half meets the
// other).
template <int G>
__device__ __forceinline__ float group_sum(float x) {
  auto dpp = [](float v, auto ctrl) {
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), decltype(ctrl)::value,
                                                      0xF, 0xF, false));
  };
  x += dpp(x, std::integral_constant<int, 0xB1>{});   // quad_perm [1,0,3,2]
  x += dpp(x, std::integral_constant<int, 0x4E>{});   // quad_perm [2,3,0,1]
  x += dpp(x, std::integral_constant<int, 0x141>{});  // row_half_mirror
  if constexpr (G == 16) x += dpp(x, std::integral_constant<int, 0x140>{});  // row_mirror
  return x;
}

template <typename T, int D>
struct DecodeTile {
  static constexpr int C = D / 8;                     // lanes holding one row
  static constexpr int G = C <= 8 ? 8 : 16;           // lanes per row group
  static constexpr int KPW = 64 / G;                  // rows per wave step
  static constexpr int NB = Elem<T>::W == 4 ? NEOX_DEC_NB : NEOX_DEC_NB / 2;  // steps per batch
  static constexpr int RB = 4 * KPW * NB;             // rows per workgroup batch
  static_assert(DEC_TILE % RB == 0, "whole batches per tile");
};

template <typename T, int D>
__global__ __launch_bounds__(DEC_NT) void decode_split_kernel(DecodeParams p) {
  using DT = DecodeTile<T, D>;
  constexpr int G = DT::G, C = DT::C, KPW = DT::KPW, NB = DT::NB, EW = Elem<T>::W;
  __shared__ float qs[D], ks[D], vs[D];
  __shared__ float wm[4], wl[4], st_new;
  __shared__ __align__(16) float wo[4][D];

  const int s = blockIdx.x % p.nsplit;
  const int bh = blockIdx.x / p.nsplit;
  const int b = bh / p.H;
  const int t = decode_pos(p, b);
  const int k0 = s * p.chunk;
  if (k0 > t) return;  // chunk past the new token: the combine pass skips it
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const bool last = t - k0 < p.chunk;         // this chunk holds the new token
  const int kend = min(k0 + p.chunk, t);      // cached rows of this chunk: [k0, kend)
  const int nbt = (kend - k0 + DT::RB - 1) / DT::RB;  // batches (0 when none)
  const T* kb = (const T*)p.k_cache + (int64_t)bh * p.cap * D;
  const T* vb = (const T*)p.v_cache + (int64_t)bh * p.cap * D;
  const int g = lane & (G - 1), kl = lane / G;
  const bool act = g < C;
  const int d0 = act ? 8 * g : D - 8;  // idle lanes re-read valid dims, weighted by 0

  // Batch bt: wave w, step i reads row k0 + bt * RB + (i * 4 + w) * KPW + kl; rows
  // past kend re-read row kend - 1 and are masked.
  uint32_t kw[1 + NEOX_DEC_PIPE][NB][EW], vw[1 + NEOX_DEC_PIPE][NB][EW];
  auto issue = [&](int bt, uint32_t (&kd)[NB][EW], uint32_t (&vd)[NB][EW]) {
#pragma unroll
    for (int i = 0; i < NB; ++i) {
      const int j = k0 + bt * DT::RB + (i * 4 + wave) * KPW + kl;
      const int64_t row = j < kend ? j : kend - 1;
      Elem<T>::load8(kb + row * D + d0, kd[i]);
      Elem<T>::load8(vb + row * D + d0, vd[i]);
    }
  };
#if NEOX_DEC_EARLY
  if (nbt > 0) issue(0, kw[0], vw[0]);
  __builtin_amdgcn_sched_barrier(0);
#endif

  // Rotated query (every workgroup) and, in the chunk of t, the new key and value.
  if (tid < D) {
    qs[tid] = rope_elem((const T*)p.q + (int64_t)bh * D, tid, t, p.rd, p.rope);
    if (last) {
      const float kr = rope_elem((const T*)p.k + (int64_t)bh * D, tid, t, p.rd, p.rope);
      const T vraw = ((const T*)p.v)[(int64_t)bh * D + tid];
      ks[tid] = kr;
      vs[tid] = Elem<T>::load1(&vraw);
      Elem<T>::store1((T*)p.k_cache + ((int64_t)bh * p.cap + t) * D + tid, kr);
      ((T*)p.v_cache)[((int64_t)bh * p.cap + t) * D + tid] = vraw;
    }
  }
  __syncthreads();

  float qv[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) qv[e] = act ? qs[d0 + e] : 0.0f;
  const float c2 = p.scale_log2;

  float m = -INFINITY, l = 0.0f, o[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) o[e] = 0.0f;
  auto consume = [&](int bt, const uint32_t (&kd)[NB][EW], const uint32_t (&vd)[NB][EW]) {
    float sc[NB];
    float mb = -INFINITY;
#pragma unroll
    for (int i = 0; i < NB; ++i) {
      const int j = k0 + bt * DT::RB + (i * 4 + wave) * KPW + kl;
      float dot = 0.0f;
#pragma unroll
      for (int e = 0; e < 8; ++e) dot = fmaf(qv[e], Elem<T>::get(kd[i], e), dot);
      dot = group_sum<G>(dot);
      sc[i] = j < kend ? dot * c2 : -INFINITY;
      mb = fmaxf(mb, sc[i]);
    }
    const float m_new = fmaxf(m, mb);
    if (m_new != -INFINITY) {  // some row of this group's batch is in range
      const float corr = fast_exp2(m - m_new);
      l *= corr;
#pragma unroll
      for (int e = 0; e < 8; ++e) o[e] *= corr;
#pragma unroll
      for (int i = 0; i < NB; ++i) {
        const float pr = fast_exp2(sc[i] - m_new);
        l += pr;
#pragma unroll
        for (int e = 0; e < 8; ++e) o[e] = fmaf(pr, Elem<T>::get(vd[i], e), o[e]);
      }
      m = m_new;
    }
  };
  if (nbt > 0) {
#if !NEOX_DEC_EARLY
    issue(0, kw[0], vw[0]);
#endif
#if NEOX_DEC_PIPE
    // Two buffers: batch bt + 1 is in flight while batch bt is consumed.
    for (int bt = 0; bt < nbt; bt += 2) {
      if (bt + 1 < nbt) issue(bt + 1, kw[1], vw[1]);
      __builtin_amdgcn_sched_barrier(0);
      consume(bt, kw[0], vw[0]);
      if (bt + 1 < nbt) {
        if (bt + 2 < nbt) issue(bt + 2, kw[0], vw[0]);
        __builtin_amdgcn_sched_barrier(0);
        consume(bt + 1, kw[1], vw[1]);
      }
    }
#else
    for (int bt = 0; bt < nbt; ++bt) {
      if (bt > 0) issue(bt, kw[0], vw[0]);
      __builtin_amdgcn_sched_barrier(0);  // the whole batch is in flight before any use
      consume(bt, kw[0], vw[0]);
    }
#endif
    // Merge the KPW row groups of the wave (lanes holding the same dims).
#pragma unroll
    for (int x = G; x < 64; x <<= 1) {
      const float m2 = __shfl_xor(m, x), l2 = __shfl_xor(l, x);
      const float mm = fmaxf(m, m2);
      const float f1 = mm == -INFINITY ? 0.0f : fast_exp2(m - mm);
      const float f2 = mm == -INFINITY ? 0.0f : fast_exp2(m2 - mm);
      l = l * f1 + l2 * f2;
#pragma unroll
      for (int e = 0; e < 8; ++e) o[e] = o[e] * f1 + __shfl_xor(o[e], x) * f2;
      m = mm;
    }
  }
  if (lane == 0) {
    wm[wave] = m;
    wl[wave] = l;
  }
  if (kl == 0 && act) {
    *reinterpret_cast<f32x4*>(&wo[wave][d0]) = f32x4{o[0], o[1], o[2], o[3]};
    *reinterpret_cast<f32x4*>(&wo[wave][d0 + 4]) = f32x4{o[4], o[5], o[6], o[7]};
  }
  if (last && wave == 0) {  // score of the new key
    float dot = 0.0f;
    for (int d = lane; d < D; d += 64) dot = fmaf(qs[d], ks[d], dot);
#pragma unroll
    for (int x = 32; x >= 1; x >>= 1) dot += __shfl_xor(dot, x);
    if (lane == 0) st_new = dot * c2;
  }
  __syncthreads();

  // One partial per chunk: the 4 waves plus, in the chunk of t, the new key.
  if (tid < D) {
    const float sn = last ? st_new : -INFINITY;
    const float M = fmaxf(fmaxf(fmaxf(wm[0], wm[1]), fmaxf(wm[2], wm[3])), sn);
    float L = 0.0f, O = 0.0f;
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      const float f = wm[w] == -INFINITY ? 0.0f : fast_exp2(wm[w] - M);
      L = fmaf(wl[w], f, L);
      O = fmaf(wo[w][tid], f, O);
    }
    if (last) {
      const float f = fast_exp2(sn - M);
      L += f;
      O = fmaf(vs[tid], f, O);
    }
    if (p.nsplit == 1) {  // the only chunk: final output
      Elem<T>::store1((T*)p.o + (int64_t)bh * D + tid, O / L);
      if (tid == 0) p.lse[bh] = (M + __log2f(L)) * kLn2;
    } else {
      float* part = p.part + ((int64_t)bh * p.nsplit + s) * (D + 4);
      part[4 + tid] = O;
      if (tid == 0) {
        part[0] = M;
        part[1] = L;
      }
    }
  }
}

// One wave per (batch, head): merge the partials of chunks 0 .. t / chunk.
template <typename T, int D>
__global__ __launch_bounds__(256) void decode_combine_kernel(DecodeParams p) {
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int bh = blockIdx.x * 4 + wave;
  if (bh >= p.B * p.H) return;  // whole waves only
  const int b = bh / p.H;
  const int t = decode_pos(p, b);
  const int nch = t / p.chunk + 1;
  const float* part = p.part + (int64_t)bh * p.nsplit * (D + 4);
  float M = -INFINITY;
  for (int i = lane; i < nch; i += 64) M = fmaxf(M, part[i * (D + 4)]);
#pragma unroll
  for (int x = 32; x >= 1; x >>= 1) M = fmaxf(M, __shfl_xor(M, x));
  float L = 0.0f, O0 = 0.0f, O1 = 0.0f;
  const int d0 = lane < D ? lane : 0;
  const int d1 = lane + 64 < D ? lane + 64 : lane;  // D <= 128
  for (int i0 = 0; i0 < nch; i0 += 64) {
    const int i = i0 + lane;
    const float mi = i < nch ? part[i * (D + 4)] : -INFINITY;
    const float w = mi == -INFINITY ? 0.0f : fast_exp2(mi - M);
    if (i < nch) L = fmaf(part[i * (D + 4) + 1], w, L);
    // Chunks past nch - 1 carry weight 0 and re-read the last partial.
    const int n8 = (min(64, nch - i0) + 7) & ~7;
    for (int c = 0; c < n8; c += 8) {
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const float wc = __shfl(w, c + u);
        const float* pc = part + min(i0 + c + u, nch - 1) * (D + 4) + 4;
        O0 = fmaf(pc[d0], wc, O0);
        O1 = fmaf(pc[d1], wc, O1);
      }
    }
  }
#pragma unroll
  for (int x = 32; x >= 1; x >>= 1) L += __shfl_xor(L, x);
  const float inv = 1.0f / L;
  T* o = (T*)p.o + (int64_t)bh * D;
  if (lane < D) Elem<T>::store1(o + lane, O0 * inv);
  if (lane + 64 < D) Elem<T>::store1(o + lane + 64, O1 * inv);
  if (lane == 0) p.lse[bh] = (M + __log2f(L)) * kLn2;
}

template <typename T, int D>
hipError_t launch_decode_d(const DecodeParams& p, hipStream_t st) {
  const unsigned BH = (unsigned)(p.B * p.H);
  hipLaunchKernelGGL((decode_split_kernel<T, D>), dim3(BH * (unsigned)p.nsplit), dim3(DEC_NT), 0,
                     st, p);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || p.nsplit == 1) return e;
  hipLaunchKernelGGL((decode_combine_kernel<T, D>), dim3((BH + 3) / 4), dim3(256), 0, st, p);
  return hipGetLastError();
}

template <typename T>
hipError_t launch_decode_t(const DecodeParams& p, hipStream_t st) {
  switch (p.D) {
    case 64: return launch_decode_d<T, 64>(p, st);
    case 96: return launch_decode_d<T, 96>(p, st);
    case 128: return launch_decode_d<T, 128>(p, st);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace

int decode_tile_rows() { return DEC_TILE; }

// Chunk size: the largest power-of-two multiple of 256 rows (at most the
// cache rounded up) that still gives at least NEOX_DEC_MIN_GROUPS split
// workgroups, so that the chip stays full while the partial merge shrinks
// (a single chunk needs no combine pass at all).
void decode_plan(int BH, int cap, int* chunk, int* nsplit) {
  int c = DEC_TILE;
#if NEOX_DEC_FORCE_CHUNK
  c = NEOX_DEC_FORCE_CHUNK;
#else
  while (c < cap && (int64_t)BH * ((cap + 2 * c - 1) / (2 * c)) >= NEOX_DEC_MIN_GROUPS) c *= 2;
#endif
  *chunk = c;
  *nsplit = (cap + c - 1) / c;
}

// Device address of `scratch` on device `dev`, which must be the current
// device; looked up once per device and kept.
hipError_t decode_scratch(int dev, float** out) {
  static std::mutex mu;
  static std::vector<float*> addr;  // indexed by device
  if (dev < 0) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lk(mu);
  if ((size_t)dev >= addr.size()) addr.resize((size_t)dev + 1, nullptr);
  if (addr[dev] == nullptr) {
    void* ptr = nullptr;
    const hipError_t e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (ptr == nullptr) return hipErrorInvalidSymbol;
    addr[dev] = static_cast<float*>(ptr);
  }
  *out = addr[dev];
  return hipSuccess;
}

hipError_t launch_decode(const DecodeParams& p, hipStream_t st) {
  switch (p.dtype) {
    case 0: return launch_decode_t<float>(p, st);
    case 1: return launch_decode_t<uint16_t>(p, st);
    case 2: return launch_decode_t<half_t>(p, st);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace neox
