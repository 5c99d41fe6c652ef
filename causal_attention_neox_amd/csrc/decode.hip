// Autoregressive decoding step on gfx950: one new token per (batch, head)
// against a key/value cache ("FasterTransformer GPT-NeoX 推理指南", section
// "背景": the decoder that generates one token at a time).  Three passes:
//
//   append:  position t = cache_lens[b]; q~ = R_t q and k~ = R_t k (NeoX
//            rotate-half); k~ and v are written into cache row t, q~ (fp32)
//            into the workspace.
//   split:   the t + 1 cached keys are cut into chunks of 256; each wave of a
//            chunk's workgroup streams its share of key rows (16-byte loads,
//            one key row per group of D/8 lanes, so every load instruction
//            covers whole rows), reduces q~ . k~ across the group with lane
//            swaps, and keeps its own online softmax (running max, sum and the
//            weighted value sum of its dims).  Each wave writes one partial
//            (m, l, o) in the exp2 domain.
//   combine: one wave per (batch, head) merges the partials of the non-empty
//            chunks: o = sum 2^(m_i - M) o_i / sum 2^(m_i - M) l_i, and
//            lse = (M + log2 L) ln 2.
//
// This step reads every cached key and value once, so it is bound by HBM
// bandwidth: 2 (t + 1) D bytes per element size per (batch, head).
#include "device_common.hpp"

namespace neox {
namespace {

constexpr int DEC_CHUNK = 256;  // keys per split workgroup
constexpr int DEC_NT = 256;     // threads per split workgroup (4 waves)

template <typename T>
struct Elem;
template <>
struct Elem<uint16_t> {  // bf16 storage
  static __device__ __forceinline__ void load8(const uint16_t* p, float* x) {
    const u32x4 w = *reinterpret_cast<const u32x4*>(p);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      x[2 * e] = bf_lo(w[e]);
      x[2 * e + 1] = bf_hi(w[e]);
    }
  }
  static __device__ __forceinline__ float load1(const uint16_t* p) { return bf2f(*p); }
  static __device__ __forceinline__ void store1(uint16_t* p, float x) {
    *p = __builtin_bit_cast(uint16_t, (__bf16)x);  // round to nearest even
  }
};
template <>
struct Elem<float> {  // fp32 storage
  static __device__ __forceinline__ void load8(const float* p, float* x) {
    const f32x4 a = *reinterpret_cast<const f32x4*>(p);
    const f32x4 b = *reinterpret_cast<const f32x4*>(p + 4);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      x[e] = a[e];
      x[4 + e] = b[e];
    }
  }
  static __device__ __forceinline__ float load1(const float* p) { return *p; }
  static __device__ __forceinline__ void store1(float* p, float x) { *p = x; }
};

__device__ __forceinline__ int decode_pos(const DecodeParams& p, int b) {
  const int t = p.lens[b];
  return t < 0 ? 0 : (t >= p.cap ? p.cap - 1 : t);  // malformed lengths: no stray access
}

// One wave per (batch, head); lane l handles dims l and l + 64.
template <typename T, int D>
__global__ __launch_bounds__(256) void decode_append_kernel(DecodeParams p) {
  __shared__ float rowbuf[4][2][D];
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int bh = blockIdx.x * 4 + wave;
  if (bh >= p.B * p.H) return;  // whole waves only
  const int b = bh / p.H;
  const int t = decode_pos(p, b);
  const int rd = p.rd, half = rd >> 1;
  const T* qs = (const T*)p.q + (int64_t)bh * D;
  const T* ks = (const T*)p.k + (int64_t)bh * D;
  const T* vs = (const T*)p.v + (int64_t)bh * D;
  T* kc = (T*)p.k_cache + ((int64_t)bh * p.cap + t) * D;
  T* vc = (T*)p.v_cache + ((int64_t)bh * p.cap + t) * D;
#pragma unroll
  for (int r = 0; r < 2; ++r) {
    const int d = lane + 64 * r;
    if (d < D) {
      rowbuf[wave][0][d] = Elem<T>::load1(qs + d);
      rowbuf[wave][1][d] = Elem<T>::load1(ks + d);
      Elem<T>::store1(vc + d, Elem<T>::load1(vs + d));
    }
  }
  lds_wave_sync();
#pragma unroll
  for (int r = 0; r < 2; ++r) {
    const int d = lane + 64 * r;
    if (d >= D) continue;
    float xq = rowbuf[wave][0][d], xk = rowbuf[wave][1][d];
    if (d < rd) {
      const bool first = d < half;
      const int pd = first ? d + half : d - half;
      const float2 cs = p.rope[(int64_t)t * half + (first ? d : d - half)];
      const float sn = first ? -cs.y : cs.y;  // rotate-half: (-x2, x1)
      xq = fmaf(rowbuf[wave][0][pd], sn, xq * cs.x);
      xk = fmaf(rowbuf[wave][1][pd], sn, xk * cs.x);
    }
    p.qrot[(int64_t)bh * D + d] = xq;
    Elem<T>::store1(kc + d, xk);
  }
}

// Workgroup (chunk s, head bh): keys [s * CHUNK, min((s + 1) * CHUNK, t + 1)).
template <typename T, int D>
__global__ __launch_bounds__(DEC_NT) void decode_split_kernel(DecodeParams p) {
  using RG = RowGroups<D>;
  constexpr int C = RG::C, G = RG::G;
  constexpr int KPW = 64 / G;                 // keys per wave step
  constexpr int STEPS = DEC_CHUNK / 4 / KPW;  // steps per wave
  const int s = blockIdx.x % p.nsplit;
  const int bh = blockIdx.x / p.nsplit;
  const int b = bh / p.H;
  const int t = decode_pos(p, b);
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int k0 = s * DEC_CHUNK;
  if (k0 > t) return;  // empty chunk: the combine pass skips it
  const int g = lane & (G - 1), kl = lane / G;
  const bool act = g < C;
  const int d0 = 8 * g;
  const int kend = min(k0 + DEC_CHUNK, t + 1);

  float qv[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) qv[e] = act ? p.qrot[(int64_t)bh * D + d0 + e] : 0.0f;
  const T* kb = (const T*)p.k_cache + (int64_t)bh * p.cap * D + d0;
  const T* vb = (const T*)p.v_cache + (int64_t)bh * p.cap * D + d0;
  const float c2 = p.scale_log2;

  float m = -INFINITY, l = 0.0f, o[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) o[e] = 0.0f;
  // Wave w takes the key rows k0 + (step * 4 + w) * KPW + kl.
#pragma unroll 4
  for (int st = 0; st < STEPS; ++st) {
    const int j = k0 + (st * 4 + wave) * KPW + kl;
    const bool valid = j < kend;
    float kx[8], vx[8];
    if (valid && act) {
      Elem<T>::load8(kb + (int64_t)j * D, kx);
      Elem<T>::load8(vb + (int64_t)j * D, vx);
    } else {
#pragma unroll
      for (int e = 0; e < 8; ++e) kx[e] = vx[e] = 0.0f;
    }
    float dot = 0.0f;
#pragma unroll
    for (int e = 0; e < 8; ++e) dot = fmaf(qv[e], kx[e], dot);
#pragma unroll
    for (int x = G / 2; x >= 1; x >>= 1) dot += __shfl_xor(dot, x);
    const float sc = valid ? dot * c2 : -INFINITY;
    const float m_new = fmaxf(m, sc);
    if (m_new != -INFINITY) {
      const float corr = fast_exp2(m - m_new);
      const float pr = fast_exp2(sc - m_new);
      l = l * corr + pr;
#pragma unroll
      for (int e = 0; e < 8; ++e) o[e] = fmaf(pr, vx[e], o[e] * corr);
      m = m_new;
    }
  }
  // Merge the KPW key groups of the wave (lanes with the same dims slot).
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
  // Partial (m, l, o[D]) of this wave: index s * 4 + wave.
  float* part = p.part + ((int64_t)bh * p.nsplit * 4 + s * 4 + wave) * (D + 4);
  if (lane == 0) {
    part[0] = m;
    part[1] = l;
  }
  if (kl == 0 && act) {
    *reinterpret_cast<f32x4*>(part + 4 + d0) = f32x4{o[0], o[1], o[2], o[3]};
    *reinterpret_cast<f32x4*>(part + 4 + d0 + 4) = f32x4{o[4], o[5], o[6], o[7]};
  }
}

// One wave per (batch, head): merge the partials of chunks 0 .. t / CHUNK.
template <typename T, int D>
__global__ __launch_bounds__(256) void decode_combine_kernel(DecodeParams p) {
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int bh = blockIdx.x * 4 + wave;
  if (bh >= p.B * p.H) return;
  const int b = bh / p.H;
  const int t = decode_pos(p, b);
  const int np = (t / DEC_CHUNK + 1) * 4;
  const float* part = p.part + (int64_t)bh * p.nsplit * 4 * (D + 4);
  float M = -INFINITY;
  for (int i = 0; i < np; ++i) M = fmaxf(M, part[i * (D + 4)]);
  float L = 0.0f, O0 = 0.0f, O1 = 0.0f;
  for (int i = 0; i < np; ++i) {
    const float* pi = part + i * (D + 4);
    const float mi = pi[0];
    if (mi == -INFINITY) continue;  // a wave with no key in range
    const float f = fast_exp2(mi - M);
    L = fmaf(pi[1], f, L);
    if (lane < D) O0 = fmaf(pi[4 + lane], f, O0);
    if (lane + 64 < D) O1 = fmaf(pi[4 + 64 + lane], f, O1);
  }
  const float inv = 1.0f / L;
  T* o = (T*)p.o + (int64_t)bh * D;
  if (lane < D) Elem<T>::store1(o + lane, O0 * inv);
  if (lane + 64 < D) Elem<T>::store1(o + 64 + lane, O1 * inv);
  if (lane == 0) p.lse[bh] = (M + __log2f(L)) * kLn2;
}

template <typename T, int D>
hipError_t launch_decode_d(const DecodeParams& p, hipStream_t st) {
  const unsigned BH = (unsigned)(p.B * p.H);
  hipLaunchKernelGGL((decode_append_kernel<T, D>), dim3((BH + 3) / 4), dim3(256), 0, st, p);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((decode_split_kernel<T, D>), dim3(BH * (unsigned)p.nsplit), dim3(DEC_NT), 0,
                     st, p);
  if ((e = hipGetLastError()) != hipSuccess) return e;
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

int decode_chunk_keys() { return DEC_CHUNK; }

hipError_t launch_decode(const DecodeParams& p, hipStream_t st) {
  return p.bf16 ? launch_decode_t<uint16_t>(p, st) : launch_decode_t<float>(p, st);
}

}  // namespace neox
