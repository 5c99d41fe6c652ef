// Forward attention with fp32 storage and fp32 arithmetic throughout.
//
// The bf16 MFMA path cannot meet an fp32 accuracy bound, so fp32 inputs run on
// the vector ALUs: the same tiled, online-softmax algorithm (exact attention,
// "GPT-NeoX 开源训练框架深度解读", section "问题二：注意力计算太慢") with K/V
// tiles of 32 keys staged in LDS.  Eight lanes share a query row, each
// holding an eighth of the head dims; the partial dot products meet with three
// lane swaps.
#include "device_common.hpp"

namespace neox {
namespace {

constexpr int QB = 16;          // queries per workgroup
constexpr int LQ = 8;           // lanes per query, each with D / 8 dims
constexpr int KB = 32;          // keys per tile
constexpr int NT = QB * LQ;     // 128 threads

// Rotated value of dim d of an fp32 row at position pos (rotate-half pairs).
__device__ __forceinline__ float rot_elem_f32(const float* row, int d, int pos, int rd,
                                              const float2* rope) {
  const float x = row[d];
  if (d >= rd) return x;
  const int half = rd >> 1;
  if (d < half) {
    const float2 cs = rope[(int64_t)pos * half + d];
    return x * cs.x - row[d + half] * cs.y;
  }
  const float2 cs = rope[(int64_t)pos * half + d - half];
  return x * cs.x + row[d - half] * cs.y;
}

// Small problems are latency bound (one fp32 S=128 head pair is a handful of
// workgroups), so every global load of a tile -- K and V rows and the rotary
// table entries of its keys -- is issued at once into registers, one tile
// ahead of the tile being computed; the raw rows then go to LDS and the rotary
// pairs of K are turned in place there.
template <int D>
__global__ __launch_bounds__(NT) void fwd_f32_kernel(FwdParams p) {
  constexpr int DL = D / LQ;                 // dims per lane
  constexpr int RS = D + 4;                  // LDS row stride (floats), 16-byte rows
  constexpr int NV4 = KB * D / 4 / NT;       // float4 of K (and of V) per thread per tile
  constexpr int NCS = KB * (D / 2) / NT;     // rotary pairs per thread per tile, at most
  static_assert(DL % 4 == 0 && (KB * D / 4) % NT == 0, "tile split");
  __shared__ __attribute__((aligned(16))) float Ks[KB * RS];
  __shared__ __attribute__((aligned(16))) float Vs[KB * RS];

  const AttnShape& a = p.a;
  const int S = a.S;
  const int nqt = (S + QB - 1) / QB;
  const int BH = a.B * a.H;
  const int qt = nqt - 1 - (int)(blockIdx.x / BH);
  const int bh = (int)(blockIdx.x % BH);
  const int b = bh / a.H, h = bh % a.H;
  const int tid = threadIdx.x;
  const int part = tid & (LQ - 1);
  const int q0 = qt * QB;
  const int qi = q0 + tid / LQ;
  const int qc = qi < S ? qi : S - 1;
  const int rd = a.rd, half = rd >> 1;

  const float* qb = (const float*)p.q + b * p.sq.b + h * p.sq.h;
  const float* kb = (const float*)p.k + b * p.sk.b + h * p.sk.h;
  const float* vb = (const float*)p.v + b * p.sv.b + h * p.sv.h;
  const int32_t* drow = a.docs ? a.docs + (int64_t)b * (a.n_docs + 1) : nullptr;

  int lo = 0, hi = S - 1;
  if (drow) {
    int ds, de;
    doc_bounds(drow, a.n_docs, S, qc, ds, de);
    lo = ds;
    hi = de - 1;
  }
  if (a.causal && qi < hi) hi = qi;
  const int qlast = (q0 + QB - 1 < S - 1) ? q0 + QB - 1 : S - 1;
  int blo = 0, bhi = S - 1;
  if (drow) {
    int s0, e0, s1, e1;
    doc_bounds(drow, a.n_docs, S, q0, s0, e0);
    doc_bounds(drow, a.n_docs, S, qlast, s1, e1);
    blo = s0;
    bhi = e1 - 1;
  }
  if (a.causal && qlast < bhi) bhi = qlast;

  // Tile prefetch registers: raw K and V rows, rotary (cos, sin) of the pairs.
  f32x4 kr[NV4], vr[NV4];
  float2 cs[NCS > 0 ? NCS : 1];
  auto fetch = [&](int k0) {
#pragma unroll
    for (int i = 0; i < NV4; ++i) {
      const int idx = tid + NT * i, row = idx / (D / 4), c4 = idx % (D / 4);
      const int j = min(k0 + row, S - 1);
      kr[i] = *reinterpret_cast<const f32x4*>(kb + (int64_t)j * p.sk.s + 4 * c4);
      vr[i] = *reinterpret_cast<const f32x4*>(vb + (int64_t)j * p.sv.s + 4 * c4);
    }
#pragma unroll
    for (int i = 0; i < NCS; ++i) {
      const int it = tid + NT * i;
      if (it < KB * half) {
        const int row = it / half, d = it % half;
        cs[i] = a.rope[(int64_t)min(k0 + row, S - 1) * half + d];
      }
    }
  };

  float qh[DL], oh[DL];
#pragma unroll
  for (int e = 0; e < DL; ++e) {
    qh[e] = qi < S ? rot_elem_f32(qb + (int64_t)qc * p.sq.s, part * DL + e, qi, rd, a.rope) : 0.0f;
    oh[e] = 0.0f;
  }
  const float slope = a.alibi ? (a.slopes ? a.slopes[h] : exp2f(-8.0f * (float)(h + 1) / (float)a.H))
                              : 0.0f;
  float m_run = -INFINITY, l_run = 0.0f;

  const int kfirst = (blo / KB) * KB;
  if (kfirst <= bhi) fetch(kfirst);
  for (int k0 = kfirst; k0 <= bhi; k0 += KB) {
    __syncthreads();  // the previous tile is no longer read
#pragma unroll
    for (int i = 0; i < NV4; ++i) {
      const int idx = tid + NT * i, row = idx / (D / 4), c4 = idx % (D / 4);
      *reinterpret_cast<f32x4*>(Ks + row * RS + 4 * c4) = kr[i];
      *reinterpret_cast<f32x4*>(Vs + row * RS + 4 * c4) = vr[i];
    }
    if (rd > 0) {
      __syncthreads();
#pragma unroll
      for (int i = 0; i < NCS; ++i) {
        const int it = tid + NT * i;
        if (it < KB * half) {
          const int row = it / half, d = it % half;
          const float x1 = Ks[row * RS + d], x2 = Ks[row * RS + d + half];
          Ks[row * RS + d] = x1 * cs[i].x - x2 * cs[i].y;
          Ks[row * RS + d + half] = x2 * cs[i].x + x1 * cs[i].y;
        }
      }
    }
    __syncthreads();
    if (k0 + KB <= bhi) fetch(k0 + KB);  // next tile's loads fly during this one

    float sc[KB];
    float mloc = -INFINITY;
#pragma unroll
    for (int r = 0; r < KB; ++r) {
      const float* krow = Ks + r * RS + part * DL;
      float acc = 0.0f;
#pragma unroll
      for (int e4 = 0; e4 < DL / 4; ++e4) {
        const f32x4 kv = *reinterpret_cast<const f32x4*>(krow + 4 * e4);
        acc = fmaf(qh[4 * e4], kv[0], acc);
        acc = fmaf(qh[4 * e4 + 1], kv[1], acc);
        acc = fmaf(qh[4 * e4 + 2], kv[2], acc);
        acc = fmaf(qh[4 * e4 + 3], kv[3], acc);
      }
      acc += __shfl_xor(acc, 1);
      acc += __shfl_xor(acc, 2);
      acc += __shfl_xor(acc, 4);
      float s = acc * a.scale;
      const int j = k0 + r;
      if (a.alibi) s -= slope * (float)(qi - j);
      if (j < lo || j > hi) s = -INFINITY;
      sc[r] = s;
      mloc = fmaxf(mloc, s);
    }
    const float m_new = fmaxf(m_run, mloc);
    const float m_use = (m_new == -INFINITY) ? 0.0f : m_new;
    const float alpha = expf(m_run - m_use);
    l_run *= alpha;
#pragma unroll
    for (int e = 0; e < DL; ++e) oh[e] *= alpha;
#pragma unroll
    for (int r = 0; r < KB; ++r) {
      const float pr = expf(sc[r] - m_use);
      l_run += pr;
      const float* vrow = Vs + r * RS + part * DL;
#pragma unroll
      for (int e4 = 0; e4 < DL / 4; ++e4) {
        const f32x4 vv = *reinterpret_cast<const f32x4*>(vrow + 4 * e4);
        oh[4 * e4] = fmaf(pr, vv[0], oh[4 * e4]);
        oh[4 * e4 + 1] = fmaf(pr, vv[1], oh[4 * e4 + 1]);
        oh[4 * e4 + 2] = fmaf(pr, vv[2], oh[4 * e4 + 2]);
        oh[4 * e4 + 3] = fmaf(pr, vv[3], oh[4 * e4 + 3]);
      }
    }
    m_run = m_new;
  }

  if (qi < S) {
    const float inv_l = l_run > 0.0f ? 1.0f / l_run : 0.0f;
    if (part == 0) p.lse[(int64_t)bh * S + qi] = m_run + logf(l_run);
    float* orow = (float*)p.o + b * p.so.b + h * p.so.h + (int64_t)qi * p.so.s + part * DL;
#pragma unroll
    for (int e4 = 0; e4 < DL / 4; ++e4)
      *reinterpret_cast<f32x4*>(orow + 4 * e4) =
          f32x4{oh[4 * e4] * inv_l, oh[4 * e4 + 1] * inv_l, oh[4 * e4 + 2] * inv_l,
                oh[4 * e4 + 3] * inv_l};
  }
}

template <int D>
hipError_t launch_d(const FwdParams& p, hipStream_t st) {
  const int nqt = (p.a.S + QB - 1) / QB;
  hipLaunchKernelGGL((fwd_f32_kernel<D>), dim3((unsigned)(nqt * p.a.B * p.a.H)), dim3(NT), 0, st,
                     p);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_fwd_f32(const FwdParams& p, hipStream_t st) {
  switch (p.a.D) {
    case 64: return launch_d<64>(p, st);
    case 96: return launch_d<96>(p, st);
    case 128: return launch_d<128>(p, st);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace neox
