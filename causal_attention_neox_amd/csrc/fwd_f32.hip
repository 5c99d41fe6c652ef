// Forward attention with fp32 storage and fp32 arithmetic throughout.
//
// The bf16 MFMA path cannot meet an fp32 accuracy bound, so fp32 inputs run on
// the vector ALUs: the same tiled, online-softmax algorithm (exact attention,
// "GPT-NeoX 开源训练框架深度解读", section "问题二：注意力计算太慢") with K/V
// tiles of 32 keys staged in LDS.  Two lanes share a query row, each holding
// half of the head dims; the two partial dot products meet with one lane swap.
#include "device_common.hpp"

namespace neox {
namespace {

constexpr int QB = 64;          // queries per workgroup
constexpr int KB = 32;          // keys per tile
constexpr int NT = 2 * QB;      // two lanes per query

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

template <int D>
__global__ __launch_bounds__(NT) void fwd_f32_kernel(FwdParams p) {
  constexpr int DH = D / 2;
  __shared__ float Ks[KB][D + 1];
  __shared__ float Vs[KB][D + 1];

  const AttnShape& a = p.a;
  const int S = a.S;
  const int nqt = (S + QB - 1) / QB;
  const int BH = a.B * a.H;
  const int qt = nqt - 1 - (int)(blockIdx.x / BH);
  const int bh = (int)(blockIdx.x % BH);
  const int b = bh / a.H, h = bh % a.H;
  const int tid = threadIdx.x;
  const int half_id = tid & 1;
  const int q0 = qt * QB;
  const int qi = q0 + (tid >> 1);
  const int qc = qi < S ? qi : S - 1;

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

  float qh[DH], oh[DH];
  {
    const float* qrow = qb + (int64_t)qc * p.sq.s;
#pragma unroll
    for (int e = 0; e < DH; ++e) {
      const int d = half_id * DH + e;
      qh[e] = qi < S ? rot_elem_f32(qrow, d, qi, a.rd, a.rope) : 0.0f;
      oh[e] = 0.0f;
    }
  }
  const float slope = a.alibi ? (a.slopes ? a.slopes[h] : exp2f(-8.0f * (float)(h + 1) / (float)a.H))
                              : 0.0f;
  float m_run = -INFINITY, l_run = 0.0f;

  for (int k0 = (blo / KB) * KB; k0 <= bhi; k0 += KB) {
    __syncthreads();
    for (int it = tid; it < KB * D; it += NT) {
      const int r = it / D, d = it % D;
      const int j = k0 + r;
      float kv = 0.0f, vv = 0.0f;
      if (j < S) {
        kv = rot_elem_f32(kb + (int64_t)j * p.sk.s, d, j, a.rd, a.rope);
        vv = vb[(int64_t)j * p.sv.s + d];
      }
      Ks[r][d] = kv;
      Vs[r][d] = vv;
    }
    __syncthreads();
    float sc[KB];
    float mloc = -INFINITY;
#pragma unroll 4
    for (int r = 0; r < KB; ++r) {
      float part = 0.0f;
#pragma unroll
      for (int e = 0; e < DH; ++e) part = fmaf(qh[e], Ks[r][half_id * DH + e], part);
      float s = (part + __shfl_xor(part, 1)) * a.scale;
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
    for (int e = 0; e < DH; ++e) oh[e] *= alpha;
#pragma unroll 4
    for (int r = 0; r < KB; ++r) {
      const float pr = expf(sc[r] - m_use);
      l_run += pr;
#pragma unroll
      for (int e = 0; e < DH; ++e) oh[e] = fmaf(pr, Vs[r][half_id * DH + e], oh[e]);
    }
    m_run = m_new;
  }

  if (qi < S) {
    const float inv_l = l_run > 0.0f ? 1.0f / l_run : 0.0f;
    if (half_id == 0) p.lse[(int64_t)bh * S + qi] = m_run + logf(l_run);
    float* orow = (float*)p.o + b * p.so.b + h * p.so.h + (int64_t)qi * p.so.s + half_id * DH;
#pragma unroll
    for (int e = 0; e < DH; ++e) orow[e] = oh[e] * inv_l;
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
