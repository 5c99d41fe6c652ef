// Backward attention with fp32 storage and fp32 arithmetic (vector ALUs).
//
// Same recompute-from-logsumexp backward as the bf16 path, arranged for
// accuracy rather than speed and without atomics:
//   dkdv kernel: one workgroup per (batch, head, 64 keys), 4 lanes per key,
//                q-tiles of 32 rows staged in LDS; accumulates dK~ and dV and
//                applies R^T to dK~ in the epilogue.
//   dq kernel:   one workgroup per (batch, head, 64 queries), 4 lanes per
//                query, k-tiles of 32 rows in LDS; writes dQ~ to the
//                workspace, and the finalize kernel applies R^T.
// Delta_i = dO_i . o_i comes from the shared preprocess kernel.
#include "device_common.hpp"

namespace neox {

namespace {

constexpr int RB = 64;  // rows (keys or queries) per workgroup
constexpr int TB = 32;  // streamed rows per tile
constexpr int NT = 256; // 4 lanes per row

__device__ __forceinline__ float rot_elem(const float* row, int d, int pos, int rd,
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

// Delta_i = dO_i . o_i and a zeroed dq accumulator row; one wave per row.
template <int D>
__global__ __launch_bounds__(256) void pre_f32_kernel(BwdParams p) {
  const int S = p.a.S;
  const int64_t rows = (int64_t)p.a.B * p.a.H * S;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int64_t r = (int64_t)blockIdx.x * 4 + wave;
  if (r >= rows) return;
  const int bh = (int)(r / S), i = (int)(r % S);
  const int b = bh / p.a.H, h = bh % p.a.H;
  const float* orow = (const float*)p.o + b * p.so.b + h * p.so.h + (int64_t)i * p.so.s;
  const float* grow = (const float*)p.dout + b * p.sdo.b + h * p.sdo.h + (int64_t)i * p.sdo.s;
  float sum = 0.0f;
  for (int d = lane; d < D; d += 64) {
    sum = fmaf(orow[d], grow[d], sum);
    p.dq_acc[r * D + d] = 0.0f;
  }
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) sum += __shfl_xor(sum, m);
  if (lane == 0) p.delta[r] = sum;
}

__device__ __forceinline__ float sum4(float x) {
  x += __shfl_xor(x, 1);
  x += __shfl_xor(x, 2);
  return x;
}

template <int D>
__global__ __launch_bounds__(NT) void dkdv_f32_kernel(BwdParams p) {
  constexpr int DQ = D / 4;
  // q-tile staging during the loop; reused for the dK~ epilogue afterwards.
  constexpr int NF = (2 * TB > RB ? 2 * TB : RB) * (D + 1);
  __shared__ float sbuf[NF];
  __shared__ float Ls[TB], Dl[TB];
  float (*Qs)[D + 1] = reinterpret_cast<float (*)[D + 1]>(sbuf);
  float (*Gs)[D + 1] = reinterpret_cast<float (*)[D + 1]>(sbuf + TB * (D + 1));
  float (*stage)[D + 1] = reinterpret_cast<float (*)[D + 1]>(sbuf);

  const AttnShape& a = p.a;
  const int S = a.S, BH = a.B * a.H;
  const int kt = (int)(blockIdx.x / BH), bh = (int)(blockIdx.x % BH);
  const int b = bh / a.H, h = bh % a.H;
  const int tid = threadIdx.x, part = tid & 3;
  const int k0 = kt * RB, j = k0 + (tid >> 2), jc = j < S ? j : S - 1;
  const float* qb = (const float*)p.q + b * p.sq.b + h * p.sq.h;
  const float* kb = (const float*)p.k + b * p.sk.b + h * p.sk.h;
  const float* vb = (const float*)p.v + b * p.sv.b + h * p.sv.h;
  const float* gb = (const float*)p.dout + b * p.sdo.b + h * p.sdo.h;
  const int32_t* drow = a.docs ? a.docs + (int64_t)b * (a.n_docs + 1) : nullptr;

  int qlo = a.causal ? j : 0, qhi = S - 1;
  if (drow) {
    int ds, de;
    doc_bounds(drow, a.n_docs, S, jc, ds, de);
    qhi = de - 1;
    if (!a.causal) qlo = ds;
  }
  if (j >= S) qlo = S;
  const int klast = (k0 + RB - 1 < S - 1) ? k0 + RB - 1 : S - 1;
  int bqlo = a.causal ? k0 : 0, bqhi = S - 1;
  if (drow) {
    int s0, e0, s1, e1;
    doc_bounds(drow, a.n_docs, S, k0, s0, e0);
    doc_bounds(drow, a.n_docs, S, klast, s1, e1);
    bqhi = e1 - 1;
    if (!a.causal) bqlo = s0;
  }

  float kr[DQ], vr[DQ], dk[DQ], dv[DQ];
#pragma unroll
  for (int e = 0; e < DQ; ++e) {
    const int d = part * DQ + e;
    kr[e] = j < S ? rot_elem(kb + (int64_t)jc * p.sk.s, d, j, a.rd, a.rope) : 0.0f;
    vr[e] = j < S ? vb[(int64_t)jc * p.sv.s + d] : 0.0f;
    dk[e] = 0.0f;
    dv[e] = 0.0f;
  }
  const float slope = a.alibi ? (a.slopes ? a.slopes[h] : exp2f(-8.0f * (float)(h + 1) / (float)a.H))
                              : 0.0f;

  for (int q0 = (bqlo / TB) * TB; q0 <= bqhi; q0 += TB) {
    __syncthreads();
    for (int it = tid; it < TB * D; it += NT) {
      const int r = it / D, d = it % D, i = q0 + r;
      Qs[r][d] = i < S ? rot_elem(qb + (int64_t)i * p.sq.s, d, i, a.rd, a.rope) : 0.0f;
      Gs[r][d] = i < S ? gb[(int64_t)i * p.sdo.s + d] : 0.0f;
    }
    if (tid < TB) {
      const int i = q0 + tid;
      Ls[tid] = i < S ? p.lse[(int64_t)bh * S + i] : 0.0f;
      Dl[tid] = i < S ? p.delta[(int64_t)bh * S + i] : 0.0f;
    }
    __syncthreads();
    for (int r = 0; r < TB; ++r) {
      const int i = q0 + r;
      float sp = 0.0f, dpp = 0.0f;
#pragma unroll
      for (int e = 0; e < DQ; ++e) {
        sp = fmaf(Qs[r][part * DQ + e], kr[e], sp);
        dpp = fmaf(Gs[r][part * DQ + e], vr[e], dpp);
      }
      float s = sum4(sp) * a.scale;
      const float dp = sum4(dpp);
      if (a.alibi) s -= slope * (float)(i - j);
      const bool ok = i >= qlo && i <= qhi && i < S;
      const float pr = ok ? expf(s - Ls[r]) : 0.0f;
      const float ds = pr * (dp - Dl[r]) * a.scale;
#pragma unroll
      for (int e = 0; e < DQ; ++e) {
        dv[e] = fmaf(pr, Gs[r][part * DQ + e], dv[e]);
        dk[e] = fmaf(ds, Qs[r][part * DQ + e], dk[e]);
      }
    }
  }

  // dK = R^T dK~ (partners may sit in other lanes: go through LDS), dV as is.
  __syncthreads();
#pragma unroll
  for (int e = 0; e < DQ; ++e) stage[tid >> 2][part * DQ + e] = dk[e];
  __syncthreads();
  if (j < S) {
    const int half = a.rd >> 1;
    float* dkrow = (float*)p.dk + b * p.sdk.b + h * p.sdk.h + (int64_t)j * p.sdk.s;
    float* dvrow = (float*)p.dv + b * p.sdv.b + h * p.sdv.h + (int64_t)j * p.sdv.s;
#pragma unroll
    for (int e = 0; e < DQ; ++e) {
      const int d = part * DQ + e;
      float y = stage[tid >> 2][d];
      if (d < a.rd) {
        const bool first = d < half;
        const float2 cs = a.rope[(int64_t)j * half + (first ? d : d - half)];
        const float xp = stage[tid >> 2][first ? d + half : d - half];
        y = first ? (y * cs.x + xp * cs.y) : (y * cs.x - xp * cs.y);
      }
      dkrow[d] = y;
      dvrow[d] = dv[e];
    }
  }
}

template <int D>
__global__ __launch_bounds__(NT) void dq_f32_kernel(BwdParams p) {
  constexpr int DQ = D / 4;
  __shared__ float Ks[TB][D + 1];
  __shared__ float Vs[TB][D + 1];

  const AttnShape& a = p.a;
  const int S = a.S, BH = a.B * a.H;
  const int nqt = (S + RB - 1) / RB;
  const int qt = nqt - 1 - (int)(blockIdx.x / BH), bh = (int)(blockIdx.x % BH);
  const int b = bh / a.H, h = bh % a.H;
  const int tid = threadIdx.x, part = tid & 3;
  const int q0 = qt * RB, i = q0 + (tid >> 2), ic = i < S ? i : S - 1;
  const float* qb = (const float*)p.q + b * p.sq.b + h * p.sq.h;
  const float* kb = (const float*)p.k + b * p.sk.b + h * p.sk.h;
  const float* vb = (const float*)p.v + b * p.sv.b + h * p.sv.h;
  const float* gb = (const float*)p.dout + b * p.sdo.b + h * p.sdo.h;
  const int32_t* drow = a.docs ? a.docs + (int64_t)b * (a.n_docs + 1) : nullptr;

  int lo = 0, hi = S - 1;
  if (drow) {
    int ds, de;
    doc_bounds(drow, a.n_docs, S, ic, ds, de);
    lo = ds;
    hi = de - 1;
  }
  if (a.causal && i < hi) hi = i;
  const int qlast = (q0 + RB - 1 < S - 1) ? q0 + RB - 1 : S - 1;
  int blo = 0, bhi = S - 1;
  if (drow) {
    int s0, e0, s1, e1;
    doc_bounds(drow, a.n_docs, S, q0, s0, e0);
    doc_bounds(drow, a.n_docs, S, qlast, s1, e1);
    blo = s0;
    bhi = e1 - 1;
  }
  if (a.causal && qlast < bhi) bhi = qlast;

  float qr[DQ], gr[DQ], dq[DQ];
#pragma unroll
  for (int e = 0; e < DQ; ++e) {
    const int d = part * DQ + e;
    qr[e] = i < S ? rot_elem(qb + (int64_t)ic * p.sq.s, d, i, a.rd, a.rope) : 0.0f;
    gr[e] = i < S ? gb[(int64_t)ic * p.sdo.s + d] : 0.0f;
    dq[e] = 0.0f;
  }
  const float lse_i = i < S ? p.lse[(int64_t)bh * S + i] : 0.0f;
  const float del_i = i < S ? p.delta[(int64_t)bh * S + i] : 0.0f;
  const float slope = a.alibi ? (a.slopes ? a.slopes[h] : exp2f(-8.0f * (float)(h + 1) / (float)a.H))
                              : 0.0f;

  for (int k0 = (blo / TB) * TB; k0 <= bhi; k0 += TB) {
    __syncthreads();
    for (int it = tid; it < TB * D; it += NT) {
      const int r = it / D, d = it % D, jj = k0 + r;
      Ks[r][d] = jj < S ? rot_elem(kb + (int64_t)jj * p.sk.s, d, jj, a.rd, a.rope) : 0.0f;
      Vs[r][d] = jj < S ? vb[(int64_t)jj * p.sv.s + d] : 0.0f;
    }
    __syncthreads();
    for (int r = 0; r < TB; ++r) {
      const int jj = k0 + r;
      float sp = 0.0f, dpp = 0.0f;
#pragma unroll
      for (int e = 0; e < DQ; ++e) {
        sp = fmaf(qr[e], Ks[r][part * DQ + e], sp);
        dpp = fmaf(gr[e], Vs[r][part * DQ + e], dpp);
      }
      float s = sum4(sp) * a.scale;
      const float dp = sum4(dpp);
      if (a.alibi) s -= slope * (float)(i - jj);
      const bool ok = jj >= lo && jj <= hi && jj < S;
      const float pr = ok ? expf(s - lse_i) : 0.0f;
      const float ds = pr * (dp - del_i) * a.scale;
#pragma unroll
      for (int e = 0; e < DQ; ++e) dq[e] = fmaf(ds, Ks[r][part * DQ + e], dq[e]);
    }
  }
  if (i < S) {
    float* acc = p.dq_acc + ((int64_t)bh * S + i) * D + part * DQ;
#pragma unroll
    for (int e = 0; e < DQ; ++e) acc[e] = dq[e];
  }
}

template <int D>
hipError_t launch_main(const BwdParams& p, hipStream_t st) {
  const int BH = p.a.B * p.a.H;
  const int nblk = (p.a.S + RB - 1) / RB;
  hipLaunchKernelGGL((dkdv_f32_kernel<D>), dim3((unsigned)(nblk * BH)), dim3(NT), 0, st, p);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((dq_f32_kernel<D>), dim3((unsigned)(nblk * BH)), dim3(NT), 0, st, p);
  return hipGetLastError();
}

// dq = R^T dQ~ (rotation by -theta) from the fp32 workspace accumulator.  Row
// groups of G lanes, 16 B each; rotary partners are exchanged through LDS.
template <int D>
__global__ __launch_bounds__(256) void dq_finalize_f32_kernel(BwdParams p) {
  using RG = RowGroups<D>;
  constexpr int C = RG::C, G = RG::G, RPW = RG::RPW;
  __shared__ __attribute__((aligned(16))) float rowbuf[4][RPW][D];
  const int S = p.a.S, rd = p.a.rd, half = rd >> 1;
  const int rows = p.a.B * p.a.H * S;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int g = lane & (G - 1), rw = lane / G;
  const int wrow0 = (blockIdx.x * 4 + wave) * RPW;
  if (wrow0 >= rows) return;  // whole waves only
  const int r = wrow0 + rw;
  const bool act = r < rows && g < C;
  const int bh = r / S, i = r - bh * S;
  const int b = bh / p.a.H, h = bh - b * p.a.H;
  const int d0 = 8 * g;
  const bool rot_lane = act && d0 < rd;
  f32x4 lo = f32x4{0.f, 0.f, 0.f, 0.f}, hi = lo;
  float2 cs[8];
  if (act) {
    const float* acc = p.dq_acc + (int64_t)r * D + d0;
    lo = *reinterpret_cast<const f32x4*>(acc);
    hi = *reinterpret_cast<const f32x4*>(acc + 4);
  }
  if (rot_lane) {
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const int d = d0 + e;
      cs[e] = d < rd ? p.a.rope[(int64_t)i * half + (d < half ? d : d - half)]
                     : float2{1.0f, 0.0f};
    }
  }
  float x[8];
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    x[e] = lo[e];
    x[4 + e] = hi[e];
  }
  if (rd > 0) {
    if (act) {
      *reinterpret_cast<f32x4*>(&rowbuf[wave][rw][d0]) = lo;
      *reinterpret_cast<f32x4*>(&rowbuf[wave][rw][d0 + 4]) = hi;
    }
    lds_wave_sync();
    if (rot_lane) {
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int d = d0 + e;
        if (d < rd) {
          const bool first = d < half;
          const float xp = rowbuf[wave][rw][first ? d + half : d - half];
          const float sn = first ? cs[e].y : -cs[e].y;  // transpose of rotate-half
          x[e] = fmaf(xp, sn, x[e] * cs[e].x);
        }
      }
    }
  }
  if (!act) return;
  float* orow = (float*)p.dq + b * p.sdq.b + h * p.sdq.h + (int64_t)i * p.sdq.s + d0;
  *reinterpret_cast<f32x4*>(orow) = f32x4{x[0], x[1], x[2], x[3]};
  *reinterpret_cast<f32x4*>(orow + 4) = f32x4{x[4], x[5], x[6], x[7]};
}

template <int D>
hipError_t launch_finalize(const BwdParams& p, hipStream_t st) {
  const int64_t rows = (int64_t)p.a.B * p.a.H * p.a.S;
  const dim3 grid((unsigned)((rows + RowGroups<D>::RPB - 1) / RowGroups<D>::RPB));
  hipLaunchKernelGGL((dq_finalize_f32_kernel<D>), grid, dim3(256), 0, st, p);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_bwd_f32(const BwdParams& p, hipStream_t st, const hipEvent_t* ev) {
  hipError_t e;
  if ((e = record_event(ev, 0, st)) != hipSuccess) return e;
  const dim3 row_grid((unsigned)(((int64_t)p.a.B * p.a.H * p.a.S + 3) / 4));
  switch (p.a.D) {
    case 64: hipLaunchKernelGGL((pre_f32_kernel<64>), row_grid, dim3(256), 0, st, p); break;
    case 96: hipLaunchKernelGGL((pre_f32_kernel<96>), row_grid, dim3(256), 0, st, p); break;
    case 128: hipLaunchKernelGGL((pre_f32_kernel<128>), row_grid, dim3(256), 0, st, p); break;
    default: return hipErrorInvalidValue;
  }
  if ((e = hipGetLastError()) != hipSuccess) return e;
  if ((e = record_event(ev, 1, st)) != hipSuccess) return e;
  switch (p.a.D) {
    case 64: e = launch_main<64>(p, st); break;
    case 96: e = launch_main<96>(p, st); break;
    case 128: e = launch_main<128>(p, st); break;
    default: return hipErrorInvalidValue;
  }
  if (e != hipSuccess) return e;
  if ((e = record_event(ev, 2, st)) != hipSuccess) return e;
  switch (p.a.D) {
    case 64: e = launch_finalize<64>(p, st); break;
    case 96: e = launch_finalize<96>(p, st); break;
    case 128: e = launch_finalize<128>(p, st); break;
    default: return hipErrorInvalidValue;
  }
  if (e != hipSuccess) return e;
  return record_event(ev, 3, st);
}

}  // namespace neox
