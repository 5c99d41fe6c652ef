// Backward attention on gfx950, bf16 storage, bf16 MFMA with fp32 accumulation.
//
// Recompute-based backward of the tiled exact attention (GPT-NeoX trains with
// the FlashAttention-2 form, "GPT-NeoX 开源训练框架深度解读", section
// "问题二：注意力计算太慢"): the probabilities are rebuilt from the forward's
// row logsumexp instead of being stored, so memory stays O(S).
//
//   pre:      Delta_i = dO_i . o_i, and the fp32 dQ~ accumulator is zeroed.
//   main:     one workgroup per (batch, head, 128 keys); K~ and V stay in
//             registers/LDS while q-tiles of 64 rows stream through:
//               S = Q~ K~^T,  P = exp(S*scale - lse),  dP = dO V^T,
//               dS = P (dP - Delta) * scale,
//               dV~^T += dO^T P,   dK~^T += Q~^T dS   (registers),
//               dQ~ += dS K~                          (fp32 atomics).
//             The epilogue applies R^T (rotation by -theta) to dK~ and writes
//             dK and dV.
//   finalize: dq = R^T dQ~, cast to the output type.
//
// Orientation: S and dP use M = queries, N = keys, so each lane owns one key
// (column) and the P / dS registers are directly the B operand of the dV^T and
// dK^T products; Q~^T and dO^T are staged transposed with the query order
// permuted inside groups of 16 to match that register order.  dS is written to
// LDS once per tile for the dQ product, which needs the other orientation.
#include "device_common.hpp"

namespace neox {
namespace {

constexpr int BNK = 128;  // keys per workgroup (4 waves x 32)
constexpr int BMQ = 64;   // queries per streamed tile
constexpr int NT = 256;
constexpr int PAD = 8;

template <int D>
struct BwdSmem {
  static constexpr int QS = D + PAD;    // row-major Q~ / dO stride
  static constexpr int TS = BMQ + PAD;  // transposed Q~^T / dO^T stride
  static constexpr int SS = BNK + PAD;  // dS [query][key] stride
  static constexpr int KTS = BNK + PAD; // K~^T [dim][key] stride
  static constexpr int OFF_QS = 0;
  static constexpr int OFF_QT = OFF_QS + BMQ * QS;
  static constexpr int OFF_DOS = OFF_QT + D * TS;
  static constexpr int OFF_DOT = OFF_DOS + BMQ * QS;
  static constexpr int OFF_DSS = OFF_DOT + D * TS;
  static constexpr int OFF_KT = OFF_DSS + BMQ * SS;
  static constexpr int OFF_F = OFF_KT + D * KTS;     // fp32 area (lse2, delta)
  static constexpr int N16 = OFF_F + 2 * (2 * BMQ);  // in uint16 units
  static constexpr int FS = D + 4;                   // epilogue staging stride (floats)
  static_assert(OFF_F % 8 == 0, "fp32 area must be 16-byte aligned");
  static_assert(BNK * QS <= OFF_DOS, "K~ staging must fit in the Q~ areas");
  static_assert(BNK * FS * 2 <= N16, "epilogue staging must fit");
};

template <int D, int ROT>
__global__ __launch_bounds__(NT, 1) void bwd_bf16_kernel(BwdParams p) {
  using L = BwdSmem<D>;
  __shared__ __attribute__((aligned(16))) uint16_t smem[L::N16];
  uint16_t* Qs = smem + L::OFF_QS;
  uint16_t* Qt = smem + L::OFF_QT;
  uint16_t* dOs = smem + L::OFF_DOS;
  uint16_t* dOt = smem + L::OFF_DOT;
  uint16_t* dSs = smem + L::OFF_DSS;
  uint16_t* KtT = smem + L::OFF_KT;
  float* lse2s = reinterpret_cast<float*>(smem + L::OFF_F);
  float* dels = lse2s + BMQ;

  const AttnShape& a = p.a;
  const int S = a.S;
  const int BH = a.B * a.H;
  const int kt = (int)(blockIdx.x / BH);  // small kt = most queries: heaviest first
  const int bh = (int)(blockIdx.x % BH);
  const int b = bh / a.H, h = bh % a.H;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int ql = lane & 31, hh = lane >> 5;
  const int k0 = kt * BNK;
  const int j = k0 + 32 * wave + ql;  // this lane's key
  const int jc = j < S ? j : S - 1;

  const uint16_t* qb = (const uint16_t*)p.q + b * p.sq.b + h * p.sq.h;
  const uint16_t* kb = (const uint16_t*)p.k + b * p.sk.b + h * p.sk.h;
  const uint16_t* vb = (const uint16_t*)p.v + b * p.sv.b + h * p.sv.h;
  const uint16_t* dob = (const uint16_t*)p.dout + b * p.sdo.b + h * p.sdo.h;
  const float* lseb = p.lse + (int64_t)bh * S;
  const float* delb = p.delta + (int64_t)bh * S;
  float* dqab = p.dq_acc + (int64_t)bh * S * D;

  // Queries that may see this lane's key: [qlo, qhi].
  const int32_t* drow = a.docs ? a.docs + (int64_t)b * (a.n_docs + 1) : nullptr;
  int qlo = a.causal ? j : 0, qhi = S - 1;
  if (drow) {
    int ds, de;
    doc_bounds(drow, a.n_docs, S, jc, ds, de);
    qhi = de - 1;
    if (!a.causal) qlo = ds;
  }
  if (j >= S) qlo = S;  // no queries for keys past the end
  const int klast = (k0 + BNK - 1 < S - 1) ? k0 + BNK - 1 : S - 1;
  int bqlo = a.causal ? k0 : 0, bqhi = S - 1;
  if (drow) {
    int s0, e0, s1, e1;
    doc_bounds(drow, a.n_docs, S, k0, s0, e0);
    doc_bounds(drow, a.n_docs, S, klast, s1, e1);
    bqhi = e1 - 1;
    if (!a.causal) bqlo = s0;
  }
  const int qt_lo = bqlo / BMQ, qt_hi = bqhi / BMQ + 1;

  // Stationary K~ (rotated) and V.  K~ rows go through LDS once: row-major for
  // the per-lane B operand, transposed for the dQ product.
  load_tile<D, ROT, BNK, NT, true, true, false>(kb, p.sk.s, k0, S, a.rd, a.rope, Qs, L::QS, KtT,
                                                L::KTS, tid);
  __syncthreads();
  bf16x8 kreg[D / 16], vreg[D / 16];
#pragma unroll
  for (int c = 0; c < D / 16; ++c) {
    kreg[c] = lds_read8(Qs + (32 * wave + ql) * L::QS + 16 * c + 8 * hh);
    if (j < S) {
      vreg[c] = __builtin_bit_cast(
          bf16x8, *reinterpret_cast<const u32x4*>(vb + (int64_t)j * p.sv.s + 16 * c + 8 * hh));
    } else {
      vreg[c] = __builtin_bit_cast(bf16x8, u32x4{0u, 0u, 0u, 0u});
    }
  }
  __syncthreads();

  const float sl2 = a.alibi ? alibi_slope_log2(a, h) : 0.0f;
  const float c2 = a.scale_log2;
  const float scale = a.scale;
  f32x16 dvacc[D / 32], dkacc[D / 32];
#pragma unroll
  for (int db = 0; db < D / 32; ++db) {
    dvacc[db] = f32x16{};
    dkacc[db] = f32x16{};
  }

  for (int qt = qt_lo; qt < qt_hi; ++qt) {
    const int q0 = qt * BMQ;
    load_tile<D, ROT, BMQ, NT, true, true, true>(qb, p.sq.s, q0, S, a.rd, a.rope, Qs, L::QS, Qt,
                                                 L::TS, tid);
    load_tile<D, 0, BMQ, NT, true, true, true>(dob, p.sdo.s, q0, S, 0, nullptr, dOs, L::QS, dOt,
                                               L::TS, tid);
    if (tid < BMQ) {
      const int i = q0 + tid;
      lse2s[tid] = i < S ? lseb[i] * kLog2e : INFINITY;
      dels[tid] = i < S ? delb[i] : 0.0f;
    }
    __syncthreads();

    const bool lane_any = (q0 + BMQ - 1 >= qlo) && (q0 <= qhi);
    if (__any(lane_any)) {
      const bool lane_full = (q0 >= qlo) && (q0 + BMQ - 1 <= qhi);
      const bool need_mask = !__all(lane_full);
      f32x16 sacc[2] = {f32x16{}, f32x16{}};
      f32x16 dpacc[2] = {f32x16{}, f32x16{}};
#pragma unroll
      for (int c = 0; c < D / 16; ++c) {
#pragma unroll
        for (int qb2 = 0; qb2 < 2; ++qb2) {
          const bf16x8 qa = lds_read8(Qs + (32 * qb2 + ql) * L::QS + 16 * c + 8 * hh);
          const bf16x8 da = lds_read8(dOs + (32 * qb2 + ql) * L::QS + 16 * c + 8 * hh);
          sacc[qb2] = mfma32x32x16(qa, kreg[c], sacc[qb2]);
          dpacc[qb2] = mfma32x32x16(da, vreg[c], dpacc[qb2]);
        }
      }
      // P and dS; register r of block qb2 is query q0 + 32 qb2 + 8 (r/4) + 4 hh + r%4.
      float pv[32], dsv[32];
#pragma unroll
      for (int qb2 = 0; qb2 < 2; ++qb2) {
#pragma unroll
        for (int a4 = 0; a4 < 4; ++a4) {
          const int ioff = 32 * qb2 + 8 * a4 + 4 * hh;
          const f32x4 l4 = *reinterpret_cast<const f32x4*>(lse2s + ioff);
          const f32x4 d4 = *reinterpret_cast<const f32x4*>(dels + ioff);
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const int r = 4 * a4 + e;
            const int i = q0 + ioff + e;
            float x = sacc[qb2][r] * c2 - l4[e];
            if (a.alibi) x += sl2 * (float)(j - i);
            float pr = fast_exp2(x);
            if (need_mask && (i < qlo || i > qhi)) pr = 0.0f;
            pv[16 * qb2 + r] = pr;
            dsv[16 * qb2 + r] = pr * (dpacc[qb2][r] - d4[e]) * scale;
          }
        }
      }
#pragma unroll
      for (int qc = 0; qc < BMQ / 16; ++qc) {
        const int base = 16 * (qc >> 1) + 8 * (qc & 1);
        const bf16x8 pb = pack8(pv + base);
        const bf16x8 sb = pack8(dsv + base);
#pragma unroll
        for (int db = 0; db < D / 32; ++db) {
          const bf16x8 doa = lds_read8(dOt + (32 * db + ql) * L::TS + 16 * qc + 8 * hh);
          const bf16x8 qta = lds_read8(Qt + (32 * db + ql) * L::TS + 16 * qc + 8 * hh);
          dvacc[db] = mfma32x32x16(doa, pb, dvacc[db]);
          dkacc[db] = mfma32x32x16(qta, sb, dkacc[db]);
        }
        // dS to LDS as [query][key] for the dQ product (same bf16 values).
        const u32x4 w = __builtin_bit_cast(u32x4, sb);
#pragma unroll
        for (int s = 0; s < 8; ++s) {
          const int r = 8 * (qc & 1) + s;
          const int row = 32 * (qc >> 1) + 8 * (r >> 2) + 4 * hh + (r & 3);
          const uint32_t word = w[s >> 1];
          dSs[row * L::SS + 32 * wave + ql] = (uint16_t)((s & 1) ? (word >> 16) : (word & 0xffffu));
        }
      }
    } else {
#pragma unroll
      for (int rr = 0; rr < 32; ++rr) dSs[(32 * hh + rr) * L::SS + 32 * wave + ql] = 0;
    }
    __syncthreads();

    // dQ~ += dS K~ for this tile: units of 32 queries x 32 dims over all 128 keys.
    for (int u = wave; u < (D / 32) * (BMQ / 32); u += NT / 64) {
      const int db = u % (D / 32), qb2 = u / (D / 32);
      f32x16 acc = f32x16{};
#pragma unroll
      for (int kc = 0; kc < BNK / 16; ++kc) {
        const bf16x8 sa = lds_read8(dSs + (32 * qb2 + ql) * L::SS + 16 * kc + 8 * hh);
        const bf16x8 kt2 = lds_read8(KtT + (32 * db + ql) * L::KTS + 16 * kc + 8 * hh);
        acc = mfma32x32x16(sa, kt2, acc);
      }
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int i = q0 + 32 * qb2 + 8 * (r >> 2) + 4 * hh + (r & 3);
        if (i < S) unsafeAtomicAdd(dqab + (int64_t)i * D + 32 * db + ql, acc[r]);
      }
    }
    __syncthreads();
  }

  // Epilogue: stage dK~ and dV (fp32) by key row, then write rows coalesced.
  float* stage = reinterpret_cast<float*>(smem);
  const int half = a.rd >> 1;
#pragma unroll 1
  for (int pass = 0; pass < 2; ++pass) {
#pragma unroll
    for (int db = 0; db < D / 32; ++db)
#pragma unroll
      for (int a4 = 0; a4 < 4; ++a4) {
        f32x4 w;
#pragma unroll
        for (int e = 0; e < 4; ++e) w[e] = pass == 0 ? dkacc[db][4 * a4 + e] : dvacc[db][4 * a4 + e];
        *reinterpret_cast<f32x4*>(stage + (32 * wave + ql) * L::FS + 32 * db + 8 * a4 + 4 * hh) = w;
      }
    __syncthreads();
    void* outp = pass == 0 ? p.dk : p.dv;
    const Strides so = pass == 0 ? p.sdk : p.sdv;
    for (int it = tid; it < BNK * (D / 8); it += NT) {
      const int row = it / (D / 8), d0 = 8 * (it % (D / 8));
      const int jj = k0 + row;
      if (jj >= S) continue;
      const float* srow = stage + row * L::FS;
      float x[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int d = d0 + e;
        float y = srow[d];
        if (pass == 0 && d < a.rd) {
          const bool first = d < half;
          const float2 cs = a.rope[(int64_t)jj * half + (first ? d : d - half)];
          const float xp = srow[first ? d + half : d - half];
          y = first ? (y * cs.x + xp * cs.y) : (y * cs.x - xp * cs.y);
        }
        x[e] = y;
      }
      if (p.out_f32) {
        float* orow = (float*)outp + b * so.b + h * so.h + (int64_t)jj * so.s + d0;
        *reinterpret_cast<f32x4*>(orow) = f32x4{x[0], x[1], x[2], x[3]};
        *reinterpret_cast<f32x4*>(orow + 4) = f32x4{x[4], x[5], x[6], x[7]};
      } else {
        uint16_t* orow = (uint16_t*)outp + b * so.b + h * so.h + (int64_t)jj * so.s + d0;
        *reinterpret_cast<u32x4*>(orow) =
            u32x4{pack2(x[0], x[1]), pack2(x[2], x[3]), pack2(x[4], x[5]), pack2(x[6], x[7])};
      }
    }
    __syncthreads();
  }
}

// Delta_i = dO_i . o_i (fp32) and zeroing of the dQ~ accumulator; 16 lanes per row.
template <int D, bool F32>
__global__ __launch_bounds__(256) void bwd_pre_kernel(BwdParams p) {
  const int S = p.a.S;
  const int64_t rows = (int64_t)p.a.B * p.a.H * S;
  const int64_t r = (int64_t)blockIdx.x * 16 + (threadIdx.x >> 4);
  const int l16 = threadIdx.x & 15;
  if (r >= rows) return;
  const int bh = (int)(r / S), i = (int)(r % S);
  const int b = bh / p.a.H, h = bh % p.a.H;
  float sum = 0.0f;
  if (l16 < D / 8) {
    const int d0 = 8 * l16;
    if (F32) {
      const float* orow = (const float*)p.o + b * p.so.b + h * p.so.h + (int64_t)i * p.so.s + d0;
      const float* grow = (const float*)p.dout + b * p.sdo.b + h * p.sdo.h + (int64_t)i * p.sdo.s + d0;
#pragma unroll
      for (int e = 0; e < 8; ++e) sum = fmaf(orow[e], grow[e], sum);
    } else {
      const uint16_t* orow = (const uint16_t*)p.o + b * p.so.b + h * p.so.h + (int64_t)i * p.so.s + d0;
      const uint16_t* grow =
          (const uint16_t*)p.dout + b * p.sdo.b + h * p.sdo.h + (int64_t)i * p.sdo.s + d0;
      const u32x4 ow = *reinterpret_cast<const u32x4*>(orow);
      const u32x4 gw = *reinterpret_cast<const u32x4*>(grow);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        sum = fmaf(bf_lo(ow[e]), bf_lo(gw[e]), sum);
        sum = fmaf(bf_hi(ow[e]), bf_hi(gw[e]), sum);
      }
    }
    float* acc = p.dq_acc + r * D + d0;
    *reinterpret_cast<f32x4*>(acc) = f32x4{0.f, 0.f, 0.f, 0.f};
    *reinterpret_cast<f32x4*>(acc + 4) = f32x4{0.f, 0.f, 0.f, 0.f};
  }
  sum += __shfl_xor(sum, 8, 16);
  sum += __shfl_xor(sum, 4, 16);
  sum += __shfl_xor(sum, 2, 16);
  sum += __shfl_xor(sum, 1, 16);
  if (l16 == 0) p.delta[r] = sum;
}

// dq = R^T dQ~ (rotation by -theta), cast to the output type; 8 dims per thread.
template <int D>
__global__ __launch_bounds__(256) void dq_finalize_kernel(BwdParams p, int out_f32) {
  const int S = p.a.S;
  const int64_t rows = (int64_t)p.a.B * p.a.H * S;
  const int64_t it = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (it >= rows * (D / 8)) return;
  const int64_t r = it / (D / 8);
  const int d0 = 8 * (int)(it % (D / 8));
  const int bh = (int)(r / S), i = (int)(r % S);
  const int b = bh / p.a.H, h = bh % p.a.H;
  const float* acc = p.dq_acc + r * D;
  const int rd = p.a.rd, half = rd >> 1;
  float x[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    const int d = d0 + e;
    float y = acc[d];
    if (d < rd) {
      const bool first = d < half;
      const float2 cs = p.a.rope[(int64_t)i * half + (first ? d : d - half)];
      const float xp = acc[first ? d + half : d - half];
      y = first ? (y * cs.x + xp * cs.y) : (y * cs.x - xp * cs.y);
    }
    x[e] = y;
  }
  if (out_f32) {
    float* orow = (float*)p.dq + b * p.sdq.b + h * p.sdq.h + (int64_t)i * p.sdq.s + d0;
    *reinterpret_cast<f32x4*>(orow) = f32x4{x[0], x[1], x[2], x[3]};
    *reinterpret_cast<f32x4*>(orow + 4) = f32x4{x[4], x[5], x[6], x[7]};
  } else {
    uint16_t* orow = (uint16_t*)p.dq + b * p.sdq.b + h * p.sdq.h + (int64_t)i * p.sdq.s + d0;
    *reinterpret_cast<u32x4*>(orow) =
        u32x4{pack2(x[0], x[1]), pack2(x[2], x[3]), pack2(x[4], x[5]), pack2(x[6], x[7])};
  }
}

template <int D, int ROT>
hipError_t launch_main(const BwdParams& p, hipStream_t st) {
  const int nkt = (p.a.S + BNK - 1) / BNK;
  hipLaunchKernelGGL((bwd_bf16_kernel<D, ROT>), dim3((unsigned)(nkt * p.a.B * p.a.H)), dim3(NT), 0,
                     st, p);
  return hipGetLastError();
}

template <int D>
hipError_t launch_main_rot(const BwdParams& p, hipStream_t st) {
  if (p.a.rd == 0) return launch_main<D, 0>(p, st);
  if (p.a.rd % 8 == 0) return launch_main<D, 1>(p, st);
  return launch_main<D, 2>(p, st);
}

}  // namespace

hipError_t launch_bwd_bf16(const BwdParams& p, hipStream_t st, const hipEvent_t* ev) {
  hipError_t e;
  if ((e = record_event(ev, 0, st)) != hipSuccess) return e;
  if ((e = launch_bwd_pre(p, st, false)) != hipSuccess) return e;
  if ((e = record_event(ev, 1, st)) != hipSuccess) return e;
  switch (p.a.D) {
    case 64: e = launch_main_rot<64>(p, st); break;
    case 96: e = launch_main_rot<96>(p, st); break;
    case 128: e = launch_main_rot<128>(p, st); break;
    default: return hipErrorInvalidValue;
  }
  if (e != hipSuccess) return e;
  if ((e = record_event(ev, 2, st)) != hipSuccess) return e;
  if ((e = launch_dq_finalize(p, st, p.out_f32)) != hipSuccess) return e;
  return record_event(ev, 3, st);
}

// fp32 storage shares the preprocess and finalize kernels (see bwd_f32.hip).
hipError_t launch_bwd_pre(const BwdParams& p, hipStream_t st, bool f32) {
  const int64_t rows = (int64_t)p.a.B * p.a.H * p.a.S;
  const dim3 grid((unsigned)((rows + 15) / 16));
  switch (p.a.D) {
    case 64:
      if (f32) hipLaunchKernelGGL((bwd_pre_kernel<64, true>), grid, dim3(256), 0, st, p);
      else hipLaunchKernelGGL((bwd_pre_kernel<64, false>), grid, dim3(256), 0, st, p);
      break;
    case 96:
      if (f32) hipLaunchKernelGGL((bwd_pre_kernel<96, true>), grid, dim3(256), 0, st, p);
      else hipLaunchKernelGGL((bwd_pre_kernel<96, false>), grid, dim3(256), 0, st, p);
      break;
    case 128:
      if (f32) hipLaunchKernelGGL((bwd_pre_kernel<128, true>), grid, dim3(256), 0, st, p);
      else hipLaunchKernelGGL((bwd_pre_kernel<128, false>), grid, dim3(256), 0, st, p);
      break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_dq_finalize(const BwdParams& p, hipStream_t st, int out_f32) {
  const int64_t items = (int64_t)p.a.B * p.a.H * p.a.S * (p.a.D / 8);
  const dim3 grid((unsigned)((items + 255) / 256));
  switch (p.a.D) {
    case 64: hipLaunchKernelGGL((dq_finalize_kernel<64>), grid, dim3(256), 0, st, p, out_f32); break;
    case 96: hipLaunchKernelGGL((dq_finalize_kernel<96>), grid, dim3(256), 0, st, p, out_f32); break;
    case 128: hipLaunchKernelGGL((dq_finalize_kernel<128>), grid, dim3(256), 0, st, p, out_f32); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace neox
