// Forward attention on gfx950, bf16 storage, bf16 MFMA with fp32 accumulation.
//
// Tiled, IO-aware exact attention (the FlashAttention-2 form the GPT-NeoX pages
// name in "GPT-NeoX 开源训练框架深度解读", section "问题二：注意力计算太慢"):
// each workgroup owns 128 query rows of one (batch, head); it streams K/V in
// tiles of 64 keys through LDS, keeps a running row max and row sum (online
// softmax) in registers, and never materialises the S x S score matrix.  The
// NeoX rotary rotation of Q and K ("FasterTransformer GPT-NeoX 推理指南",
// neox_rotary_style_ / rotary_embedding) is applied while the rows are loaded.
//
// Layout choices (one wave = 64 lanes = 32 queries):
//  * Scores are computed transposed, S^T = K~ Q~^T, with v_mfma_f32_32x32x16_bf16:
//    A = K~ rows from LDS, B = Q~ held in registers for the whole loop.  The
//    accumulator gives lane l the scores of query l%32 against 16 keys per
//    32-key block, so the row max / row sum need only one cross-lane step
//    (lanes l and l^32) instead of a 32-lane reduction.
//  * O is accumulated transposed, O^T += V^T P^T: A = V^T from LDS (V is stored
//    transposed, with keys reordered inside groups of 16 so that the score
//    accumulator registers are directly the B operand), B = P in registers.
//    Each lane then owns one query row of O, so the online-softmax rescale is
//    a per-lane multiply.
//  * Workgroups are issued heaviest q-tile first; consecutive workgroup ids
//    walk over heads, so with B*H a multiple of 8 every q-tile of a head lands
//    on the same XCD (ids are dealt to the 8 XCDs round-robin) and shares its
//    K/V through that XCD's L2.
#include "device_common.hpp"

namespace neox {
namespace {

constexpr int BM = 128;      // query rows per workgroup (4 waves x 32)
constexpr int BN = 64;       // keys per tile
constexpr int NT = 256;      // threads per workgroup
constexpr int PAD = 8;       // bf16 padding per LDS row

template <int D, int ROT>
__global__ __launch_bounds__(NT, 2) void fwd_bf16_kernel(FwdParams p) {
  constexpr int KS = D + PAD;   // K~ tile row stride (elements)
  constexpr int VS = BN + PAD;  // V^T tile row stride
  __shared__ __attribute__((aligned(16))) uint16_t Ks[BN * KS];
  __shared__ __attribute__((aligned(16))) uint16_t Vt[D * VS];

  const AttnShape& a = p.a;
  const int S = a.S;
  const int nqt = (S + BM - 1) / BM;
  const int BH = a.B * a.H;
  const int qt = nqt - 1 - (int)(blockIdx.x / BH);
  const int bh = (int)(blockIdx.x % BH);
  const int b = bh / a.H, h = bh % a.H;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int ql = lane & 31, hh = lane >> 5;
  const int q0 = qt * BM;
  const int qi = q0 + wave * 32 + ql;  // this lane's query row

  const uint16_t* qb = (const uint16_t*)p.q + b * p.sq.b + h * p.sq.h;
  const uint16_t* kb = (const uint16_t*)p.k + b * p.sk.b + h * p.sk.h;
  const uint16_t* vb = (const uint16_t*)p.v + b * p.sv.b + h * p.sv.h;

  // Allowed keys of this lane's query: [lo, hi].
  const int32_t* drow = a.docs ? a.docs + (int64_t)b * (a.n_docs + 1) : nullptr;
  const int qc = qi < S ? qi : S - 1;
  int lo = 0, hi = S - 1;
  if (drow) {
    int ds, de;
    doc_bounds(drow, a.n_docs, S, qc, ds, de);
    lo = ds;
    hi = de - 1;
  }
  if (a.causal && qi < hi) hi = qi;
  // Keys any query of the workgroup may see.
  const int qlast = (q0 + BM - 1 < S - 1) ? q0 + BM - 1 : S - 1;
  int blo = 0, bhi = S - 1;
  if (drow) {
    int s0, e0, s1, e1;
    doc_bounds(drow, a.n_docs, S, q0, s0, e0);
    doc_bounds(drow, a.n_docs, S, qlast, s1, e1);
    blo = s0;
    bhi = e1 - 1;
  }
  if (a.causal && qlast < bhi) bhi = qlast;
  const int kt_lo = blo / BN, kt_hi = bhi / BN + 1;

  // Q~ of this lane's row as the B operand: chunk c holds dims 16c + 8hh .. +7.
  bf16x8 qreg[D / 16];
  {
    const uint16_t* qrow = qb + (int64_t)qc * p.sq.s;
#pragma unroll
    for (int c = 0; c < D / 16; ++c) {
      const int d0 = 16 * c + 8 * hh;
      float x[8];
      if (qi < S) {
        const u32x4 w = *reinterpret_cast<const u32x4*>(qrow + d0);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          x[2 * e] = bf_lo(w[e]);
          x[2 * e + 1] = bf_hi(w[e]);
        }
        if (ROT != 0) rotate8_scalar(qrow, d0, x, qi, a.rd, a.rope);
      } else {
#pragma unroll
        for (int e = 0; e < 8; ++e) x[e] = 0.0f;
      }
      qreg[c] = pack8(x);
    }
  }

  const float sl2 = a.alibi ? alibi_slope_log2(a, h) : 0.0f;
  const float c2 = a.scale_log2;
  float m_run = -INFINITY, l_run = 0.0f;
  f32x16 oacc[D / 32];
#pragma unroll
  for (int db = 0; db < D / 32; ++db) oacc[db] = f32x16{};

  for (int kt = kt_lo; kt < kt_hi; ++kt) {
    const int k0 = kt * BN;
    __syncthreads();
    load_tile<D, ROT, BN, NT, true, false, false>(kb, p.sk.s, k0, S, a.rd, a.rope, Ks, KS,
                                                  nullptr, 0, tid);
    load_tile<D, 0, BN, NT, false, true, true>(vb, p.sv.s, k0, S, 0, nullptr, nullptr, 0, Vt,
                                               VS, tid);
    __syncthreads();

    const bool lane_any = (k0 <= hi) && (k0 + BN - 1 >= lo);
    if (!__any(lane_any)) continue;
    const bool lane_full = (k0 >= lo) && (k0 + BN - 1 <= hi);
    const bool need_mask = !__all(lane_full);

    f32x16 sacc[2] = {f32x16{}, f32x16{}};
#pragma unroll
    for (int c = 0; c < D / 16; ++c) {
      const bf16x8 ka0 = lds_read8(Ks + ql * KS + 16 * c + 8 * hh);
      const bf16x8 ka1 = lds_read8(Ks + (32 + ql) * KS + 16 * c + 8 * hh);
      sacc[0] = mfma32x32x16(ka0, qreg[c], sacc[0]);
      sacc[1] = mfma32x32x16(ka1, qreg[c], sacc[1]);
    }

    // Scores in the log2 domain; key of register r of block blk:
    // k0 + 32 blk + 8 (r/4) + 4 hh + r%4.
    float t[32];
    const float abase = sl2 * (float)(k0 + 4 * hh - qi);
#pragma unroll
    for (int blk = 0; blk < 2; ++blk) {
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int koff = 32 * blk + 8 * (r >> 2) + (r & 3);
        float x = sacc[blk][r] * c2;
        if (a.alibi) x += abase + sl2 * (float)koff;
        if (need_mask) {
          const int j = k0 + 4 * hh + koff;
          if (j < lo || j > hi) x = -INFINITY;
        }
        t[16 * blk + r] = x;
      }
    }
    float mloc = t[0];
#pragma unroll
    for (int i = 1; i < 32; ++i) mloc = fmaxf(mloc, t[i]);
    mloc = fmaxf(mloc, __shfl_xor(mloc, 32));
    const float m_new = fmaxf(m_run, mloc);
    const float m_use = (m_new == -INFINITY) ? 0.0f : m_new;
    const float alpha = fast_exp2(m_run - m_use);
    float psum = 0.0f;
#pragma unroll
    for (int i = 0; i < 32; ++i) {
      t[i] = fast_exp2(t[i] - m_use);
      psum += t[i];
    }
    l_run = l_run * alpha + psum;
    m_run = m_new;
#pragma unroll
    for (int db = 0; db < D / 32; ++db) oacc[db] *= alpha;

#pragma unroll
    for (int cp = 0; cp < BN / 16; ++cp) {
      const bf16x8 pb = pack8(t + 16 * (cp >> 1) + 8 * (cp & 1));
#pragma unroll
      for (int db = 0; db < D / 32; ++db) {
        const bf16x8 va = lds_read8(Vt + (32 * db + ql) * VS + 16 * cp + 8 * hh);
        oacc[db] = mfma32x32x16(va, pb, oacc[db]);
      }
    }
  }

  // Epilogue: o = O / l, lse = (m + log2 l) ln 2.
  const float l_tot = l_run + __shfl_xor(l_run, 32);
  const float inv_l = l_tot > 0.0f ? 1.0f / l_tot : 0.0f;
  if (qi < S) {
    if (hh == 0) p.lse[(int64_t)bh * S + qi] = (m_run + __log2f(l_tot)) * kLn2;
    // Register r of block db holds dim 32 db + 8 (r/4) + 4 hh + r%4.
    if (p.out_f32) {
      float* orow = (float*)p.o + b * p.so.b + h * p.so.h + (int64_t)qi * p.so.s;
#pragma unroll
      for (int db = 0; db < D / 32; ++db)
#pragma unroll
        for (int a4 = 0; a4 < 4; ++a4) {
          f32x4 w;
#pragma unroll
          for (int e = 0; e < 4; ++e) w[e] = oacc[db][4 * a4 + e] * inv_l;
          *reinterpret_cast<f32x4*>(orow + 32 * db + 8 * a4 + 4 * hh) = w;
        }
    } else {
      uint16_t* orow = (uint16_t*)p.o + b * p.so.b + h * p.so.h + (int64_t)qi * p.so.s;
#pragma unroll
      for (int db = 0; db < D / 32; ++db)
#pragma unroll
        for (int a4 = 0; a4 < 4; ++a4) {
          u32x2 w;
          w[0] = pack2(oacc[db][4 * a4] * inv_l, oacc[db][4 * a4 + 1] * inv_l);
          w[1] = pack2(oacc[db][4 * a4 + 2] * inv_l, oacc[db][4 * a4 + 3] * inv_l);
          *reinterpret_cast<u32x2*>(orow + 32 * db + 8 * a4 + 4 * hh) = w;
        }
    }
  }
}

template <int D, int ROT>
hipError_t launch_d(const FwdParams& p, hipStream_t st) {
  const int nqt = (p.a.S + BM - 1) / BM;
  const dim3 grid((unsigned)(nqt * p.a.B * p.a.H));
  hipLaunchKernelGGL((fwd_bf16_kernel<D, ROT>), grid, dim3(NT), 0, st, p);
  return hipGetLastError();
}

template <int D>
hipError_t launch_rot(const FwdParams& p, hipStream_t st) {
  if (p.a.rd == 0) return launch_d<D, 0>(p, st);
  if (p.a.rd % 8 == 0) return launch_d<D, 1>(p, st);
  return launch_d<D, 2>(p, st);
}

}  // namespace

hipError_t launch_fwd_bf16(const FwdParams& p, hipStream_t st) {
  switch (p.a.D) {
    case 64: return launch_rot<64>(p, st);
    case 96: return launch_rot<96>(p, st);
    case 128: return launch_rot<128>(p, st);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace neox
