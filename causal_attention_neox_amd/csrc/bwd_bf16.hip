// Backward attention on gfx950, bf16 storage, bf16 MFMA with fp32 accumulation.
//
// Recompute-based backward of the tiled exact attention (GPT-NeoX trains with
// the FlashAttention-2 form, "GPT-NeoX 开源训练框架深度解读", section
// "问题二：注意力计算太慢"): probabilities are rebuilt from the forward's row
// logsumexp instead of being stored, so memory stays O(S).
//
//   prep:     per row, Delta_i = dO_i . o_i, nlse_i = -lse_i log2(e) (with the
//             ALiBi row term folded in), the fp32 dQ~ accumulator zeroed, and
//             the rotated rows q~ = R q, k~ = R k written once to the workspace
//             (NeoX rotate-half, "FasterTransformer GPT-NeoX 推理指南"), so the
//             main loop never rotates.
//   main:     one workgroup per (batch, head, 128 keys); K~ and V stay in
//             registers (and K~ in LDS) while q-tiles of 64 rows stream through:
//               S = Q~ K~^T,  P = exp2(S scale log2e + nlse),  dP = dO V^T,
//               dS = P (dP - Delta) scale,
//               dV^T += dO^T P,   dK~^T += Q~^T dS   (registers),
//               dQ~ += dS K~                       (fp32 atomics, coalesced).
//             The epilogue applies R^T (rotation by -theta) to dK~ and writes
//             dK and dV.
//   finalize: dq = R^T dQ~, cast to the output type.
//
// Orientation: S and dP use M = queries, N = keys, so each lane owns one key
// and P / dS are directly the B operands of the dV^T and dK~^T products.  The
// transposed operands (dO^T, Q~^T, dS^T, K~^T) come from row-major LDS tiles
// through ds_read_b64_tr_b16.  Q~ and dO tiles go global -> LDS directly
// (global_load_lds_dwordx4), double buffered with dS, one barrier per tile.
#include "device_common.hpp"

namespace neox {
namespace {

constexpr int BNK = 128;  // keys per workgroup (4 waves x 32)
constexpr int NT = 256;
// Queries per streamed tile: 64, or 32 at D = 128 where the stationary
// operands and accumulators leave less room for the score tiles.
template <int D>
struct QTile {
  static constexpr int BMQ = D == 128 ? 32 : 64;
};

typedef short s16x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ s16x4 tr4(const uint16_t* p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (__attribute__((address_space(3))) s16x4*)(reinterpret_cast<uintptr_t>(p)));
}
__device__ __forceinline__ bf16x8 tr8(const uint16_t* p, int second) {
  const s16x4 a = tr4(p), b = tr4(p + second);
  return __builtin_bit_cast(bf16x8, __builtin_shufflevector(a, b, 0, 1, 2, 3, 4, 5, 6, 7));
}
__device__ __forceinline__ void load_lds16(const void* gsrc, uint16_t* lds_block) {
  __builtin_amdgcn_global_load_lds((__attribute__((address_space(1))) void*)(gsrc),
                                   (__attribute__((address_space(3))) void*)(lds_block), 16, 0, 0);
}

// LDS tiles are rows of C 16-byte chunks, unpadded; chunk c of row r sits at
// r*C + (c ^ swz(r)).  The swizzle keeps both access patterns conflict-free on
// the 64 banks: 16 B row reads (16 rows x same chunk per lane group) and the
// transposed ds_read_b64_tr_b16 reads (4 rows x 4 chunks per 32 lanes).
template <int C>
__device__ __forceinline__ int swz(int row) {
  return C == 16 ? (((row & 3) << 2) | ((row >> 2) & 3))
                 : (C == 12 ? ((row >> 2) & 3)
                            : (C == 8 ? ((((row >> 1) & 1) << 2) | ((row >> 2) & 3)) : 0));
}
template <int C>
__device__ __forceinline__ int tpos(int row, int chunk) {
  return row * C + (chunk ^ swz<C>(row));
}

// ------------------------------------------------------------------------ prep

template <int D>
__global__ __launch_bounds__(256) void bwd_prep_kernel(BwdParams p) {
  using RG = RowGroups<D>;
  constexpr int C = RG::C, G = RG::G, RPW = RG::RPW;
  __shared__ __attribute__((aligned(16))) uint16_t rowbuf[4][RPW][2][D];
  const AttnShape& a = p.a;
  const int S = a.S, rd = a.rd, half = rd >> 1;
  const int rows = a.B * a.H * S;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int g = lane & (G - 1), rw = lane / G;
  const int wrow0 = (blockIdx.x * 4 + wave) * RPW;
  if (wrow0 >= rows) return;  // whole waves only
  const int r = wrow0 + rw;
  const bool act = r < rows && g < C;
  const int bh = r / S, i = r - bh * S;
  const int b = bh / a.H, h = bh - b * a.H;
  const int d0 = 8 * g;
  const bool rot_lane = act && d0 < rd;

  u32x4 ow = u32x4{0u, 0u, 0u, 0u}, gw = ow, qw = ow, kw = ow;
  float lse = 0.0f;
  float2 cs[8];
  if (act) {
    ow = *reinterpret_cast<const u32x4*>((const uint16_t*)p.o + b * p.so.b + h * p.so.h +
                                         (int64_t)i * p.so.s + d0);
    gw = *reinterpret_cast<const u32x4*>((const uint16_t*)p.dout + b * p.sdo.b + h * p.sdo.h +
                                         (int64_t)i * p.sdo.s + d0);
    if (rd > 0) {
      qw = *reinterpret_cast<const u32x4*>((const uint16_t*)p.q + b * p.sq.b + h * p.sq.h +
                                           (int64_t)i * p.sq.s + d0);
      kw = *reinterpret_cast<const u32x4*>((const uint16_t*)p.k + b * p.sk.b + h * p.sk.h +
                                           (int64_t)i * p.sk.s + d0);
    }
    if (g == 0) lse = p.lse[r];
  }
  if (rot_lane) {
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const int d = d0 + e;
      cs[e] = d < rd ? a.rope[(int64_t)i * half + (d < half ? d : d - half)] : float2{1.0f, 0.0f};
    }
  }

  float sum = 0.0f;
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    sum = fmaf(bf_lo(ow[e]), bf_lo(gw[e]), sum);
    sum = fmaf(bf_hi(ow[e]), bf_hi(gw[e]), sum);
  }
#pragma unroll
  for (int m = G / 2; m >= 1; m >>= 1) sum += __shfl_xor(sum, m);
  if (act) {
    float* acc = p.dq_acc + (int64_t)r * D + d0;
    *reinterpret_cast<f32x4*>(acc) = f32x4{0.f, 0.f, 0.f, 0.f};
    *reinterpret_cast<f32x4*>(acc + 4) = f32x4{0.f, 0.f, 0.f, 0.f};
    if (g == 0) {
      p.delta[r] = sum;
      float nl = -lse * kLog2e;
      if (a.alibi) nl -= alibi_slope_log2(a, h) * (float)i;
      p.nlse[r] = nl;
    }
  }
  if (rd == 0) return;

  if (act) {
    *reinterpret_cast<u32x4*>(&rowbuf[wave][rw][0][d0]) = qw;
    *reinterpret_cast<u32x4*>(&rowbuf[wave][rw][1][d0]) = kw;
  }
  lds_wave_sync();
  if (rot_lane) {
    float xq[8], xk[8];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      xq[2 * e] = bf_lo(qw[e]);
      xq[2 * e + 1] = bf_hi(qw[e]);
      xk[2 * e] = bf_lo(kw[e]);
      xk[2 * e + 1] = bf_hi(kw[e]);
    }
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const int d = d0 + e;
      if (d < rd) {
        const bool first = d < half;
        const int pd = first ? d + half : d - half;
        const float sn = first ? -cs[e].y : cs[e].y;  // rotate-half: (-x2, x1)
        xq[e] = fmaf(bf2f(rowbuf[wave][rw][0][pd]), sn, xq[e] * cs[e].x);
        xk[e] = fmaf(bf2f(rowbuf[wave][rw][1][pd]), sn, xk[e] * cs[e].x);
      }
    }
    qw = u32x4{pack2(xq[0], xq[1]), pack2(xq[2], xq[3]), pack2(xq[4], xq[5]), pack2(xq[6], xq[7])};
    kw = u32x4{pack2(xk[0], xk[1]), pack2(xk[2], xk[3]), pack2(xk[4], xk[5]), pack2(xk[6], xk[7])};
  }
  if (act) {
    *reinterpret_cast<u32x4*>(p.qrot + (int64_t)r * D + d0) = qw;
    *reinterpret_cast<u32x4*>(p.krot + (int64_t)r * D + d0) = kw;
  }
}

// ------------------------------------------------------------------------ main

template <int D>
struct BwdLds {
  static constexpr int BMQ = QTile<D>::BMQ;
  static constexpr int C = D / 8;
  static constexpr int KT = 0;                   // K~ [BNK][D]
  static constexpr int Q0 = KT + BNK * D;        // Q~ tiles [BMQ][D] x2
  static constexpr int G0 = Q0 + 2 * BMQ * D;    // dO tiles x2
  static constexpr int DS0 = G0 + 2 * BMQ * D;   // dS tiles [BNK][BMQ] x2 (rows of BMQ/8 chunks)
  static constexpr int F0 = DS0 + 2 * BNK * BMQ; // floats: nlse x2, Delta x2 (BMQ each)
  static constexpr int N16 = F0 + 2 * 4 * BMQ;   // total in uint16 units
  static_assert((F0 * 2) % 16 == 0, "float area alignment");
};

template <int D, bool ALIBI>
__global__ __launch_bounds__(NT, 1) void bwd_main_kernel(BwdParams p) {
  using L = BwdLds<D>;
  constexpr int BMQ = L::BMQ;
  constexpr int QB = BMQ / 32;   // 32-query blocks per tile
  constexpr int CS = BMQ / 8;    // 16-byte chunks per dS row
  constexpr int C = L::C;
  constexpr int NB = D / 32;
  __shared__ __attribute__((aligned(16))) uint16_t lds[L::N16];
  float* fl = reinterpret_cast<float*>(lds + L::F0);  // nlse[2][BMQ], delta[2][BMQ]

  const AttnShape& a = p.a;
  const int S = a.S;
  const int BH = a.B * a.H;
  const int kt = (int)(blockIdx.x / BH);  // small kt = most queries: heaviest first
  const int bh = (int)(blockIdx.x % BH);
  const int b = bh / a.H, h = bh % a.H;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int ql = lane & 31, hh = lane >> 5;
  const int g16 = lane >> 4, j16 = lane & 15;
  const int k0 = kt * BNK;
  const int j = k0 + 32 * wave + ql;  // this lane's key

  const bool rot = a.rd > 0;
  const uint16_t* qb = rot ? p.qrot + (int64_t)bh * S * D
                           : (const uint16_t*)p.q + b * p.sq.b + h * p.sq.h;
  const int64_t qs = rot ? D : p.sq.s;
  const uint16_t* kb = rot ? p.krot + (int64_t)bh * S * D
                           : (const uint16_t*)p.k + b * p.sk.b + h * p.sk.h;
  const int64_t ks = rot ? D : p.sk.s;
  const uint16_t* vb = (const uint16_t*)p.v + b * p.sv.b + h * p.sv.h;
  const uint16_t* gb = (const uint16_t*)p.dout + b * p.sdo.b + h * p.sdo.h;
  const float* nlb = p.nlse + (int64_t)bh * S;
  const float* dlb = p.delta + (int64_t)bh * S;
  float* dqab = p.dq_acc + (int64_t)bh * S * D;

  // Queries that may see this lane's key: [qlo, qhi].
  const int32_t* drow = a.docs ? a.docs + (int64_t)b * (a.n_docs + 1) : nullptr;
  int qlo = a.causal ? j : 0, qhi = S - 1;
  if (drow) {
    int ds, de;
    doc_bounds(drow, a.n_docs, S, j < S ? j : S - 1, ds, de);
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

  // Direct-load plans: tile position P = 64 * block + lane -> (row, chunk).
  // K~: BNK*C/64 blocks over 4 waves; Q~ and dO tiles: BMQ*C/64 = C blocks.
  constexpr int NKB = BNK * C / 64 / 4;
  constexpr int NQB = BMQ * C / 64 / 4;
  int qoff[NQB], goff[NQB];
#pragma unroll
  for (int n = 0; n < NQB; ++n) {
    const int P = 64 * (wave + 4 * n) + lane;
    const int row = P / C, ch = (P % C) ^ swz<C>(row);
    qoff[n] = (int)(row * qs) + 8 * ch;
    goff[n] = (int)(row * p.sdo.s) + 8 * ch;
  }
  auto fetch_q = [&](int qt, int buf) {
    const int q0 = qt * BMQ;
    uint16_t* Qt = lds + L::Q0 + buf * BMQ * D;
    uint16_t* Gt = lds + L::G0 + buf * BMQ * D;
    if (q0 + BMQ <= S) {
      const uint16_t* q_t = qb + (int64_t)q0 * qs;
      const uint16_t* g_t = gb + (int64_t)q0 * p.sdo.s;
#pragma unroll
      for (int n = 0; n < NQB; ++n) {
        load_lds16(q_t + qoff[n], Qt + 512 * (wave + 4 * n));
        load_lds16(g_t + goff[n], Gt + 512 * (wave + 4 * n));
      }
      if ((S & 3) == 0) {  // rows of nlse / Delta start 16-byte aligned
        if (wave == 0 && lane < BMQ / 4)
          load_lds16(nlb + q0 + 4 * lane, lds + L::F0 + buf * 2 * BMQ);
        if (wave == 1 && lane < BMQ / 4)
          load_lds16(dlb + q0 + 4 * lane, lds + L::F0 + 4 * BMQ + buf * 2 * BMQ);
      } else if (wave < 2 && lane < BMQ / 4) {
        const float* src = wave == 0 ? nlb : dlb;
        f32x4 w;
#pragma unroll
        for (int e = 0; e < 4; ++e) w[e] = src[q0 + 4 * lane + e];
        *reinterpret_cast<f32x4*>(fl + wave * 2 * BMQ + buf * BMQ + 4 * lane) = w;
      }
    } else {
      // last tile: rows past S re-read row S-1 (their P is masked to 0)
#pragma unroll
      for (int n = 0; n < NQB; ++n) {
        const int P = 64 * (wave + 4 * n) + lane;
        const int row = P / C, ch = (P % C) ^ swz<C>(row);
        const int rr = min(q0 + row, S - 1);
        load_lds16(qb + (int64_t)rr * qs + 8 * ch, Qt + 512 * (wave + 4 * n));
        load_lds16(gb + (int64_t)rr * p.sdo.s + 8 * ch, Gt + 512 * (wave + 4 * n));
      }
      // nlse / Delta: 4 floats per lane; rows past S get 0 and are masked
      if (wave < 2 && lane < BMQ / 4) {
        const float* src = wave == 0 ? nlb : dlb;
        f32x4 w;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int ii = q0 + 4 * lane + e;
          w[e] = ii < S ? src[ii] : 0.0f;
        }
        *reinterpret_cast<f32x4*>(fl + wave * 2 * BMQ + buf * BMQ + 4 * lane) = w;
      }
    }
  };

  // Stationary K~ tile and the first q-tile.
#pragma unroll
  for (int n = 0; n < NKB; ++n) {
    const int P = 64 * (wave + 4 * n) + lane;
    const int row = P / C, ch = (P % C) ^ swz<C>(row);
    const int rr = min(k0 + row, S - 1);
    load_lds16(kb + (int64_t)rr * ks + 8 * ch, lds + L::KT + 512 * (wave + 4 * n));
  }
  fetch_q(qt_lo, 0);
  bf16x8 vreg[D / 16];
#pragma unroll
  for (int c = 0; c < D / 16; ++c) {
    vreg[c] = __builtin_bit_cast(bf16x8, u32x4{0u, 0u, 0u, 0u});
    if (j < S)
      vreg[c] = __builtin_bit_cast(
          bf16x8, *reinterpret_cast<const u32x4*>(vb + (int64_t)j * p.sv.s + 16 * c + 8 * hh));
  }
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  bf16x8 kreg[D / 16];
  {
    const int row = 32 * wave + ql;
#pragma unroll
    for (int c = 0; c < D / 16; ++c) kreg[c] = lds_read8(lds + L::KT + 8 * tpos<C>(row, 2 * c + hh));
  }

  // Per-lane LDS offsets (elements) of the row reads and transposed reads.
  // Row reads (A of S and dP): row 32 qb + ql, chunk 2c + hh.
  const int rsw = swz<C>(ql);  // rows ql and 32 + ql share the swizzle
  // Transposed reads of a [rows][C chunks] tile: lane 16g + j16 supplies row
  // 16 t + 4 hh + j16/4 (+8 for the second read), 4 columns at chunk
  // 4 db + 2 (g&1) + (j16&3)/2, half (j16&1).
  const int trow = 4 * hh + (j16 >> 2);
  const int tch = 2 * (g16 & 1) + ((j16 & 3) >> 1);
  const int thalf = 4 * (j16 & 1);
  int taddr[2][NB];  // [second read][dim block] element offsets within a [*][D] tile
#pragma unroll
  for (int s2 = 0; s2 < 2; ++s2)
#pragma unroll
    for (int db = 0; db < NB; ++db)
      taddr[s2][db] = 8 * ((trow + 8 * s2) * C + ((4 * db + tch) ^ swz<C>(trow + 8 * s2))) + thalf;
  // dS tiles: [BNK keys][BMQ queries] rows of CS chunks.  dQ A operand:
  // supplier lane reads key row 16 kc + 8 hh + j16/4 (+4), queries at chunk
  // 4 qb + 2 (g&1) + (j16&3)/2.
  const int srow = 8 * hh + (j16 >> 2);
  int saddr[2][QB];  // [second read (+4 keys)][qb]
#pragma unroll
  for (int s2 = 0; s2 < 2; ++s2)
#pragma unroll
    for (int qb2 = 0; qb2 < QB; ++qb2)
      saddr[s2][qb2] =
          8 * ((srow + 4 * s2) * CS + ((4 * qb2 + tch) ^ swz<CS>(srow + 4 * s2))) + thalf;
  // dQ B operand (K~ transposed): key row 16 kc + 8 hh + j16/4 (+4), dims at
  // chunk 4 db + 2 (g&1) + (j16&3)/2.
  int kaddr[2];  // [second read] for this wave's dim block (db = wave)
#pragma unroll
  for (int s2 = 0; s2 < 2; ++s2)
    kaddr[s2] = 8 * ((srow + 4 * s2) * C + ((4 * (wave < NB ? wave : 0) + tch) ^ swz<C>(srow + 4 * s2))) + thalf;
  // dS write: this lane's key row (32 wave + ql), 4 queries 32 qb + 8 a4 + 4 hh.
  const int wrow = 32 * wave + ql;
  const int wsw = swz<CS>(wrow);

  const float c2 = a.scale_log2;
  const float scale = a.scale;
  const float slj = ALIBI ? alibi_slope_log2(a, h) * (float)j : 0.0f;
  f32x16 dvacc[NB], dkacc[NB];
#pragma unroll
  for (int db = 0; db < NB; ++db) {
    dvacc[db] = f32x16{};
    dkacc[db] = f32x16{};
  }

  for (int qt = qt_lo; qt < qt_hi; ++qt) {
    const int buf = (qt - qt_lo) & 1;
    const int q0 = qt * BMQ;
    const uint16_t* Qt = lds + L::Q0 + buf * BMQ * D;
    const uint16_t* Gt = lds + L::G0 + buf * BMQ * D;
    uint16_t* DSt = lds + L::DS0 + buf * BNK * BMQ;
    const float* nlt = fl + buf * BMQ;
    const float* dlt = fl + 2 * BMQ + buf * BMQ;
    if (qt + 1 < qt_hi) fetch_q(qt + 1, buf ^ 1);

    // Every wave computes every tile (fully masked rows give P = dS = 0): a
    // skip branch here would split the loop-carried accumulators across paths.
    {
      const bool lane_full = (q0 >= qlo) && (q0 + BMQ - 1 <= qhi);
      const bool need_mask = !__all(lane_full);
      f32x16 sacc[QB], dpacc[QB];
#pragma unroll
      for (int qb2 = 0; qb2 < QB; ++qb2) {
        sacc[qb2] = f32x16{};
        dpacc[qb2] = f32x16{};
      }
#pragma unroll
      for (int c = 0; c < D / 16; ++c) {
#pragma unroll
        for (int qb2 = 0; qb2 < QB; ++qb2) {
          const int off = 8 * ((32 * qb2 + ql) * C + ((2 * c + hh) ^ rsw));
          sacc[qb2] = mfma32x32x16(lds_read8(Qt + off), kreg[c], sacc[qb2]);
          dpacc[qb2] = mfma32x32x16(lds_read8(Gt + off), vreg[c], dpacc[qb2]);
        }
      }
      // P and dS in place; register r of block qb2 is query
      // q0 + 32 qb2 + 8 (r/4) + 4 hh + r%4.
#pragma unroll
      for (int qb2 = 0; qb2 < QB; ++qb2) {
#pragma unroll
        for (int a4 = 0; a4 < 4; ++a4) {
          const int ioff = 32 * qb2 + 8 * a4 + 4 * hh;
          const f32x4 n4 = *reinterpret_cast<const f32x4*>(nlt + ioff);
          const f32x4 d4 = *reinterpret_cast<const f32x4*>(dlt + ioff);
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const int r = 4 * a4 + e;
            const float nl = ALIBI ? n4[e] + slj : n4[e];
            float pr = fast_exp2(__builtin_fmaf(sacc[qb2][r], c2, nl));
            if (need_mask) {
              const int i = q0 + ioff + e;
              if (i < qlo || i > qhi) pr = 0.0f;
            }
            sacc[qb2][r] = pr;
            dpacc[qb2][r] = pr * (dpacc[qb2][r] - d4[e]) * scale;
          }
        }
      }
#pragma unroll
      for (int qc = 0; qc < BMQ / 16; ++qc) {
        float pv[8], sv[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          pv[e] = sacc[qc >> 1][8 * (qc & 1) + e];
          sv[e] = dpacc[qc >> 1][8 * (qc & 1) + e];
        }
        const bf16x8 pb = pack8(pv);
        const bf16x8 sb = pack8(sv);
#pragma unroll
        for (int db = 0; db < NB; ++db) {
          const int off = taddr[0][db] + 16 * qc * D;
          const bf16x8 ga = tr8(Gt + off, taddr[1][db] - taddr[0][db]);
          const bf16x8 qa = tr8(Qt + off, taddr[1][db] - taddr[0][db]);
          dvacc[db] = mfma32x32x16(ga, pb, dvacc[db]);
          dkacc[db] = mfma32x32x16(qa, sb, dkacc[db]);
        }
        // dS (same bf16 values) to LDS, row = this lane's key, 4 queries each.
        const u32x4 w = __builtin_bit_cast(u32x4, sb);
#pragma unroll
        for (int hv = 0; hv < 2; ++hv) {
          const int qoff2 = 16 * qc + 8 * hv + 4 * hh;  // first query of the 4
          const int ch = qoff2 >> 3;
          *reinterpret_cast<u32x2*>(DSt + 8 * (wrow * CS + (ch ^ wsw)) + (qoff2 & 7)) =
              u32x2{w[2 * hv], w[2 * hv + 1]};
        }
        // keep the operand reads of one query chunk together (bounds register use)
        __builtin_amdgcn_sched_barrier(0);
      }
    }
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();

    // dQ~ += dS K~ for this tile: wave w < D/32 handles dims 32w..32w+31 for
    // all the tile's queries (the 32-query blocks share the K~ operand).
    if (wave < NB) {
      f32x16 acc[QB];
#pragma unroll
      for (int qb2 = 0; qb2 < QB; ++qb2) acc[qb2] = f32x16{};
#pragma unroll
      for (int kc = 0; kc < BNK / 16; ++kc) {
        const uint16_t* kt2 = lds + L::KT + kaddr[0] + 16 * kc * D;
        const bf16x8 kb8 = tr8(kt2, kaddr[1] - kaddr[0]);
#pragma unroll
        for (int qb2 = 0; qb2 < QB; ++qb2) {
          const uint16_t* sp = DSt + saddr[0][qb2] + 16 * kc * BMQ;
          const bf16x8 sa = tr8(sp, saddr[1][qb2] - saddr[0][qb2]);
          acc[qb2] = mfma32x32x16(sa, kb8, acc[qb2]);
        }
        if (kc & 1) __builtin_amdgcn_sched_barrier(0);
      }
      float* dst = dqab + (int64_t)(q0 + 4 * hh) * D + 32 * wave + ql;
      if (q0 + BMQ <= S) {
#pragma unroll
        for (int qb2 = 0; qb2 < QB; ++qb2)
#pragma unroll
          for (int r = 0; r < 16; ++r)
            unsafeAtomicAdd(dst + (32 * qb2 + 8 * (r >> 2) + (r & 3)) * D, acc[qb2][r]);
      } else {
#pragma unroll
        for (int qb2 = 0; qb2 < QB; ++qb2)
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int io = 32 * qb2 + 8 * (r >> 2) + (r & 3);
            if (q0 + 4 * hh + io < S) unsafeAtomicAdd(dst + io * D, acc[qb2][r]);
          }
      }
    }
  }

  // Epilogue: stage dK~ and dV (fp32) by key row over the (now idle) tile
  // areas, then write rows coalesced; dK = R^T dK~.
  __syncthreads();
  float* stage = reinterpret_cast<float*>(lds + L::KT);
  constexpr int FS = D + 4;
  static_assert(BNK * FS * 2 <= L::F0, "epilogue staging must fit");
  const int half = a.rd >> 1;
#pragma unroll 1
  for (int pass = 0; pass < 2; ++pass) {
#pragma unroll
    for (int db = 0; db < NB; ++db)
#pragma unroll
      for (int a4 = 0; a4 < 4; ++a4) {
        f32x4 w;
#pragma unroll
        for (int e = 0; e < 4; ++e) w[e] = pass == 0 ? dkacc[db][4 * a4 + e] : dvacc[db][4 * a4 + e];
        *reinterpret_cast<f32x4*>(stage + (32 * wave + ql) * FS + 32 * db + 8 * a4 + 4 * hh) = w;
      }
    __syncthreads();
    void* outp = pass == 0 ? p.dk : p.dv;
    const Strides so = pass == 0 ? p.sdk : p.sdv;
    for (int it = tid; it < BNK * (D / 8); it += NT) {
      const int row = it / (D / 8), d0 = 8 * (it % (D / 8));
      const int jj = k0 + row;
      if (jj >= S) continue;
      const float* srow = stage + row * FS;
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

// ------------------------------------------------------------------ finalize

// dq = R^T dQ~ (rotation by -theta), cast to the output type.  Row groups as
// in the prep pass; rotary partners are exchanged through LDS.
template <int D>
__global__ __launch_bounds__(256) void dq_finalize_kernel(BwdParams p, int out_f32) {
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

template <int D>
dim3 row_grid(const BwdParams& p) {
  const int64_t rows = (int64_t)p.a.B * p.a.H * p.a.S;
  return dim3((unsigned)((rows + RowGroups<D>::RPB - 1) / RowGroups<D>::RPB));
}

template <int D>
hipError_t launch_d(const BwdParams& p, hipStream_t st, const hipEvent_t* ev) {
  hipError_t e;
  if ((e = record_event(ev, 0, st)) != hipSuccess) return e;
  hipLaunchKernelGGL((bwd_prep_kernel<D>), row_grid<D>(p), dim3(256), 0, st, p);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  if ((e = record_event(ev, 1, st)) != hipSuccess) return e;
  const int nkt = (p.a.S + BNK - 1) / BNK;
  const dim3 grid((unsigned)(nkt * p.a.B * p.a.H));
  if (p.a.alibi)
    hipLaunchKernelGGL((bwd_main_kernel<D, true>), grid, dim3(NT), 0, st, p);
  else
    hipLaunchKernelGGL((bwd_main_kernel<D, false>), grid, dim3(NT), 0, st, p);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  if ((e = record_event(ev, 2, st)) != hipSuccess) return e;
  hipLaunchKernelGGL((dq_finalize_kernel<D>), row_grid<D>(p), dim3(256), 0, st, p, p.out_f32);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  return record_event(ev, 3, st);
}

}  // namespace

hipError_t launch_bwd_bf16(const BwdParams& p, hipStream_t st, const hipEvent_t* ev) {
  switch (p.a.D) {
    case 64: return launch_d<64>(p, st, ev);
    case 96: return launch_d<96>(p, st, ev);
    case 128: return launch_d<128>(p, st, ev);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_dq_finalize(const BwdParams& p, hipStream_t st, int out_f32) {
  switch (p.a.D) {
    case 64: hipLaunchKernelGGL((dq_finalize_kernel<64>), row_grid<64>(p), dim3(256), 0, st, p, out_f32); break;
    case 96: hipLaunchKernelGGL((dq_finalize_kernel<96>), row_grid<96>(p), dim3(256), 0, st, p, out_f32); break;
    case 128: hipLaunchKernelGGL((dq_finalize_kernel<128>), row_grid<128>(p), dim3(256), 0, st, p, out_f32); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace neox
