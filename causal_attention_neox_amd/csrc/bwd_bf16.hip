// Backward attention on gfx950, 16-bit storage (bf16; bwd_f16.hip compiles this
// file again for IEEE half), MFMA on that type with fp32 accumulation.
//
// Recompute-based backward of the tiled exact attention (GPT-NeoX trains with
// the FlashAttention-2 form, "GPT-NeoX 开源训练框架深度解读", section
// "问题二：注意力计算太慢"): probabilities are rebuilt from the forward's row
// logsumexp instead of being stored, so memory stays O(S).  Passes, in order:
//
//   prep:  the rotated rows q~ = R q, k~ = R k written once to the workspace
//          (NeoX rotate-half, "FasterTransformer GPT-NeoX 推理指南"), so the
//          other passes never rotate; skipped when the rotation is off or the
//          forward already left q~ and k~ in that workspace.
//   dQ:    one workgroup per (batch, head, 128 queries), Q-stationary.  Its
//          prologue forms the row terms Delta_i = dO_i . o_i and
//          nlse_i = -lse_i log2(e) (with the ALiBi row term folded in) and
//          writes them to the workspace (Delta negated: the dP accumulators
//          start from -Delta, so dP - Delta costs no extra step); 64-key
//          tiles stream through LDS, S and dP are recomputed, dQ~ += dS' K~
//          accumulates in registers, and the epilogue writes dq = scale R^T dQ~.
//   dK/dV: one workgroup per (batch, head, 64 keys; 128 at D = 128),
//          K-stationary; 64-row q-tiles (with their Delta and nlse) stream
//          through LDS:
//            S = Q~ K~^T,  P = exp2(S scale log2e + nlse),  dP = dO V^T,
//            dS' = P (dP - Delta),  dV^T += dO^T P,  dK~^T += Q~^T dS'.
//          The epilogue writes dV and dK = scale R^T dK~.
//
// Splitting dQ off costs two extra products (S and dP recomputed) but needs
// no fp32 atomics: accumulating dQ~ across key blocks with atomics is bound by
// the L2 atomic rate (about one 4-byte add per channel per clock), far below
// the matrix cores, and it also makes dq deterministic.
#include <type_traits>

#include "device_common.hpp"

namespace neox {
namespace NEOX_ELEM_NS {
namespace {

constexpr int NT = 256;
typedef short s16x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ s16x4 tr4(const uint16_t* p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (__attribute__((address_space(3))) s16x4*)(reinterpret_cast<uintptr_t>(p)));
}
__device__ __forceinline__ elem8 tr8(const uint16_t* p, int second) {
  const s16x4 a = tr4(p), b = tr4(p + second);
  return __builtin_bit_cast(elem8, __builtin_shufflevector(a, b, 0, 1, 2, 3, 4, 5, 6, 7));
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

// q~ = R q and k~ = R k into the workspace, one row group of G lanes per row
// (rotary partners exchanged through LDS); a wave takes one position in RPW
// heads, so the rotary table entries are loaded once for its rows.  Launched
// only when the rotation is on and the forward did not leave q~ and k~ in
// the workspace.
template <int D>
__global__ __launch_bounds__(256) void bwd_prep_kernel(BwdParams p) {
  using RG = RowGroups<D>;
  constexpr int C = RG::C, G = RG::G, RPW = RG::RPW;
  __shared__ __attribute__((aligned(16))) uint16_t rowbuf[4][RPW][2][D];
  const AttnShape& a = p.a;
  const int S = a.S, rd = a.rd, half = rd >> 1;
  const int BH = a.B * a.H;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int g = lane & (G - 1), rw = lane / G;
  const int wid = blockIdx.x * 4 + wave;
  const int i = wid % S, bh0 = (wid / S) * RPW;  // position; first head of the wave
  if (bh0 >= BH) return;                          // whole waves only
  const int bh = bh0 + rw;
  const int r = bh * S + i;
  const bool act = bh < BH && g < C;
  const int b = bh / a.H, h = bh - b * a.H;
  const int d0 = 8 * g;
  const bool rot_lane = act && d0 < rd;

  u32x4 qw = u32x4{0u, 0u, 0u, 0u}, kw = qw;
  float2 cs[8];
  if (act) {
    qw = *reinterpret_cast<const u32x4*>((const uint16_t*)p.q + b * p.sq.b + h * p.sq.h +
                                         (int64_t)i * p.sq.s + d0);
    kw = *reinterpret_cast<const u32x4*>((const uint16_t*)p.k + b * p.sk.b + h * p.sk.h +
                                         (int64_t)i * p.sk.s + d0);
  }
  if (g < C && d0 < rd) rope_entries8(a.rope + (int64_t)i * half, d0, half, rd, cs);
  if (act) {
    *reinterpret_cast<u32x4*>(&rowbuf[wave][rw][0][d0]) = qw;
    *reinterpret_cast<u32x4*>(&rowbuf[wave][rw][1][d0]) = kw;
  }
  lds_wave_sync();
  if (rot_lane) {
    float xq[8], xk[8];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      xq[2 * e] = el_lo(qw[e]);
      xq[2 * e + 1] = el_hi(qw[e]);
      xk[2 * e] = el_lo(kw[e]);
      xk[2 * e + 1] = el_hi(kw[e]);
    }
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const int d = d0 + e;
      if (d < rd) {
        const bool first = d < half;
        const int pd = first ? d + half : d - half;
        const float sn = first ? -cs[e].y : cs[e].y;  // rotate-half: (-x2, x1)
        xq[e] = fmaf(el2f(rowbuf[wave][rw][0][pd]), sn, xq[e] * cs[e].x);
        xk[e] = fmaf(el2f(rowbuf[wave][rw][1][pd]), sn, xk[e] * cs[e].x);
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

// ------------------------------------------------------------------- dK / dV

// 2 KG waves, two waves per SIMD in all (KG key groups; two 4-wave
// workgroups per CU at D <= 96, one 8-wave workgroup at D = 128).  Wave w
// owns the 32 keys 32 (w % KG) .. +31 of the workgroup's 32 KG and query half
// w / KG (32 rows) of every 64-row q-tile; the two waves of a key group add
// their dV / dK~ partial sums in the epilogue.  (With 128-row q-tiles each
// wave would take two 32-row quarters of a tile between barriers, halving the
// barriers and tile loads per row; the layout keeps that form.)  K~ and V are
// the B operands of S and dP: held in registers at D = 64 (where they fit),
// else re-read from stationary LDS tiles.
constexpr int kDkdvPrefetch = 1;  // MFMA steps between an LDS operand's read and its use

template <int D>
struct DkdvLds {
  // Key groups of 32 keys per workgroup (two waves each, one per query half):
  // two at D <= 96, where the LDS of a 64-key workgroup (64-row q-tiles)
  // lets two workgroups share a CU, so that one's prologue and epilogue run
  // beside the other's q-tiles; four at D = 128 (one workgroup per CU either
  // way, and 128-key blocks halve the Q~ / dO tile loads).
  static constexpr int KG = D <= 96 ? 2 : 4;
  static constexpr int BNK = 32 * KG;   // keys per workgroup
  static constexpr int NW = 2 * KG;     // waves per workgroup
  static constexpr int NTH = 64 * NW;   // threads per workgroup
  // q-tile rows per barrier: 128 where the double-buffered tiles fit in LDS
  // (each wave then takes two 32-row quarters of a tile), else 64.
  static constexpr int BMQ = (D <= 96 && KG == 4) ? 128 : 64;
  static constexpr int NQQ = BMQ / 64;  // quarters per wave per tile
  static constexpr int C = D / 8;
  static constexpr bool kRegK = D <= 64;         // K~ B operands held in registers
  static constexpr bool kRegV = D <= 64;         // V B operands held in registers
  static constexpr int KT = 0;                   // K~ [BNK][D] (staging for the registers)
  static constexpr int VT = KT + BNK * D;        // V [BNK][D] (when not in registers)
  static constexpr int Q0 = VT + (kRegV ? 0 : BNK * D);  // Q~ tiles [BMQ][D] x2
  static constexpr int G0 = Q0 + 2 * BMQ * D;    // dO tiles x2
  static constexpr int F0 = G0 + 2 * BMQ * D;    // floats: nlse x2, Delta x2 (BMQ each)
  static constexpr int N16T = F0 + 2 * 4 * BMQ;  // tile-loop areas in uint16 units
  static constexpr int EPI_BYTES = 2 * BNK * (D + 4) * 4;  // epilogue: dK~ and dV rows in fp32
  static constexpr int N16 = N16T * 2 > EPI_BYTES ? N16T : EPI_BYTES / 2;  // LDS, uint16 units
  static_assert((F0 * 2) % 16 == 0, "float area alignment");
};
template <int D, bool ALIBI>
__global__ __launch_bounds__(DkdvLds<D>::NTH, 8 / DkdvLds<D>::NW) void bwd_dkdv_kernel(BwdParams p) {
  using L = DkdvLds<D>;
  constexpr int BNK = L::BNK, NW = L::NW, KG = L::KG, NT8 = L::NTH;
  constexpr int BMQ = L::BMQ;
  constexpr int C = L::C;
  constexpr int NB = D / 32;
  constexpr int NQQ = L::NQQ;
  constexpr int CB = C * BMQ / 64;  // 1 KB blocks of one q-tile tensor (Q~ or dO)
  constexpr int NFB = 2 * CB / NW;  // direct-load blocks per wave of a q-tile (Q~ and dO)
  constexpr int NKB = BNK * C / 64 / NW;  // direct-load blocks per wave of the stationary K~ (or V)
  static_assert((2 * CB) % NW == 0 && (BNK * C / 64) % NW == 0,
                "tile blocks must split evenly over the waves");
  constexpr bool kRegK = L::kRegK, kRegV = L::kRegV;
  __shared__ __attribute__((aligned(16))) uint16_t lds[L::N16];
  float* fl = reinterpret_cast<float*>(lds + L::F0);  // nlse[2][BMQ], delta[2][BMQ]

  const AttnShape& a = p.a;
  const int S = a.S;
  const int BH = a.B * a.H;
  int kt, bh;  // kt 0 (most queries) first; Q~ and dO of a head: 4 S D bytes
  xcd_order((S + BNK - 1) / BNK, BH, (int64_t)4 * S * D, kt, bh);
  const int b = bh / a.H, h = bh % a.H;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform (scalar)
  const int kg = wave % KG, qhalf = wave / KG;
  const int ql = lane & 31, hh = lane >> 5;
  const int g16 = lane >> 4, j16 = lane & 15;
  const int k0 = kt * BNK;
  const int j = k0 + 32 * kg + ql;  // this lane's key

  const bool rot = a.rd > 0;
  const uint16_t* qb = rot ? p.qrot + (int64_t)bh * S * D
                           : (const uint16_t*)p.q + b * p.sq.b + h * p.sq.h;
  const int64_t qstr = rot ? D : p.sq.s;
  const uint16_t* kb = rot ? p.krot + (int64_t)bh * S * D
                           : (const uint16_t*)p.k + b * p.sk.b + h * p.sk.h;
  const int64_t kstr = rot ? D : p.sk.s;
  const uint16_t* vb = (const uint16_t*)p.v + b * p.sv.b + h * p.sv.h;
  const uint16_t* gb = (const uint16_t*)p.dout + b * p.sdo.b + h * p.sdo.h;
  const float* nlb = p.nlse + (int64_t)bh * S;
  const float* dlb = p.delta + (int64_t)bh * S;

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

  // Direct-load plan of a q-tile: 2 CB blocks of 64 chunks (CB of Q~, then
  // CB of dO); this wave loads blocks wave + 8 n.  Position P = 64 * blk +
  // lane of a tile -> (row P / C, chunk (P % C) ^ swizzle(row)).
  int foff[NFB], fdst[NFB];
  bool fdo[NFB];
#pragma unroll
  for (int n = 0; n < NFB; ++n) {
    const int fbk = wave + NW * n;
    fdo[n] = fbk >= CB;
    const int blk = fdo[n] ? fbk - CB : fbk;
    const int P = 64 * blk + lane;
    const int row = P / C, ch = (P % C) ^ swz<C>(row);
    foff[n] = (int)(row * (fdo[n] ? p.sdo.s : qstr)) + 8 * ch;
    fdst[n] = (fdo[n] ? L::G0 - L::Q0 : 0) + 512 * blk;
  }
  // Q~ tile to Qd, dO tile to Qd + G0 - Q0, nlse to Fd[0..BMQ), Delta to
  // Fd[2 BMQ..); on the last tile rows past S re-read row S-1 (masked).
  auto fetch_q = [&](int qt, uint16_t* Qd, float* Fd) {
    const int q0 = qt * BMQ;
    const buf_rsrc qr = raw_rsrc(qb + (int64_t)q0 * qstr);
    const buf_rsrc gr = raw_rsrc(gb + (int64_t)q0 * p.sdo.s);
    if (q0 + BMQ <= S) {
#pragma unroll
      for (int n = 0; n < NFB; ++n) dma16(fdo[n] ? gr : qr, 2u * (uint32_t)foff[n], Qd + fdst[n]);
    } else {
#pragma unroll
      for (int n = 0; n < NFB; ++n) {
        const int fbk = wave + NW * n;
        const int blk = fdo[n] ? fbk - CB : fbk;
        const int P = 64 * blk + lane;
        const int row = P / C, ch = (P % C) ^ swz<C>(row);
        const int rr = min(q0 + row, S - 1) - q0;
        const int str = (int)(fdo[n] ? p.sdo.s : qstr);  // offsets stay 32-bit (bounded strides)
        dma16(fdo[n] ? gr : qr, 2u * (uint32_t)(rr * str + 8 * ch), Qd + fdst[n]);
      }
    }
    if (wave < 2 && lane < BMQ / 4) {
      const float* src = wave == 0 ? nlb : dlb;
      if ((S & 3) == 0 && q0 + BMQ <= S) {  // 16-byte aligned, whole tile
        dma16(raw_rsrc(src + q0), 16u * (uint32_t)lane, Fd + wave * 2 * BMQ);
      } else {
        f32x4 w;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int ii = q0 + 4 * lane + e;
          w[e] = ii < S ? src[ii] : 0.0f;  // rows past S: 0, masked
        }
        *reinterpret_cast<f32x4*>(Fd + wave * 2 * BMQ + 4 * lane) = w;
      }
    }
  };

  // Stationary K~ (and V) tiles (2C blocks each, rows past S repeat row S-1)
  // and the first q-tile.
  {
    const buf_rsrc kr = raw_rsrc(kb + (int64_t)k0 * kstr);
    const buf_rsrc vr = raw_rsrc(vb + (int64_t)k0 * p.sv.s);
#pragma unroll
    for (int n = 0; n < NKB; ++n) {
      const int blk = wave + NW * n;
      const int P = 64 * blk + lane;
      const int row = P / C, ch = (P % C) ^ swz<C>(row);
      const int rr = min(k0 + row, S - 1) - k0;
      dma16(kr, 2u * (uint32_t)(rr * (int)kstr + 8 * ch), lds + L::KT + 512 * blk);
      if constexpr (!kRegV)
        dma16(vr, 2u * (uint32_t)(rr * (int)p.sv.s + 8 * ch), lds + L::VT + 512 * blk);
    }
  }
  fetch_q(qt_lo, lds + L::Q0, fl);
  elem8 kreg[kRegK ? D / 16 : 1], vreg[kRegV ? D / 16 : 1];
  if constexpr (kRegV) {
#pragma unroll
    for (int c = 0; c < D / 16; ++c) {
      vreg[c] = __builtin_bit_cast(elem8, u32x4{0u, 0u, 0u, 0u});
      if (j < S)
        vreg[c] = __builtin_bit_cast(
            elem8, *reinterpret_cast<const u32x4*>(vb + (int64_t)j * p.sv.s + 16 * c + 8 * hh));
    }
  }
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  if constexpr (kRegK) {
#pragma unroll
    for (int c = 0; c < D / 16; ++c)
      kreg[c] = lds_read8(lds + L::KT + 8 * tpos<C>(32 * kg + ql, 2 * c + hh));
  }
  // Operand offsets (elements).  Row reads of Q~ / dO (A of S and dP): row
  // 32 qhalf + ql (+ 64 in the second quarter), chunk 2c + hh.  Transposed reads of a [rows][C chunks]
  // tile: lane 16g + j16 supplies row 16 t + 4 hh + j16/4 (+8 for the second
  // read), 4 columns at chunk 4 db + 2 (g&1) + (j16&3)/2, half (j16&1).
  const int rsw = swz<C>(ql);
  const int trow = 4 * hh + (j16 >> 2);
  const int tch = 2 * (g16 & 1) + ((j16 & 3) >> 1);
  const int thalf = 4 * (j16 & 1);
  int taddr[2][NB];
#pragma unroll
  for (int s2 = 0; s2 < 2; ++s2)
#pragma unroll
    for (int db = 0; db < NB; ++db)
      taddr[s2][db] = 8 * ((trow + 8 * s2) * C + ((4 * db + tch) ^ swz<C>(trow + 8 * s2))) +
                      thalf + 32 * qhalf * D + L::Q0;
  // Row-read offsets: Q~ / dO row 32 qhalf + ql (the second quarter adds the
  // constant 64 rows), K~ / V row 32 kg + ql.  The Q~ offsets (rofs, taddr)
  // are absolute element addresses of the current q-tile buffer: they move to
  // the other buffer after every tile, so that each operand read is one
  // register plus an immediate (the dO tiles sit a constant distance above).
  constexpr int NS = D / 16;  // dims steps of S and dP
  int rofs[NS], kofs[NS];
#pragma unroll
  for (int c = 0; c < NS; ++c) {
    rofs[c] = 8 * ((32 * qhalf + ql) * C + ((2 * c + hh) ^ rsw)) + L::Q0;
    kofs[c] = 8 * ((32 * kg + ql) * C + ((2 * c + hh) ^ rsw));
  }
  constexpr int GQ = L::G0 - L::Q0;  // dO tile of a buffer, relative to its Q~ tile

  const float c2 = a.scale_log2;
  const float scale = a.scale;
  const float slj = ALIBI ? alibi_slope_log2(a, h) * (float)j : 0.0f;
  f32x16 dvacc[NB], dkacc[NB];
#pragma unroll
  for (int db = 0; db < NB; ++db) {
    dvacc[db] = f32x16{};
    dkacc[db] = f32x16{};
  }

  // One q-tile (its Q~ / dO operands at the current rofs / taddr).
  auto tile = [&](auto masked, int qt, uint16_t* __restrict__ Qn, const uint16_t* __restrict__ KTp,
                  const uint16_t* __restrict__ VTp, const float* __restrict__ Fc,
                  float* __restrict__ Fn) __attribute__((always_inline)) {
    const int q0 = qt * BMQ;
    if (qt + 1 < qt_hi) fetch_q(qt + 1, Qn, Fn);
  // Quarter r of this wave (r = 0, 1): its rows 32 qhalf + 64 r .. + 31.
  auto quarter = [&](auto rc) __attribute__((always_inline)) {
    constexpr int R = decltype(rc)::value;
    constexpr int RQ = 8 * 64 * R * C;  // element offset of the quarter's rows
    const float* nlt = Fc + 32 * qhalf + 64 * R;
    const float* dlt = Fc + 2 * BMQ + 32 * qhalf + 64 * R;
    const int qw0 = q0 + 32 * qhalf + 64 * R;

    // The tile in four product groups, each MFMA independent of the VALU work
    // placed beside it so that the two overlap:
    //   S = Q~ K~^T;  dP = dO V^T beside P = exp2(S scale log2e + nlse);
    //   dV^T += dO^T P beside dS' = P (dP - Delta);  dK~^T += Q~^T dS'.
    // (The softmax scale is applied to dK~ at the end.)  Register r of S / dP
    // is query qw0 + 8 (r/4) + 4 hh + r%4.
    {
      constexpr bool kMasked = decltype(masked)::value;
      const int lo_off = qlo - qw0 - 4 * hh, hi_off = qhi - qw0 - 4 * hh;
      // nlse of this lane's rows now; -Delta (stored negated) just before the
      // dP products, which start from it.
      f32x4 n4[4], d4[4];
#pragma unroll
      for (int a4 = 0; a4 < 4; ++a4) n4[a4] = *reinterpret_cast<const f32x4*>(nlt + 8 * a4 + 4 * hh);

      // dO^T and Q~^T operands of (query chunk qc, dim block db): transposed
      // reads.
      constexpr int NG = 2 * NB;
      auto top = [&](int base, int g) {
        const int off = taddr[0][g % NB] + base + 16 * (g / NB) * D + 64 * R * D;
        return tr8(lds + off, taddr[1][g % NB] - taddr[0][g % NB]);
      };
      // One stream of MFMA steps: S (NS), dP (NS), dV (NG), dK (NG); each
      // step's LDS operands are read PF steps ahead.
      constexpr int NST = 2 * NS + 2 * NG;
      constexpr int PF = kDkdvPrefetch;
      struct Op {
        elem8 a, b;
      };
      auto rd = [&](int t) {
        Op o;
        if (t < NS) {
          o.a = lds_read8(lds + rofs[t] + RQ);
          o.b = kRegK ? o.a : lds_read8(KTp + kofs[t]);
        } else if (t < 2 * NS) {
          o.a = lds_read8(lds + GQ + rofs[t - NS] + RQ);
          o.b = kRegV ? o.a : lds_read8(VTp + kofs[t - NS]);
        } else if (t < 2 * NS + NG) {
          o.a = top(GQ, t - 2 * NS);
          o.b = o.a;
        } else {
          o.a = top(0, t - 2 * NS - NG);
          o.b = o.a;
        }
        return o;
      };
      f32x16 sacc = f32x16{}, dpacc = f32x16{};
      u32x4 pw[2], sw[2];
      Op ring[NST];
#pragma unroll
      for (int t = 0; t < PF; ++t) ring[t] = rd(t);
#pragma unroll
      for (int t = 0; t < NST; ++t) {
        if (t + PF < NST) ring[t + PF] = rd(t + PF);
        if (t == NS - 2 || (NS < 2 && t == 0)) {
#pragma unroll
          for (int a4 = 0; a4 < 4; ++a4)
            d4[a4] = *reinterpret_cast<const f32x4*>(dlt + 8 * a4 + 4 * hh);
        }
        __builtin_amdgcn_sched_barrier(0);
        const Op o = ring[t];
        if (t < NS) {
          sacc = mfma32x32x16(o.a, kRegK ? kreg[kRegK ? t : 0] : o.b, sacc);
        } else if (t < 2 * NS) {
          const int c = t - NS;
          if (c == 0) {
            // dP starts from -Delta (register r: row 8 (r/4) + 4 hh + r%4),
            // so the products leave dP - Delta
#pragma unroll
            for (int a4 = 0; a4 < 4; ++a4)
#pragma unroll
              for (int e = 0; e < 4; ++e) dpacc[4 * a4 + e] = d4[a4][e];
          }
          dpacc = mfma32x32x16(o.a, kRegV ? vreg[kRegV ? c : 0] : o.b, dpacc);
          // P for this step's share of register pairs
#pragma unroll
          for (int pp = 8 * c / NS; pp < 8 * (c + 1) / NS; ++pp) {
#pragma unroll
            for (int e = 2 * pp; e < 2 * pp + 2; ++e) {
              const float nl = ALIBI ? n4[e / 4][e % 4] + slj : n4[e / 4][e % 4];
              float pr = fast_exp2(__builtin_fmaf(sacc[e], c2, nl));
              if (kMasked) {
                const int io = 8 * (e / 4) + e % 4;
                if (io < lo_off || io > hi_off) pr = 0.0f;
              }
              sacc[e] = pr;
            }
            pw[pp / 4][pp % 4] = pack2(sacc[2 * pp], sacc[2 * pp + 1]);
          }
        } else if (t < 2 * NS + NG) {
          const int g = t - 2 * NS;
          dvacc[g % NB] = mfma32x32x16(o.a, __builtin_bit_cast(elem8, pw[g / NB]), dvacc[g % NB]);
          // dS' for this step's share of register pairs
#pragma unroll
          for (int pp = 8 * g / NG; pp < 8 * (g + 1) / NG; ++pp) {
            float x[2];
#pragma unroll
            for (int e = 0; e < 2; ++e) {
              const int r = 2 * pp + e;
              x[e] = sacc[r] * dpacc[r];
            }
            sw[pp / 4][pp % 4] = pack2(x[0], x[1]);
          }
        } else {
          const int g = t - 2 * NS - NG;
          dkacc[g % NB] = mfma32x32x16(o.a, __builtin_bit_cast(elem8, sw[g / NB]), dkacc[g % NB]);
        }
      }
    }
  };
    quarter(std::integral_constant<int, 0>{});
    if constexpr (NQQ == 2) quarter(std::integral_constant<int, 1>{});
  };
  // A wave's q-tiles fall into runs: masked ones before its first tile inside
  // every row's range (the diagonal), unmasked ones, masked ones after
  // (document ends).  An inner loop per run keeps one variant of the tile per
  // loop.
  auto full = [&](int qt) {
    const int qw0 = qt * BMQ + 32 * qhalf;  // first row of the wave's first quarter
    return __all((qw0 >= qlo) && (qw0 + 64 * (NQQ - 1) + 31 <= qhi));
  };
  auto run = [&](auto masked, int qt) __attribute__((always_inline)) {
    const int buf = (qt - qt_lo) & 1;
    tile(masked, qt, lds + L::Q0 + (buf ^ 1) * BMQ * D, lds + L::KT, lds + L::VT, fl + buf * BMQ,
         fl + (buf ^ 1) * BMQ);
    // the next tile's operands sit in the other buffer
    const int step = buf ? -BMQ * D : BMQ * D;
#pragma unroll
    for (int c = 0; c < NS; ++c) rofs[c] += step;
#pragma unroll
    for (int s2 = 0; s2 < 2; ++s2)
#pragma unroll
      for (int db = 0; db < NB; ++db) taddr[s2][db] += step;
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
  };
  // masked and unmasked runs of q-tiles (each form's code appears once)
  int qt = qt_lo;
  while (qt < qt_hi) {
    for (; qt < qt_hi && !full(qt); ++qt) run(std::true_type{}, qt);
    for (; qt < qt_hi && full(qt); ++qt) run(std::false_type{}, qt);
  }

  // Epilogue: the two query halves of a key group add their dK~ and dV partial
  // sums in fp32 over the (now idle) LDS, then rows are written coalesced;
  // dK = scale R^T dK~.
  constexpr int FS = D + 4;          // staged row stride (floats)
  constexpr int NIT = C / 4;  // 8-dim row chunks per thread (128 rows, 4 chunk groups)
  static_assert(C % 4 == 0 && NT8 == 4 * BNK, "row chunks must split evenly over the workgroup");
  float* stk = reinterpret_cast<float*>(lds);
  float* stv = stk + BNK * FS;
  static_assert(2 * BNK * FS * 4 <= L::EPI_BYTES, "epilogue staging must fit");
  auto epilogue = [&](auto rope_tag) __attribute__((always_inline)) {
    constexpr bool kRope = decltype(rope_tag)::value;
    const int rd = a.rd, half = rd >> 1;
    // This lane's staged row, derived here from the thread index (through an
    // empty asm, so that it is not computed before the tile loop and kept
    // live across it).
    int te = tid;
    __asm__ volatile("" : "+v"(te));
    const int erow = 32 * kg + (te & 31);
    // Query half 1 stores its sums, query half 0 adds its own (all reads
    // issued before the first add) and stores the total.
    if (qhalf == 1) {
#pragma unroll
      for (int db = 0; db < NB; ++db)
#pragma unroll
        for (int a4 = 0; a4 < 4; ++a4) {
          const int off = erow * FS + 32 * db + 8 * a4 + 4 * hh;
          f32x4 wk, wv;
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            wk[e] = dkacc[db][4 * a4 + e];
            wv[e] = dvacc[db][4 * a4 + e];
          }
          *reinterpret_cast<f32x4*>(stk + off) = wk;
          *reinterpret_cast<f32x4*>(stv + off) = wv;
        }
    }
    __syncthreads();
    if (qhalf == 0) {
#pragma unroll
      for (int pass = 0; pass < 2; ++pass) {
        float* st = pass == 0 ? stk : stv;
        f32x4 o4[NB][4];
#pragma unroll
        for (int db = 0; db < NB; ++db)
#pragma unroll
          for (int a4 = 0; a4 < 4; ++a4)
            o4[db][a4] = *reinterpret_cast<const f32x4*>(st + erow * FS + 32 * db + 8 * a4 + 4 * hh);
#pragma unroll
        for (int db = 0; db < NB; ++db)
#pragma unroll
          for (int a4 = 0; a4 < 4; ++a4) {
            f32x4 w;
#pragma unroll
            for (int e = 0; e < 4; ++e)
              w[e] = pass == 0 ? (dkacc[db][4 * a4 + e] + o4[db][a4][e]) * scale
                               : dvacc[db][4 * a4 + e] + o4[db][a4][e];
            *reinterpret_cast<f32x4*>(st + erow * FS + 32 * db + 8 * a4 + 4 * hh) = w;
          }
      }
    }
    __syncthreads();
    // Rows out, chunk m of this thread: with the rotation on part of the dims
    // (0 < rd < D, D <= 96) thread t takes row t % 128, chunk 4 m + t / 128, so a chunk
    // pass touches the rotary dims (or not) for a whole wave and the rotary
    // work is skipped where it is not; otherwise consecutive threads take
    // consecutive chunks of a row (whole rows per store instruction).  The
    // rotary table entries of the thread's dK chunks are requested before the
    // dV rows go out, so that their latency passes meanwhile; every staged
    // value is read before any is used.
    const bool part = kRope && D <= 96 && rd < D;  // (at D = 128 the row-major order measured faster)
    auto crow = [&](int m) { return part ? (tid & (BNK - 1)) : (tid + NT8 * m) / C; };
    auto cd0 = [&](int m) { return part ? 8 * (4 * m + tid / BNK) : 8 * ((tid + NT8 * m) % C); };
    float2 cs[NIT][8];
    if constexpr (kRope) {
#pragma unroll
      for (int m = 0; m < NIT; ++m) {
        const int d0 = cd0(m);
        if (!part || d0 < rd) {
          rope_entries8(a.rope + (int64_t)min(k0 + crow(m), S - 1) * half, d0, half, rd, cs[m]);
        }
      }
    }
#pragma unroll
    for (int pass = 1; pass >= 0; --pass) {
      void* outp = pass == 0 ? p.dk : p.dv;
      const Strides so = pass == 0 ? p.sdk : p.sdv;
      float x[NIT][8];
#pragma unroll
      for (int m = 0; m < NIT; ++m) {
        const int d0 = cd0(m);
        const float* srow_p = (pass == 0 ? stk : stv) + crow(m) * FS;
        const f32x4 lo = *reinterpret_cast<const f32x4*>(srow_p + d0);
        const f32x4 hi = *reinterpret_cast<const f32x4*>(srow_p + d0 + 4);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          x[m][e] = lo[e];
          x[m][4 + e] = hi[e];
        }
        if (kRope && pass == 0 && (!part || d0 < rd)) {
          float xp[8];
#pragma unroll
          for (int e = 0; e < 8; ++e) xp[e] = srow_p[d0 + e + rot_partner_step(d0 + e, half, rd)];
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            float cn, sn;
            rot_t_factors(cs[m][e], d0 + e, half, rd, cn, sn);
            x[m][e] = x[m][e] * cn + xp[e] * sn;
          }
        }
      }
#pragma unroll
      for (int m = 0; m < NIT; ++m) {
        const int d0 = cd0(m), jj = k0 + crow(m);
        if (jj < S) {
          if (p.out_f32) {
            float* orow = (float*)outp + b * so.b + h * so.h + (int64_t)jj * so.s + d0;
            *reinterpret_cast<f32x4*>(orow) = f32x4{x[m][0], x[m][1], x[m][2], x[m][3]};
            *reinterpret_cast<f32x4*>(orow + 4) = f32x4{x[m][4], x[m][5], x[m][6], x[m][7]};
          } else {
            uint16_t* orow = (uint16_t*)outp + b * so.b + h * so.h + (int64_t)jj * so.s + d0;
            *reinterpret_cast<u32x4*>(orow) =
                u32x4{pack2(x[m][0], x[m][1]), pack2(x[m][2], x[m][3]), pack2(x[m][4], x[m][5]),
                      pack2(x[m][6], x[m][7])};
          }
        }
      }
    }
  };
  if (a.rd > 0)
    epilogue(std::true_type{});
  else
    epilogue(std::false_type{});
}

// ------------------------------------------------------------------------ dQ

// dQ~ without atomics: one workgroup per (batch, head, 128 queries), four
// waves of 32 queries.  Q~ and dO stay in registers while K~ and V tiles of 64
// keys stream through LDS (direct loads, double buffered):
//   S^T = K~ Q~^T,  dP^T = V dO^T    (A = K~ / V rows from LDS, B = registers)
//   P = exp2(S scale log2e + nlse_i),  dS' = P (dP - Delta_i)
//   dQ~^T += K~^T dS'^T               (A = K~ transposed from LDS, B = dS')
// Lane l owns query l % 32 of its wave, so nlse_i and Delta_i are per-lane
// scalars.  The epilogue writes dq = scale R^T dQ~.
constexpr int DQ_BM = 128;  // queries per workgroup
constexpr int DQ_BN = 64;   // keys per tile

template <int D, bool ALIBI>
__global__ __launch_bounds__(NT, 2) void bwd_dq_kernel(BwdParams p) {
  constexpr int C = D / 8;
  constexpr int NB = D / 32;
  constexpr int TILE = DQ_BN * D;        // elements of one K~ or V tile buffer
  constexpr int NTB = DQ_BN * C / 64 / 4;  // 1 KB load blocks per wave, per tile and tensor
  static_assert(C % 4 == 0, "tile blocks must split evenly over 4 waves");
  constexpr int FS = D + 4;              // epilogue staging row (floats)
  constexpr int LDS_ELEMS = (4 * TILE > 4 * 32 * FS * 2) ? 4 * TILE : 4 * 32 * FS * 2;
  __shared__ __attribute__((aligned(16))) uint16_t lds[LDS_ELEMS];  // K0 K1 V0 V1

  const AttnShape& a = p.a;
  const int S = a.S;
  const int nqt = (S + DQ_BM - 1) / DQ_BM;
  const int BH = a.B * a.H;
  const int qt = nqt - 1 - (int)(blockIdx.x / BH);  // heaviest q-tile first, heads fastest
  const int bh = (int)(blockIdx.x % BH);
  const int b = bh / a.H, h = bh % a.H;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int ql = lane & 31, hh = lane >> 5;
  const int g16 = lane >> 4, j16 = lane & 15;
  const int q0 = qt * DQ_BM;
  const int qi = q0 + 32 * wave + ql;  // this lane's query
  const int qc = qi < S ? qi : S - 1;

  const bool rot = a.rd > 0;
  const uint16_t* qb = rot ? p.qrot + (int64_t)bh * S * D
                           : (const uint16_t*)p.q + b * p.sq.b + h * p.sq.h;
  const int64_t qstr = rot ? D : p.sq.s;
  const uint16_t* kb = rot ? p.krot + (int64_t)bh * S * D
                           : (const uint16_t*)p.k + b * p.sk.b + h * p.sk.h;
  const int64_t kstr = rot ? D : p.sk.s;
  const uint16_t* vb = (const uint16_t*)p.v + b * p.sv.b + h * p.sv.h;
  const uint16_t* gb = (const uint16_t*)p.dout + b * p.sdo.b + h * p.sdo.h;

  // Allowed keys of this lane's query: [lo, hi]; keys any query of the block may see.
  const int32_t* drow = a.docs ? a.docs + (int64_t)b * (a.n_docs + 1) : nullptr;
  int lo = 0, hi = S - 1;
  if (drow) {
    int ds, de;
    doc_bounds(drow, a.n_docs, S, qc, ds, de);
    lo = ds;
    hi = de - 1;
  }
  if (a.causal && qi < hi) hi = qi;
  const int qlast = (q0 + DQ_BM - 1 < S - 1) ? q0 + DQ_BM - 1 : S - 1;
  int blo = 0, bhi = S - 1;
  if (drow) {
    int s0, e0, s1, e1;
    doc_bounds(drow, a.n_docs, S, q0, s0, e0);
    doc_bounds(drow, a.n_docs, S, qlast, s1, e1);
    blo = s0;
    bhi = e1 - 1;
  }
  if (a.causal && qlast < bhi) bhi = qlast;
  const int kt_lo = blo / DQ_BN, kt_hi = bhi / DQ_BN + 1;

  // Tile loader: rows [k0, k0 + 64) of K~ and V (rows past S repeat row S-1,
  // their keys are masked).  Position P = 64 * blk + lane of a tile -> (row
  // P / C, chunk (P % C) ^ swizzle(row)); this wave loads blocks wave + 4 n.
  int koff[NTB], voff[NTB];
#pragma unroll
  for (int n = 0; n < NTB; ++n) {
    const int P = 64 * (wave + 4 * n) + lane;
    const int row = P / C, ch = (P % C) ^ swz<C>(row);
    koff[n] = (int)(row * kstr) + 8 * ch;
    voff[n] = (int)(row * p.sv.s) + 8 * ch;
  }
  auto fetch = [&](int kt, uint16_t* Kd, uint16_t* Vd) {
    const int k0 = kt * DQ_BN;
    const buf_rsrc kr = raw_rsrc(kb + (int64_t)k0 * kstr);
    const buf_rsrc vr = raw_rsrc(vb + (int64_t)k0 * p.sv.s);
    if (k0 + DQ_BN <= S) {
#pragma unroll
      for (int n = 0; n < NTB; ++n) {
        dma16(kr, 2u * (uint32_t)koff[n], Kd + 512 * (wave + 4 * n));
        dma16(vr, 2u * (uint32_t)voff[n], Vd + 512 * (wave + 4 * n));
      }
    } else {
#pragma unroll
      for (int n = 0; n < NTB; ++n) {
        const int P = 64 * (wave + 4 * n) + lane;
        const int row = P / C, ch = (P % C) ^ swz<C>(row);
        const int rr = min(k0 + row, S - 1) - k0;
        dma16(kr, 2u * (uint32_t)(rr * (int)kstr + 8 * ch), Kd + 512 * (wave + 4 * n));
        dma16(vr, 2u * (uint32_t)(rr * (int)p.sv.s + 8 * ch), Vd + 512 * (wave + 4 * n));
      }
    }
  };
  fetch(kt_lo, lds, lds + 2 * TILE);

  // Q~ and dO of this lane's query as B operands: chunk c holds dims 16c + 8hh .. +7.
  // The same chunks of o give Delta_i = dO_i . o_i (the lane halves add their
  // partial sums); with lse_i it also forms nlse_i = -lse_i log2(e) (ALiBi:
  // minus the row term).  Both go to the workspace for the dK/dV pass, which
  // runs after this one.
  elem8 qreg[D / 16], greg[D / 16];
  const uint16_t* ob = (const uint16_t*)p.o + b * p.so.b + h * p.so.h;
  const float lse_i = p.lse[(int64_t)bh * S + qc];
  float dsum = 0.0f;
#pragma unroll
  for (int c = 0; c < D / 16; ++c) {
    const int d0 = 16 * c + 8 * hh;
    u32x4 wq = *reinterpret_cast<const u32x4*>(qb + (int64_t)qc * qstr + d0);
    u32x4 wg = *reinterpret_cast<const u32x4*>(gb + (int64_t)qc * p.sdo.s + d0);
    const u32x4 wo = *reinterpret_cast<const u32x4*>(ob + (int64_t)qc * p.so.s + d0);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      dsum = fmaf(el_lo(wo[e]), el_lo(wg[e]), dsum);
      dsum = fmaf(el_hi(wo[e]), el_hi(wg[e]), dsum);
    }
    if (qi >= S) wq = wg = u32x4{0u, 0u, 0u, 0u};
    qreg[c] = __builtin_bit_cast(elem8, wq);
    greg[c] = __builtin_bit_cast(elem8, wg);
  }
  dsum += __shfl_xor(dsum, 32);
  float nl = -lse_i * kLog2e;
  if (a.alibi) nl -= alibi_slope_log2(a, h) * (float)qc;
  if (qi < S && hh == 0) {
    p.delta[(int64_t)bh * S + qi] = -dsum;  // stored negated: the dK/dV pass starts dP there
    p.nlse[(int64_t)bh * S + qi] = nl;
  }
  if (qi >= S) nl = 0.0f;
  const float dl = qi < S ? dsum : 0.0f;
  constexpr bool kNdl = D == 96;  // D = 64 would lose its third wave per SIMD to the 16 registers
  f32x16 ndl16;
#pragma unroll
  for (int r = 0; r < 16; ++r) ndl16[r] = kNdl ? -dl : 0.0f;
  const float c2 = a.scale_log2;
  const float sl2 = ALIBI ? alibi_slope_log2(a, h) : 0.0f;

  // LDS operand offsets.  Row reads (A of S^T and dP^T): row 32 blk + ql,
  // chunk 2c + hh.  Transposed K~ reads (A of dQ~^T): lane 16g + j16 supplies
  // key row 16 kc + 4 hh + j16/4 (+8 for the second read), 4 dims at chunk
  // 4 db + 2 (g&1) + (j16&3)/2, half (j16&1).
  const int rsw = swz<C>(ql);
  const int trow = 4 * hh + (j16 >> 2);
  const int tch = 2 * (g16 & 1) + ((j16 & 3) >> 1);
  const int thalf = 4 * (j16 & 1);
  int taddr[2][NB];
#pragma unroll
  for (int s2 = 0; s2 < 2; ++s2)
#pragma unroll
    for (int db = 0; db < NB; ++db)
      taddr[s2][db] = 8 * ((trow + 8 * s2) * C + ((4 * db + tch) ^ swz<C>(trow + 8 * s2))) + thalf;

  f32x16 dqacc[NB];
#pragma unroll
  for (int db = 0; db < NB; ++db) dqacc[db] = f32x16{};
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();

  // One key tile; restrict pointers let the compiler separate these reads from
  // the next tile's direct loads in flight.
  auto step = [&](int kt, const uint16_t* __restrict__ Kc, const uint16_t* __restrict__ Vc,
                  uint16_t* __restrict__ Kn, uint16_t* __restrict__ Vn) {
    const int k0 = kt * DQ_BN;
    if (kt + 1 < kt_hi) fetch(kt + 1, Kn, Vn);
    const bool lane_any = (k0 <= hi) && (k0 + DQ_BN - 1 >= lo);
    if (!__any(lane_any)) return;
    const bool lane_full = (k0 >= lo) && (k0 + DQ_BN - 1 <= hi);
    const bool masked = !__all(lane_full);
    // The tile's two 32-key halves one after the other (bounds the registers).
#pragma unroll
    for (int blk = 0; blk < 2; ++blk) {
      // dP accumulates from -Delta_i where the registers allow a constant block
      f32x16 sacc = f32x16{}, dpacc = kNdl ? ndl16 : f32x16{};
      // K~ / V rows of dims step c, read one step ahead of their MFMAs.
      auto rows = [&](int c, elem8& kr, elem8& vr) {
        const int off = 8 * (ql * C + ((2 * c + hh) ^ rsw)) + 32 * blk * D;
        kr = lds_read8(Kc + off);
        vr = lds_read8(Vc + off);
      };
      elem8 kc_, vc_;
      rows(0, kc_, vc_);
#pragma unroll
      for (int c = 0; c < D / 16; ++c) {
        elem8 kn = kc_, vn = vc_;
        if (c + 1 < D / 16) rows(c + 1, kn, vn);
        __builtin_amdgcn_sched_barrier(0);  // keep the next operands' reads ahead of these MFMAs
        sacc = mfma32x32x16(kc_, qreg[c], sacc);
        dpacc = mfma32x32x16(vc_, greg[c], dpacc);
        kc_ = kn;
        vc_ = vn;
      }
      // Register r: key k0 + 32 blk + 8 (r/4) + 4 hh + r%4.
      auto pds = [&](auto mk) {
        constexpr bool kMasked = decltype(mk)::value;
        const int jlo = lo - k0 - 32 * blk - 4 * hh, jhi = hi - k0 - 32 * blk - 4 * hh;
        const float kbase = ALIBI ? sl2 * (float)(k0 + 32 * blk + 4 * hh) + nl : nl;
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int ko = 8 * (r >> 2) + (r & 3);
          const float bias = ALIBI ? __builtin_fmaf(sl2, (float)ko, kbase) : nl;  // fma: not hoisted as 16 products
          float pr = fast_exp2(__builtin_fmaf(sacc[r], c2, bias));
          if (kMasked && (ko < jlo || ko > jhi)) pr = 0.0f;
          dpacc[r] = pr * (kNdl ? dpacc[r] : dpacc[r] - dl);
        }
      };
      if (masked) {
        asm volatile("" ::: "memory");  // keeps this a branch (no if-conversion)
        pds(std::true_type{});
      } else {
        pds(std::false_type{});
      }
      elem8 sb[2];
#pragma unroll
      for (int kh = 0; kh < 2; ++kh) {
        float sv[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) sv[e] = dpacc[8 * kh + e];
        sb[kh] = pack8(sv);
      }
      // K~^T operand of (key chunk, dim block) g, read one MFMA ahead.
      constexpr int NG = 2 * NB;
      auto kt_op = [&](int g) {
        const int kc = 2 * blk + g / NB, db = g % NB;
        return tr8(Kc + taddr[0][db] + 16 * kc * D, taddr[1][db] - taddr[0][db]);
      };
      elem8 ka = kt_op(0);
#pragma unroll
      for (int g = 0; g < NG; ++g) {
        const elem8 kn = g + 1 < NG ? kt_op(g + 1) : ka;
        __builtin_amdgcn_sched_barrier(0);  // keep the next operands' reads ahead of these MFMAs
        dqacc[g % NB] = mfma32x32x16(ka, sb[g / NB], dqacc[g % NB]);
        ka = kn;
      }
    }
  };
  for (int kt = kt_lo; kt < kt_hi; ++kt) {
    const int buf = (kt - kt_lo) & 1;
    step(kt, lds + buf * TILE, lds + (2 + buf) * TILE, lds + (1 - buf) * TILE,
         lds + (3 - buf) * TILE);
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
  }

  // Epilogue: stage this wave's 32 rows of dQ~ (fp32) in LDS, then write
  // dq = scale R^T dQ~ row-wise.  Register r of dim block db holds dim
  // 32 db + 8 (r/4) + 4 hh + r%4 of query ql.  Lane (ql, hh) writes chunks
  // 2m + hh of row ql, so a pass m either touches the rotary dims (16 m < rd)
  // or not, for the whole wave: the rotary table entries are requested, all at
  // once, only for the passes that need them, and every staged value a lane
  // needs is read before any is used.
  constexpr int NIT = C / 2;  // passes: chunks 2m and 2m + 1 of the 32 rows
  static_assert(C % 2 == 0, "row chunks must pair up");
  float* stage = reinterpret_cast<float*>(lds) + wave * 32 * FS;
  const float scale = a.scale;
  auto epilogue = [&](auto rope_tag) __attribute__((always_inline)) {
    constexpr bool kRope = decltype(rope_tag)::value;
    const int rd = a.rd, half = rd >> 1;
#pragma unroll
    for (int db = 0; db < NB; ++db)
#pragma unroll
      for (int a4 = 0; a4 < 4; ++a4) {
        f32x4 w;
#pragma unroll
        for (int e = 0; e < 4; ++e) w[e] = dqacc[db][4 * a4 + e];
        *reinterpret_cast<f32x4*>(stage + ql * FS + 32 * db + 8 * a4 + 4 * hh) = w;
      }
    lds_wave_sync();
    const int i = q0 + 32 * wave + ql;  // this lane's row
    const float* srow = stage + ql * FS;
    float2 cs[NIT][8];
    if constexpr (kRope) {
      const float2* rrow = a.rope + (int64_t)min(i, S - 1) * half;
#pragma unroll
      for (int m = 0; m < NIT; ++m) {
        if (16 * m < rd) rope_entries8(rrow, 8 * (2 * m + hh), half, rd, cs[m]);
      }
    }
    float x[NIT][8];
#pragma unroll
    for (int m = 0; m < NIT; ++m) {
      const int d0 = 8 * (2 * m + hh);
      const f32x4 lo4 = *reinterpret_cast<const f32x4*>(srow + d0);
      const f32x4 hi4 = *reinterpret_cast<const f32x4*>(srow + d0 + 4);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        x[m][e] = lo4[e];
        x[m][4 + e] = hi4[e];
      }
      if (kRope && 16 * m < rd) {
        float xp[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) xp[e] = srow[d0 + e + rot_partner_step(d0 + e, half, rd)];
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          float cn, sn;
          rot_t_factors(cs[m][e], d0 + e, half, rd, cn, sn);
          x[m][e] = x[m][e] * cn + xp[e] * sn;
        }
      }
    }
    if (i < S) {
#pragma unroll
      for (int m = 0; m < NIT; ++m) {
        const int d0 = 8 * (2 * m + hh);
#pragma unroll
        for (int e = 0; e < 8; ++e) x[m][e] *= scale;
        if (p.out_f32) {
          float* orow = (float*)p.dq + b * p.sdq.b + h * p.sdq.h + (int64_t)i * p.sdq.s + d0;
          *reinterpret_cast<f32x4*>(orow) = f32x4{x[m][0], x[m][1], x[m][2], x[m][3]};
          *reinterpret_cast<f32x4*>(orow + 4) = f32x4{x[m][4], x[m][5], x[m][6], x[m][7]};
        } else {
          uint16_t* orow = (uint16_t*)p.dq + b * p.sdq.b + h * p.sdq.h + (int64_t)i * p.sdq.s + d0;
          *reinterpret_cast<u32x4*>(orow) =
              u32x4{pack2(x[m][0], x[m][1]), pack2(x[m][2], x[m][3]), pack2(x[m][4], x[m][5]),
                    pack2(x[m][6], x[m][7])};
        }
      }
    }
  };
  if (a.rd > 0)
    epilogue(std::true_type{});
  else
    epilogue(std::false_type{});
}

// One wave per (position, group of RPW heads), four waves per block.
template <int D>
dim3 row_grid(const BwdParams& p) {
  const int64_t hpw = RowGroups<D>::RPW;
  const int64_t waves = (p.a.B * p.a.H + hpw - 1) / hpw * p.a.S;
  return dim3((unsigned)((waves + 3) / 4));
}

template <int D>
hipError_t launch_d(const BwdParams& p, hipStream_t st, const hipEvent_t* ev) {
  hipError_t e;
  if ((e = record_event(ev, 0, st)) != hipSuccess) return e;
  const BwdPlan plan = bwd_plan16(p.a.rd, p.a.alibi != 0, p.qk_ready != 0);
  if (plan.rotation_pass) {
    hipLaunchKernelGGL((bwd_prep_kernel<D>), row_grid<D>(p), dim3(256), 0, st, p);
    if ((e = hipGetLastError()) != hipSuccess) return e;
  }
  if ((e = record_event(ev, 1, st)) != hipSuccess) return e;
  // dQ first: it also writes Delta and nlse, which the dK/dV pass reads.
  const unsigned BH = (unsigned)(p.a.B * p.a.H);
  const dim3 qgrid((unsigned)((p.a.S + DQ_BM - 1) / DQ_BM) * BH);
  if (plan.alibi)
    hipLaunchKernelGGL((bwd_dq_kernel<D, true>), qgrid, dim3(NT), 0, st, p);
  else
    hipLaunchKernelGGL((bwd_dq_kernel<D, false>), qgrid, dim3(NT), 0, st, p);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  if ((e = record_event(ev, 2, st)) != hipSuccess) return e;
  using L = DkdvLds<D>;
  const dim3 kgrid((unsigned)((p.a.S + L::BNK - 1) / L::BNK) * BH);
  if (plan.alibi)
    hipLaunchKernelGGL((bwd_dkdv_kernel<D, true>), kgrid, dim3(L::NTH), 0, st, p);
  else
    hipLaunchKernelGGL((bwd_dkdv_kernel<D, false>), kgrid, dim3(L::NTH), 0, st, p);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  return record_event(ev, 3, st);
}

}  // namespace
}  // namespace NEOX_ELEM_NS

hipError_t NEOX_ELEM_FN(launch_bwd)(const BwdParams& p, hipStream_t st, const hipEvent_t* ev) {
  using namespace NEOX_ELEM_NS;
  switch (p.a.D) {
    case 64: return launch_d<64>(p, st, ev);
    case 96: return launch_d<96>(p, st, ev);
    case 128: return launch_d<128>(p, st, ev);
    default: return hipErrorInvalidValue;
  }
}


}  // namespace neox
