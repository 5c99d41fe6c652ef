// Forward attention on gfx950, 16-bit storage (bf16; fwd_f16.hip compiles this
// file again for IEEE half), MFMA on that type with fp32 accumulation.
//
// Tiled, IO-aware exact attention (the FlashAttention-2 form the GPT-NeoX pages
// name in "GPT-NeoX 开源训练框架深度解读", section "问题二：注意力计算太慢"):
// each workgroup owns 128 query rows of one (batch, head); it streams K/V in
// tiles of 64 keys (32 at D = 128) through LDS, keeps a running row max and row sum (online
// softmax) in registers, and never materialises the S x S score matrix.  The
// NeoX rotary rotation of Q and K ("FasterTransformer GPT-NeoX 推理指南",
// neox_rotary_style_ / rotary_embedding) is applied while rows are loaded.
//
// Layout (one wave = 64 lanes = 32 queries):
//  * S^T = K~ Q~^T on v_mfma_f32_32x32x16_bf16: A = K~ rows from LDS, B = Q~
//    held in registers for the whole loop.  Lane l gets the scores of query
//    l%32 against 16 keys per 32-key block, so the row max needs one lane swap
//    (l <-> l^32) and the row sum is a per-lane partial until the end.
//  * O^T += V^T P^T: B = P straight from the score registers; A = V^T read from
//    the row-major V tile with ds_read_b64_tr_b16 (two 4-key reads per 8-key
//    operand), so V needs no transposition anywhere.
//  * K/V tiles go global -> LDS directly (buffer_load_dwordx4 ... lds) into an
//    unpadded, XOR-swizzled layout that keeps the operand reads free of bank
//    conflicts; only the rotary dims of K pass through registers.  Two LDS
//    buffers (three for 32-key tiles), one barrier per tile; every LDS operand
//    address is a per-lane register offset from the buffer's base plus an
//    immediate.
//  * Tiles fully inside every row's allowed range skip the mask.  A tile's
//    probabilities are taken against the running max without first finding
//    the tile's own max; their per-lane sum bounds each of them, and only a
//    tile whose sum exceeds 2^8 (or a row's first tile) finds the max, raises
//    the running max and rescales O and the row sum.
//  * Workgroups are issued heaviest q-tile first, heads fastest: with B*H a
//    multiple of 8 all q-tiles of a head share one XCD and its L2.  (Grouping
//    each XCD's heads so that their K/V stay L2-resident cuts the fetched
//    bytes five-fold but measured slower here: the K/V re-reads are served by
//    the 256 MB Infinity Cache, and the kernel is bound by issue, not memory.)
//  * With a caller workspace, a row pass first writes q~ = R q and k~ = R k
//    (the NeoX pipeline rotates q and k before attention), and the attention
//    kernel runs its rotation-free form on them.  Without one, Q~ is rotated
//    when a workgroup loads it and the rotary K dims at every tile visit.
#include "device_common.hpp"

namespace neox {
namespace NEOX_ELEM_NS {
namespace {

constexpr int BM = 128;  // query rows per workgroup (4 waves x 32)
constexpr int NT = 256;  // threads per workgroup
// A lane's probabilities over one tile (its keys of the tile) may sum to at
// most 2^8 before the exact path raises the running max, so each stays <= 2^8.
constexpr float kTileSumLimit = 256.0f;

// K/V tile geometry per head dim.  At D = 128 a tile holds 32 keys: the
// smaller score block and LDS footprint let three workgroups share a CU (at
// most 168 registers per lane, 48 KB of LDS each), one more than 64-key tiles
// allow there.  LDS holds buffer pairs of (K, V), each K tile followed by its
// V tile (two pairs, or three for 32-key tiles); Q~ rows are staged after the
// first pair during the prologue.
template <int D>
struct FwdTile {
  static constexpr int BN = D == 128 ? 32 : 64;  // keys per tile
  static constexpr int KB = BN / 32;                          // 32-key score blocks per tile
  static constexpr int TILE = BN * D;                         // elements of one K or V buffer
  static constexpr int LDS = 2 * TILE + (2 * TILE > BM * D ? 2 * TILE : BM * D);
};

typedef short s16x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ s16x4 lds_read_tr4(const uint16_t* p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (__attribute__((address_space(3))) s16x4*)(reinterpret_cast<uintptr_t>(p)));
}

// LDS layout of a K or V tile: BN rows x D/8 chunks of 16 bytes, unpadded, chunk
// c of row r at position r*(D/8) + (c ^ swizzle(r)).  The swizzles make the
// MFMA operand reads conflict-free across the 64 LDS banks: K is read one row
// per lane (16 B, rows 0..15 of a lane group must hit 16 different bank
// groups); V is read with ds_read_b64_tr_b16 (4 rows x 4 chunks per 32 lanes).
template <int D>
struct Swz {
  static __device__ __forceinline__ int k(int row) {
    return D == 128 ? (row & 15) : (D == 64 ? ((row >> 1) & 7) : ((row >> 2) & 3));
  }
  static __device__ __forceinline__ int v(int row) {
    return D == 128 ? 4 * (row & 3) : (D == 64 ? 4 * ((row >> 1) & 1) : 0);
  }
};

// Per-thread plan for staging one K/V tile.  V, and the K chunks outside the
// rotary dims, go global -> LDS directly (lane l of a wave writes position
// 64*block + l, so each lane fetches the global chunk that belongs there;
// offsets are 32-bit element offsets from the tile's first row).  The rotary
// K dims go through registers as "pair items" (row, W consecutive pairs: dims
// p0.. and half+p0..) and are rotated before being written to LDS; for rotary
// widths that are not a multiple of 8 every K chunk goes through registers
// (rotated element-wise).
template <int D, int ROT>
struct TilePlan {
  static constexpr int BN = FwdTile<D>::BN;
  static constexpr int CPR = D / 8;             // chunks per row
  static constexpr int NB = BN * CPR / 256;     // direct-load blocks per wave (of K and of V)
  static_assert(BN * CPR % 256 == 0, "a tile is whole 1 KB blocks for every wave");
  static constexpr bool PAIRS = ROT == 1 || ROT == 2;
  static constexpr int W = ROT == 1 ? 8 : 4;    // pairs per pair item
  static constexpr int NPAIR = PAIRS ? (BN * D / (2 * W) + NT - 1) / NT : 1;
  static constexpr int NREG = ROT == 3 ? BN * CPR / NT : 1;
  int kdirect;            // bit i: this lane's K position of block i is loaded directly
  uint32_t koff[NB], voff[NB];  // byte offsets (row * stride + 8 * chunk) * 2 from the tile start
  int pitem[NPAIR];       // row << 8 | p0, -1 unused
  int plds[NPAIR];        // LDS element offsets of dims p0.. (low 16 bits) and half+p0..
  u32x4 plo[NPAIR], phi[NPAIR];
  int ritem[NREG];        // ROT 3: row << 8 | chunk
  u32x4 rk[NREG];

  __device__ __forceinline__ static int kp(int row, int chunk) {
    return row * CPR + (chunk ^ Swz<D>::k(row));
  }

  __device__ __forceinline__ void init(int wave, int lane, int tid, int rd, int64_t ks,
                                       int64_t vs) {
    const int rchunks = PAIRS ? rd / 8 : (ROT == 3 ? CPR : 0);  // K chunks not loaded directly
    kdirect = 0;
#pragma unroll
    for (int i = 0; i < NB; ++i) {
      const int P = 64 * (wave + 4 * i) + lane;
      const int row = P / CPR;
      const int ck = (P % CPR) ^ Swz<D>::k(row);
      const int cv = (P % CPR) ^ Swz<D>::v(row);
      if (ck >= rchunks) kdirect |= 1 << i;
      koff[i] = 2u * (uint32_t)(row * ks + 8 * ck);
      voff[i] = 2u * (uint32_t)(row * vs + 8 * cv);
    }
    const int half = rd >> 1;
    const int slots = PAIRS ? half / W : 0;
#pragma unroll
    for (int i = 0; i < NPAIR; ++i) {
      const int it = tid + NT * i;
      if (PAIRS && it < BN * slots) {
        const int row = it / slots, p0 = (it % slots) * W;
        pitem[i] = (row << 8) | p0;
        const int lo = kp(row, p0 >> 3) * 8 + (p0 & 7);
        const int hi = kp(row, (half + p0) >> 3) * 8 + ((half + p0) & 7);
        plds[i] = lo | (hi << 16);
      } else {
        pitem[i] = -1;
        plds[i] = 0;
      }
    }
#pragma unroll
    for (int i = 0; i < NREG; ++i) {
      const int it = tid + NT * i;
      ritem[i] = ROT == 3 ? ((it / CPR) << 8) | (it % CPR) : -1;
    }
  }

  // Issues the direct loads of tile rows [k0, k0 + BN) into Kt / Vt (rows past
  // S repeat row S-1; those keys are masked) and fetches the register items.
  __device__ __forceinline__ void fetch(const uint16_t* __restrict__ kb, int64_t ks,
                                        const uint16_t* __restrict__ vb, int64_t vs, int k0,
                                        int S, int rd, uint16_t* Kt, uint16_t* Vt, int wave) {
    // uniform tile base (buffer resource) + 32-bit per-lane byte offset
    const buf_rsrc kr = raw_rsrc(kb + (int64_t)k0 * ks);
    const buf_rsrc vr = raw_rsrc(vb + (int64_t)k0 * vs);
    if (k0 + BN <= S) {
#pragma unroll
      for (int i = 0; i < NB; ++i) {
        const int blk = wave + 4 * i;
        dma16(vr, voff[i], Vt + 512 * blk);
        if (kdirect & (1 << i)) dma16(kr, koff[i], Kt + 512 * blk);
      }
    } else {
      // last tile: rows past S re-read row S-1 (their keys are masked)
      const int lane = threadIdx.x & 63;
#pragma unroll
      for (int i = 0; i < NB; ++i) {
        const int blk = wave + 4 * i;
        const int P = 64 * blk + lane;
        const int row = P / CPR;
        const int r = min(k0 + row, S - 1) - k0;
        dma16(vr, 2u * (uint32_t)(r * (int)vs + 8 * ((P % CPR) ^ Swz<D>::v(row))), Vt + 512 * blk);
        if (kdirect & (1 << i))
          dma16(kr, 2u * (uint32_t)(r * (int)ks + 8 * ((P % CPR) ^ Swz<D>::k(row))),
                Kt + 512 * blk);
      }
    }
    const int half = rd >> 1;
    if (PAIRS) {
#pragma unroll
      for (int i = 0; i < NPAIR; ++i) {
        if (pitem[i] >= 0) {
          const int row = pitem[i] >> 8, p0 = pitem[i] & 255;
          const int r = min(k0 + row, S - 1);
          const uint16_t* src = kb + (int64_t)r * ks + p0;
          if (W == 8) {
            plo[i] = *reinterpret_cast<const u32x4*>(src);
            phi[i] = *reinterpret_cast<const u32x4*>(src + half);
          } else {
            const u32x2 a = *reinterpret_cast<const u32x2*>(src);
            const u32x2 b = *reinterpret_cast<const u32x2*>(src + half);
            plo[i] = u32x4{a[0], a[1], 0u, 0u};
            phi[i] = u32x4{b[0], b[1], 0u, 0u};
          }
        }
      }
    }
    if (ROT == 3) {
#pragma unroll
      for (int i = 0; i < NREG; ++i) {
        const int row = ritem[i] >> 8, c = ritem[i] & 255;
        const int r = min(k0 + row, S - 1);
        rk[i] = *reinterpret_cast<const u32x4*>(kb + (int64_t)r * ks + 8 * c);
      }
    }
  }

  // Rotates the register items (angle of each row's position) into Kt.
  __device__ __forceinline__ void store(uint16_t* Kt, const uint16_t* __restrict__ kb, int64_t ks,
                                        int k0, int S, int rd, const float2* __restrict__ rope) {
    const int half = rd >> 1;
    if (PAIRS) {
#pragma unroll
      for (int i = 0; i < NPAIR; ++i) {
        if (pitem[i] >= 0) {
          const int row = pitem[i] >> 8, p0 = pitem[i] & 255;
          const int pos = min(k0 + row, S - 1);
          const f32x4* cs = reinterpret_cast<const f32x4*>(rope + (int64_t)pos * half + p0);
          uint32_t lo[W / 2], hi[W / 2];
#pragma unroll
          for (int e2 = 0; e2 < W / 2; ++e2) {
            const f32x4 c = cs[e2];  // (cos, sin) of pairs p0 + 2 e2 and p0 + 2 e2 + 1
            const uint32_t a = plo[i][e2], bw = phi[i][e2];
            const float x1a = el_lo(a), x1b = el_hi(a), x2a = el_lo(bw), x2b = el_hi(bw);
            lo[e2] = pack2(x1a * c[0] - x2a * c[1], x1b * c[2] - x2b * c[3]);
            hi[e2] = pack2(x2a * c[0] + x1a * c[1], x2b * c[2] + x1b * c[3]);
          }
          uint16_t* dlo = Kt + (plds[i] & 0xffff);
          uint16_t* dhi = Kt + (plds[i] >> 16);
          if (W == 8) {
            *reinterpret_cast<u32x4*>(dlo) = u32x4{lo[0], lo[1], lo[2], lo[3]};
            *reinterpret_cast<u32x4*>(dhi) = u32x4{hi[0], hi[1], hi[2], hi[3]};
          } else {
            *reinterpret_cast<u32x2*>(dlo) = u32x2{lo[0], lo[1]};
            *reinterpret_cast<u32x2*>(dhi) = u32x2{hi[0], hi[1]};
          }
        }
      }
    }
    if (ROT == 3) {
#pragma unroll
      for (int i = 0; i < NREG; ++i) {
        const int row = ritem[i] >> 8, c = ritem[i] & 255;
        const int r = min(k0 + row, S - 1);
        u32x4 w = rk[i];
        if (8 * c < rd) {
          float x[8];
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            x[2 * e] = el_lo(w[e]);
            x[2 * e + 1] = el_hi(w[e]);
          }
          rotate8_scalar(kb + (int64_t)r * ks, 8 * c, x, r, rd, rope);
          w = u32x4{pack2(x[0], x[1]), pack2(x[2], x[3]), pack2(x[4], x[5]), pack2(x[6], x[7])};
        }
        *reinterpret_cast<u32x4*>(Kt + 8 * kp(row, c)) = w;
      }
    }
  }
};

// Workgroups per CU the register budget is sized for: 3 (at most 168
// registers per lane) for the plain-K form at D <= 96 and with 32-key tiles,
// else 2.  The rotating forms need more registers.
template <int D, int ROT>
struct FwdOccupancy {
  static constexpr int value = (ROT == 0 && (D <= 96 || FwdTile<D>::BN == 32)) ? 3 : 2;
};

// (K, V) buffer pairs: three for the plain-K form with 32-key tiles, whose
// third pair fits in the LDS the Q~ staging needs anyway (tiles then load two
// ahead, and the end-of-tile wait leaves the newest tile's loads in flight),
// else two.  (With 64-key tiles at D = 64 a third pair fits too but measured
// no faster.)
template <int D, int ROT>
struct FwdBuffers {
  static constexpr int value = (ROT == 0 && FwdTile<D>::BN == 32) ? 3 : 2;
  static constexpr int LDS = FwdTile<D>::LDS > 2 * value * FwdTile<D>::TILE
                                 ? FwdTile<D>::LDS
                                 : 2 * value * FwdTile<D>::TILE;
};

// State of one workgroup's forward pass (one wave's view).
template <int D, int ROT, bool ALIBI>
struct FwdState {
  static constexpr int CPR = D / 8;
  static constexpr int BN = FwdTile<D>::BN;
  static constexpr int KB = FwdTile<D>::KB;
  static constexpr int TILE = FwdTile<D>::TILE;
  static constexpr int NBUF = FwdBuffers<D, ROT>::value;
  // The three-buffer wait counts this wave's direct loads of one tile; only
  // the plain-K form issues no other vector memory loads inside the loop.
  static_assert(NBUF == 2 || ROT == 0, "three buffers need the plain-K form");
  uint16_t* lds;
  TilePlan<D, ROT> tp;
  elem8 qreg[D / 16];
  f32x16 oacc[D / 32];
  float m_ref, l_run;
  // LDS element offsets of this lane's operand reads, from the start of a
  // K or V tile buffer.
  int kaddr[D / 16];     // K~ A operand, rows 0..31 (per chunk pair); rows 32..63
                         // (a second score block) use the same swizzle, 32 * D
                         // elements further
  int vaddr[D / 32];     // V^T transposed reads (per dim block)
  int lo, hi, qi, hh, wave;
  float c2, sl2;

  // One tile read from LDS buffer pair `buf`; fetches tile kt + NBUF - 1 (if
  // any) into the pair read by the previous tile meanwhile.
  __device__ __forceinline__ void step(const FwdParams& p, const uint16_t* kb,
                                       const uint16_t* vb, int kt, int kt_hi, int buf) {
    const int nb = buf == 0 ? NBUF - 1 : buf - 1;
    body(p, kb, vb, kt, kt_hi, lds + buf * 2 * TILE, lds + buf * 2 * TILE + TILE,
         lds + nb * 2 * TILE, lds + nb * 2 * TILE + TILE);
  }
  // The tile buffers come in as distinct restrict pointers, so the compiler
  // knows the operand reads of this tile do not alias the direct-to-LDS loads
  // of the next one still in flight (else every LDS read waits for them).
  __device__ __forceinline__ void body(const FwdParams& p, const uint16_t* kb,
                                       const uint16_t* vb, int kt, int kt_hi,
                                       const uint16_t* __restrict__ Kc,
                                       const uint16_t* __restrict__ Vc,
                                       uint16_t* __restrict__ Kn, uint16_t* __restrict__ Vn) {
    const AttnShape& a = p.a;
    const int S = a.S;
    const int k0 = kt * BN;
    const int kf = k0 + (NBUF - 1) * BN;  // first key of the tile fetched now
    const bool more = kt + NBUF - 1 < kt_hi;
    if (more) tp.fetch(kb, p.sk.s, vb, p.sv.s, kf, S, a.rd, Kn, Vn, wave);

    const bool lane_any = (k0 <= hi) && (k0 + BN - 1 >= lo);
    if (__any(lane_any)) {
      const bool lane_full = (k0 >= lo) && (k0 + BN - 1 <= hi);
      const bool need_mask = !__all(lane_full);
      f32x16 sacc[KB];
#pragma unroll
      for (int blk = 0; blk < KB; ++blk) sacc[blk] = f32x16{};
      // K~ operands are read PF dims steps ahead of the MFMAs using them (two
      // with one score block, so that a read has two products' time to land;
      // one in the ALiBi form, whose bias terms leave no registers for it).
      constexpr int NS = D / 16, PF = (KB == 1 && !ALIBI) ? 2 : 1;
      elem8 kq[PF + 1][KB];
#pragma unroll
      for (int s = 0; s < PF; ++s)
#pragma unroll
        for (int blk = 0; blk < KB; ++blk) kq[s][blk] = lds_read8(Kc + kaddr[s] + 32 * D * blk);
#pragma unroll
      for (int c = 0; c < NS; ++c) {
        if (c + PF < NS) {
#pragma unroll
          for (int blk = 0; blk < KB; ++blk)
            kq[(c + PF) % (PF + 1)][blk] = lds_read8(Kc + kaddr[c + PF] + 32 * D * blk);
        }
        __builtin_amdgcn_sched_barrier(0);  // keep the next operands' reads ahead of these MFMAs
#pragma unroll
        for (int blk = 0; blk < KB; ++blk)
          sacc[blk] = mfma32x32x16(kq[c % (PF + 1)][blk], qreg[c], sacc[blk]);
      }
      // Register r of block blk: key k0 + 32 blk + 8 (r/4) + 4 hh + r%4.  The
      // scores stay in the accumulator registers: raw (RoPE) or exp2-domain
      // with the ALiBi bias (ALiBi).
      if (ALIBI) {
        const float base = sl2 * (float)(k0 + 4 * hh - qi);
#pragma unroll
        for (int blk = 0; blk < KB; ++blk)
#pragma unroll
          for (int r = 0; r < 16; ++r)
            sacc[blk][r] = __builtin_fmaf(
                sacc[blk][r], c2,
                __builtin_fmaf(sl2, (float)(32 * blk + 8 * (r >> 2) + (r & 3)), base));
      }
      if (need_mask) {
        const int jlo = lo - k0 - 4 * hh, jhi = hi - k0 - 4 * hh;  // allowed key offsets
#pragma unroll
        for (int blk = 0; blk < KB; ++blk)
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int ko = 32 * blk + 8 * (r >> 2) + (r & 3);
            if (ko < jlo || ko > jhi) sacc[blk][r] = -INFINITY;
          }
      }
      // Probabilities against the current running max, straight into the
      // packed bf16 B operands; the raw scores stay in sacc.  The tile's row
      // max is only needed when some probability could exceed 2^8: this
      // lane's sum over its 32 keys bounds every one of them, so a sum above
      // 2^8 (or a row without a reference yet) takes the exact path, which
      // raises the running max to the tile max, rescales O and the row sum
      // and exponentiates again.
      elem8 pb[BN / 16];
      float ts = 0.0f;
      auto expo = [&](float mref) {
        ts = 0.0f;
#pragma unroll
        for (int cp = 0; cp < BN / 16; ++cp) {
          float pv[8];
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            const float x = sacc[cp >> 1][8 * (cp & 1) + e];
            pv[e] = ALIBI ? fast_exp2(x - mref) : fast_exp2(__builtin_fmaf(x, c2, -mref));
            ts += pv[e];
          }
          pb[cp] = pack8(pv);
        }
      };
      bool exact = __any(m_ref == -INFINITY);
      if (!exact) {
        expo(m_ref);
        exact = __any(ts > kTileSumLimit);
      }
      if (exact) {
        constexpr int NSC = 16 * KB;  // this lane's scores of the tile
        float mx = fmaxf(sacc[0][0], fmaxf(sacc[0][1], sacc[0][2]));
#pragma unroll
        for (int i = 3; i + 1 < NSC; i += 2)
          mx = fmaxf(mx, fmaxf(sacc[i >> 4][i & 15], sacc[(i + 1) >> 4][(i + 1) & 15]));
        mx = fmaxf(mx, sacc[KB - 1][15]);
        mx = fmaxf(mx, __shfl_xor(mx, 32));
        const float mt = ALIBI ? mx : mx * c2;  // tile max in the exp2 domain
        const float m_new = fmaxf(m_ref, mt);
        const float alpha = m_new == -INFINITY ? 1.0f : fast_exp2(m_ref - m_new);
        l_run *= alpha;
#pragma unroll
        for (int db = 0; db < D / 32; ++db) oacc[db] *= alpha;
        m_ref = m_new;
        expo(m_ref == -INFINITY ? 0.0f : m_ref);
      }
      l_run += ts;
      // V^T operands are read PV products ahead of their use.
      constexpr int NDB = D / 32, NG = (BN / 16) * NDB;
      auto vread = [&](int g) {
        const uint16_t* vp = Vc + vaddr[g % NDB] + 16 * (g / NDB) * 8 * CPR;
        const s16x4 v0 = lds_read_tr4(vp);
        const s16x4 v1 = lds_read_tr4(vp + 8 * 8 * CPR);
        return __builtin_bit_cast(elem8, __builtin_shufflevector(v0, v1, 0, 1, 2, 3, 4, 5, 6, 7));
      };
      constexpr int PV = !ALIBI ? 2 : 1;  // MFMAs ahead
      elem8 vq[PV + 1];
#pragma unroll
      for (int g = 0; g < PV; ++g) vq[g] = vread(g);
#pragma unroll
      for (int g = 0; g < NG; ++g) {
        if (g + PV < NG) vq[(g + PV) % (PV + 1)] = vread(g + PV);
        __builtin_amdgcn_sched_barrier(0);  // keep the next operands' reads ahead of these MFMAs
        oacc[g % NDB] = mfma32x32x16(vq[g % (PV + 1)], pb[g / NDB], oacc[g % NDB]);
      }
    }
    if (more) tp.store(Kn, kb, p.sk.s, kf, S, a.rd, a.rope);
    if (NBUF == 3) {
      // Wait for the next tile's loads only, then the barrier without the
      // release fence of __syncthreads (which, even for LDS alone, would wait
      // for the direct-to-LDS loads still in flight); the acquire fence keeps
      // the next tile's LDS reads below the barrier.
      if (more)
        __builtin_amdgcn_s_waitcnt(waitcnt_vm_lgkm0(2 * TilePlan<D, ROT>::NB));
      else
        __builtin_amdgcn_s_waitcnt(0);
      __builtin_amdgcn_sched_barrier(0);
      __builtin_amdgcn_s_barrier();
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
    } else {
      __builtin_amdgcn_s_waitcnt(0);
      __syncthreads();
    }
  }
};

// ROT: how K tiles are staged (0: plain or pre-rotated K; 1, 2: rotary pair
// items; 3: every chunk through registers).  QROT: rotate Q~ at load.
template <int D, int ROT, bool ALIBI, bool QROT>
__global__ __launch_bounds__(NT, (FwdOccupancy<D, ROT>::value)) void fwd_bf16_kernel(FwdParams p) {
  constexpr int CPR = D / 8;
  constexpr int BN = FwdTile<D>::BN;
  constexpr int TILE = FwdTile<D>::TILE;  // elements per tile buffer (unpadded, swizzled)
  constexpr int NBUF = FwdBuffers<D, ROT>::value;
  __shared__ __attribute__((aligned(16))) uint16_t lds[FwdBuffers<D, ROT>::LDS];  // K0 V0 K1 V1 .. (+ Q~ staging)

  const AttnShape& a = p.a;
  const int S = a.S;
  const int nqt = (S + BM - 1) / BM;
  const int BH = a.B * a.H;
  const int qt = nqt - 1 - (int)(blockIdx.x / BH);  // heaviest q-tile first, heads fastest
  const int bh = (int)(blockIdx.x % BH);
  const int b = bh / a.H, h = bh % a.H;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // uniform: LDS bases stay scalar
  const int ql = lane & 31, hh = lane >> 5;
  const int q0 = qt * BM;

  FwdState<D, ROT, ALIBI> st;
  st.lds = lds;
  st.wave = wave;
  st.hh = hh;
  st.qi = q0 + wave * 32 + ql;  // this lane's query row
  const int qi = st.qi;

  const uint16_t* qb = (const uint16_t*)p.q + b * p.sq.b + h * p.sq.h;
  const uint16_t* kb = (const uint16_t*)p.k + b * p.sk.b + h * p.sk.h;
  const uint16_t* vb = (const uint16_t*)p.v + b * p.sv.b + h * p.sv.h;

  // Allowed keys of this lane's query: [lo, hi].
  const int32_t* drow = a.docs ? a.docs + (int64_t)b * (a.n_docs + 1) : nullptr;
  const int qc = qi < S ? qi : S - 1;
  st.lo = 0;
  st.hi = S - 1;
  if (drow) {
    int ds, de;
    doc_bounds(drow, a.n_docs, S, qc, ds, de);
    st.lo = ds;
    st.hi = de - 1;
  }
  if (a.causal && qi < st.hi) st.hi = qi;
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

  // Prologue: fetch the first tile while Q~ is being loaded.
  st.tp.init(wave, lane, tid, a.rd, p.sk.s, p.sv.s);
  st.tp.fetch(kb, p.sk.s, vb, p.sv.s, kt_lo * BN, S, a.rd, lds, lds + TILE, wave);

  // Q~ of this lane's row as the B operand: chunk c holds dims 16c + 8hh .. +7.
  // Rotation-free: the wave's 32 rows are loaded whole (16 bytes per lane, D / 8
  // lanes per row, rows past S clamped) straight into LDS past the first
  // tile pair, chunk c of row r at position c ^ (r & QSW) (row-wise writes and
  // column-wise reads both conflict-free), and read back in the operand
  // layout after the prologue barrier.
  constexpr int QSW = CPR == 16 ? 15 : (CPR == 8 ? 7 : 3);
  uint16_t* qrows = lds + 2 * TILE + wave * 32 * D;
  if (ROT == 0 && !QROT) {
    const int r0 = q0 + wave * 32;
    const int rb = min(r0, S - 1);  // rows past S re-read row S-1 (never stored)
    const buf_rsrc qr = raw_rsrc(qb + (int64_t)rb * p.sq.s);
#pragma unroll
    for (int i = 0; i < CPR / 2; ++i) {
      const int P = 64 * i + lane, row = P / CPR;
      const int ch = (P % CPR) ^ (row & QSW);
      dma16(qr, 2u * (uint32_t)((min(r0 + row, S - 1) - rb) * (int)p.sq.s + 8 * ch),
            qrows + 512 * i);
    }
  } else {
    const uint16_t* qrow = qb + (int64_t)qc * p.sq.s;
#pragma unroll
    for (int c = 0; c < D / 16; ++c) {
      const int d0 = 16 * c + 8 * hh;
      float x[8];
      const u32x4 w = *reinterpret_cast<const u32x4*>(qrow + d0);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        x[2 * e] = el_lo(w[e]);
        x[2 * e + 1] = el_hi(w[e]);
      }
      if (QROT) rotate8_scalar(qrow, d0, x, qc, a.rd, a.rope);
      if (qi >= S) {
#pragma unroll
        for (int e = 0; e < 8; ++e) x[e] = 0.0f;
      }
      st.qreg[c] = pack8(x);
    }
  }
  // LDS operand offsets.  K~ A operand: row ql (+32 per block), chunk 2c + hh.
  // V^T via transposed reads: lane 16g + j reads 4 dims (chunk 4 db + 2 (g&1) +
  // (j&3)/2, half (j&1)) of key 16 cp + 4 hh + j/4 (+8).
#pragma unroll
  for (int c = 0; c < D / 16; ++c) st.kaddr[c] = 8 * (ql * CPR + ((2 * c + hh) ^ Swz<D>::k(ql)));
  {
    const int g16 = lane >> 4, j16 = lane & 15;
    const int vkey = 4 * hh + (j16 >> 2);
    const int vsw = Swz<D>::v(vkey);  // same for keys vkey + 16 cp and vkey + 8
    const int vch = 2 * (g16 & 1) + ((j16 & 3) >> 1);
#pragma unroll
    for (int db = 0; db < D / 32; ++db)
      st.vaddr[db] = 8 * (vkey * CPR + ((4 * db + vch) ^ vsw)) + 4 * (j16 & 1);
  }
  st.tp.store(lds, kb, p.sk.s, kt_lo * BN, S, a.rd, a.rope);
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  if (ROT == 0 && !QROT) {
#pragma unroll
    for (int c = 0; c < D / 16; ++c)
      st.qreg[c] = qi < S ? lds_read8(qrows + ql * D + 8 * ((2 * c + hh) ^ (ql & QSW))) : elem8{};
    __syncthreads();  // every wave has its Q~ before the first fetch reuses the buffer
  }
  if (NBUF == 3 && kt_lo + 1 < kt_hi)
    st.tp.fetch(kb, p.sk.s, vb, p.sv.s, (kt_lo + 1) * BN, S, a.rd, lds + 2 * TILE, lds + 3 * TILE,
                wave);

  st.sl2 = ALIBI ? alibi_slope_log2(a, h) : 0.0f;
  st.c2 = a.scale_log2;
  st.m_ref = -INFINITY;  // running max in the exp2 domain (raised lazily)
  st.l_run = 0.0f;       // this lane's partial row sum (its 16 keys per block)
#pragma unroll
  for (int db = 0; db < D / 32; ++db) st.oacc[db] = f32x16{};

  int buf = 0;
  for (int kt = kt_lo; kt < kt_hi; ++kt) {
    st.step(p, kb, vb, kt, kt_hi, buf);
    buf = buf + 1 == NBUF ? 0 : buf + 1;
  }

  // Epilogue: o = O / l, lse = (m + log2 l) ln 2.
  const float l_tot = st.l_run + __shfl_xor(st.l_run, 32);
  const float inv_l = l_tot > 0.0f ? 1.0f / l_tot : 0.0f;
  if (qi < S) {
    if (hh == 0) p.lse[(int64_t)bh * S + qi] = (st.m_ref + __log2f(l_tot)) * kLn2;
    // Register r of block db holds dim 32 db + 8 (r/4) + 4 hh + r%4.
    if (p.out_f32) {
      float* orow = (float*)p.o + b * p.so.b + h * p.so.h + (int64_t)qi * p.so.s;
#pragma unroll
      for (int db = 0; db < D / 32; ++db)
#pragma unroll
        for (int a4 = 0; a4 < 4; ++a4) {
          f32x4 w;
#pragma unroll
          for (int e = 0; e < 4; ++e) w[e] = st.oacc[db][4 * a4 + e] * inv_l;
          *reinterpret_cast<f32x4*>(orow + 32 * db + 8 * a4 + 4 * hh) = w;
        }
    }
  }
  if (!p.out_f32) {
    // o rows through LDS (the tile buffers are free after the last barrier of
    // the loop; each wave uses its own 32 padded rows): whole rows out, 16
    // bytes per lane, instead of 16-byte pieces of 32 rows per store.
    constexpr int RS = D + 8;
    static_assert(4 * 32 * RS <= FwdTile<D>::LDS, "o staging exceeds the LDS array");
    uint16_t* orows = lds + wave * 32 * RS;
    // The lane index passes through an empty asm here, so the address
    // arithmetic below is not hoisted above the loop (where registers are
    // scarcest).
    int el = lane;
    __asm__ volatile("" : "+v"(el));
#pragma unroll
    for (int db = 0; db < D / 32; ++db)
#pragma unroll
      for (int a4 = 0; a4 < 4; ++a4) {
        u32x2 w;
        w[0] = pack2(st.oacc[db][4 * a4] * inv_l, st.oacc[db][4 * a4 + 1] * inv_l);
        w[1] = pack2(st.oacc[db][4 * a4 + 2] * inv_l, st.oacc[db][4 * a4 + 3] * inv_l);
        *reinterpret_cast<u32x2*>(orows + ql * RS + 32 * db + 8 * a4 + 4 * hh) = w;
      }
    uint16_t* ob = (uint16_t*)p.o + b * p.so.b + h * p.so.h;
    const int r0 = q0 + wave * 32;
#pragma unroll
    for (int i = 0; i < CPR / 2; ++i) {
      const int idx = 64 * i + el, row = idx / CPR, ch = idx % CPR;
      const u32x4 w = *reinterpret_cast<const u32x4*>(orows + row * RS + 8 * ch);
      if (r0 + row < S) *reinterpret_cast<u32x4*>(ob + (int64_t)(r0 + row) * p.so.s + 8 * ch) = w;
    }
  }
}

// q~ = R q and k~ = R k for every row, into contiguous bf16 [B][H][S][D]
// buffers (one pass: both use the row's own position).  A wave handles NR
// row groups of one position in RPW * NR heads, so the rotary table entries
// are loaded once for all its rows; every load is issued before the first use.
constexpr int kRopeNR = 2;  // row groups (of RPW heads) per wave in the rotation pass

template <int D>
__global__ __launch_bounds__(256) void rope_qk_kernel(FwdParams p) {
  using RG = RowGroups<D>;
  constexpr int C = RG::C, G = RG::G, RPW = RG::RPW, NR = kRopeNR;
  __shared__ __attribute__((aligned(16))) uint16_t rowbuf[4][NR][RPW][2][D];
  const AttnShape& a = p.a;
  const int S = a.S, rd = a.rd, half = rd >> 1;
  const int BH = a.B * a.H;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int g = lane & (G - 1), rw = lane / G;
  const int wid = blockIdx.x * 4 + wave;
  const int i = wid % S, bh0 = (wid / S) * (RPW * NR);  // position; first head of the wave
  if (bh0 >= BH) return;  // whole waves only
  const int d0 = 8 * g;
  int r[NR];
  bool act[NR];
  u32x4 w[NR][2];
  float2 cs[8];
  if (g < C && d0 < rd) rope_entries8(a.rope + (int64_t)i * half, d0, half, rd, cs);
#pragma unroll
  for (int n = 0; n < NR; ++n) {
    const int bh = bh0 + n * RPW + rw;
    r[n] = bh * S + i;
    act[n] = bh < BH && g < C;
    const int b = bh / a.H, h = bh - b * a.H;
    w[n][0] = w[n][1] = u32x4{0u, 0u, 0u, 0u};
    if (act[n]) {
      w[n][0] = *reinterpret_cast<const u32x4*>((const uint16_t*)p.q + b * p.sq.b + h * p.sq.h +
                                                (int64_t)i * p.sq.s + d0);
      w[n][1] = *reinterpret_cast<const u32x4*>((const uint16_t*)p.k + b * p.sk.b + h * p.sk.h +
                                                (int64_t)i * p.sk.s + d0);
    }
  }
#pragma unroll
  for (int n = 0; n < NR; ++n)
    if (act[n]) {
      *reinterpret_cast<u32x4*>(&rowbuf[wave][n][rw][0][d0]) = w[n][0];
      *reinterpret_cast<u32x4*>(&rowbuf[wave][n][rw][1][d0]) = w[n][1];
    }
  lds_wave_sync();
#pragma unroll
  for (int n = 0; n < NR; ++n) {
    if (!act[n]) continue;
    if (d0 < rd) {
#pragma unroll
      for (int t = 0; t < 2; ++t) {
        float x[8];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          x[2 * e] = el_lo(w[n][t][e]);
          x[2 * e + 1] = el_hi(w[n][t][e]);
        }
        const uint16_t* prow = rowbuf[wave][n][rw][t];
        if ((rd & 7) == 0) {
          // The chunk lies inside the rotary dims, and half is a multiple of 4:
          // each 4-dim group of it has its partners in one 8-byte-aligned
          // group on the other side of half, read whole; rotate-half negates
          // the partners of the first half (sign bits flipped in place).
#pragma unroll
          for (int g4 = 0; g4 < 2; ++g4) {
            const int ds = d0 + 4 * g4;
            const bool first = ds < half;
            const u32x2 pw = *reinterpret_cast<const u32x2*>(prow + (first ? ds + half : ds - half));
            const uint32_t flip = first ? 0x80008000u : 0u;
#pragma unroll
            for (int e2 = 0; e2 < 2; ++e2) {
              const uint32_t pv = pw[e2] ^ flip;
              const int e = 4 * g4 + 2 * e2;
              x[e] = fmaf(el_lo(pv), cs[e].y, x[e] * cs[e].x);
              x[e + 1] = fmaf(el_hi(pv), cs[e + 1].y, x[e + 1] * cs[e + 1].x);
            }
          }
        } else {
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            const int d = d0 + e;
            if (d < rd) {
              const bool first = d < half;
              const float sn = first ? -cs[e].y : cs[e].y;  // rotate-half: (-x2, x1)
              x[e] = fmaf(el2f(prow[first ? d + half : d - half]), sn, x[e] * cs[e].x);
            }
          }
        }
        w[n][t] = u32x4{pack2(x[0], x[1]), pack2(x[2], x[3]), pack2(x[4], x[5]), pack2(x[6], x[7])};
      }
    }
    *reinterpret_cast<u32x4*>(p.qrot + (int64_t)r[n] * D + d0) = w[n][0];
    *reinterpret_cast<u32x4*>(p.krot + (int64_t)r[n] * D + d0) = w[n][1];
  }
}

template <int D, int ROT, bool ALIBI, bool QROT>
hipError_t launch_d(const FwdParams& p, hipStream_t st) {
  const int nqt = (p.a.S + BM - 1) / BM;
  const dim3 grid((unsigned)(nqt * p.a.B * p.a.H));
  hipLaunchKernelGGL((fwd_bf16_kernel<D, ROT, ALIBI, QROT>), grid, dim3(NT), 0, st, p);
  return hipGetLastError();
}

template <int D>
hipError_t launch_dim(const FwdParams& p, hipStream_t st, const hipEvent_t* ev) {
  hipError_t e;
  const FwdPlan plan = fwd_plan16(p.a.rd, p.a.alibi != 0, p.qrot != nullptr);
  if (plan.alibi) {  // ALiBi runs without rotary
    if ((e = record_event(ev, 1, st)) != hipSuccess) return e;
    return launch_d<D, 0, true, false>(p, st);
  }
  if (plan.rotation_pass) {
    // one wave per (position, group of kRopeNR * RPW heads), four waves per block
    const int64_t hpw = kRopeNR * RowGroups<D>::RPW;
    const int64_t waves = (p.a.B * p.a.H + hpw - 1) / hpw * p.a.S;
    const dim3 grid((unsigned)((waves + 3) / 4));
    hipLaunchKernelGGL((rope_qk_kernel<D>), grid, dim3(256), 0, st, p);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    if ((e = record_event(ev, 1, st)) != hipSuccess) return e;
    FwdParams q = p;
    const Strides dense{(int64_t)p.a.H * p.a.S * D, (int64_t)p.a.S * D, D};
    q.q = p.qrot;
    q.sq = dense;
    q.k = p.krot;
    q.sk = dense;
    return launch_d<D, 0, false, false>(q, st);
  }
  if ((e = record_event(ev, 1, st)) != hipSuccess) return e;
  switch (plan.rot_mode) {
    case 1: return launch_d<D, 1, false, true>(p, st);
    case 2: return launch_d<D, 2, false, true>(p, st);
    case 3: return launch_d<D, 3, false, true>(p, st);
    default: return launch_d<D, 0, false, false>(p, st);
  }
}

}  // namespace
}  // namespace NEOX_ELEM_NS

hipError_t NEOX_ELEM_FN(launch_fwd)(const FwdParams& p, hipStream_t st, const hipEvent_t* ev) {
  using namespace NEOX_ELEM_NS;
  switch (p.a.D) {
    case 64: return launch_dim<64>(p, st, ev);
    case 96: return launch_dim<96>(p, st, ev);
    case 128: return launch_dim<128>(p, st, ev);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace neox
