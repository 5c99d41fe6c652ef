// FP8 (E4M3) forward attention on gfx950: q~, k~, v stored as E4M3 codes with
// one scale per tensor, both products on v_mfma_f32_32x32x64_f8f6f4 (64-deep
// FP8 MFMA, fp32 accumulation), softmax in fp32.  FP8 compute is what the
// GPT-NeoX training stack gets from Transformer Engine ("GPT-NeoX 开源训练框架深度解读",
// the TE image); the attention itself is the same exact tiled form as the
// 16-bit forward.
//
//  * Workgroup = 4 waves = 128 query rows of one (batch, head); K/V tiles of 64
//    keys.  S^T = K~ Q~^T: A = 32 key rows x 64 dims from LDS, B = Q~ (this
//    lane's query, 32 dims per lane half) held in registers; D = 96 pads the
//    second 64-dim step with zeros in the upper lane half.
//  * The FP8 MFMA pairs the two operands' bytes through the same (lane half,
//    byte) -> k map, so any k order works as long as A and B agree.  The
//    probabilities are used straight from the score registers: lane half hh,
//    byte j = 16 b + r holds key 32 b + 8 (r / 4) + 4 hh + r % 4 of the tile.
//    V is transposed on its way into LDS (4 x 4 byte blocks through v_perm)
//    into rows of one dim with the keys in exactly that order, so the A
//    operand of O^T += V^T P^T is two 16-byte reads.
//  * P is stored as 2^4 P in E4M3 (round to nearest even), taken against the
//    running max; a lane's tile sum above 2^8 (checked before use) raises the
//    max first (D = 128: the tile max is found every tile and the running max
//    raised when it grows by more than 2^4), so every 2^4 P <= 2^8 stays inside
//    E4M3's range (448), and the same 2^4 cancels between O and the row sum.
//  * Rows are padded by 16 bytes (K: D + 16, V^T: 64 + 16) so that the 16-byte
//    operand reads of 8 consecutive lanes fall on distinct banks.  The next
//    tile is loaded into registers while the current one is used, then
//    written to the other LDS buffer: one barrier per tile.
#include "device_common.hpp"

namespace neox {
namespace {

typedef int i32x8 __attribute__((ext_vector_type(8)));

constexpr int F8_BM = 128;           // queries per workgroup
constexpr int F8_BN = 64;            // keys per tile
constexpr int F8_NT = 256;           // threads per workgroup
constexpr float kPShift = 4.0f;      // P stored as 2^4 P
constexpr float kF8SumLimit = 256.0f;  // a lane's tile sum of 2^4 P before the max is raised

template <int D>
struct F8Tile {
  static constexpr int KS = D + 16;              // K row stride (bytes)
  static constexpr int VS = F8_BN + 16;          // V^T row stride (bytes)
  static constexpr int KBYTES = F8_BN * KS;
  static constexpr int BUF = KBYTES + D * VS;    // one buffer: K rows, then V^T rows
  static constexpr int NC = (D + 63) / 64;       // 64-deep steps of the QK product
  static constexpr int NITEM = F8_BN * D / 16;   // 16-byte K chunks = 4 x 4 V blocks per tile
  static constexpr int NPT = (NITEM + F8_NT - 1) / F8_NT;  // items per thread
};

__device__ __forceinline__ f32x16 mfma_f8(const i32x8& a, const i32x8& b, const f32x16& c) {
  // cbsz = blgp = 0: both operands E4M3; no block scales.
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 0, 0, 0, 0, 0);
}

__device__ __forceinline__ i32x8 lds_read32(const uint8_t* p) {
  const u32x4 x = *reinterpret_cast<const u32x4*>(p);
  const u32x4 y = *reinterpret_cast<const u32x4*>(p + 16);
  return i32x8{(int)x[0], (int)x[1], (int)x[2], (int)x[3], (int)y[0], (int)y[1], (int)y[2], (int)y[3]};
}

template <int D>
__global__ __launch_bounds__(F8_NT, 2) void fwd_fp8_kernel(Fp8FwdParams p) {
  using T = F8Tile<D>;
  __shared__ __attribute__((aligned(16))) uint8_t lds[2 * T::BUF];

  const int S = p.S;
  const int nqt = (S + F8_BM - 1) / F8_BM;
  const int BH = p.B * p.H;
  const int qt = nqt - 1 - (int)(blockIdx.x / BH);  // heaviest q-tile first, heads fastest
  const int bh = (int)(blockIdx.x % BH);
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int ql = lane & 31, hh = lane >> 5;
  const int q0 = qt * F8_BM;
  const int qi = q0 + wave * 32 + ql;  // this lane's query row
  const int qc = qi < S ? qi : S - 1;
  const int hi = p.causal ? qc : S - 1;  // last allowed key of this row
  const int qlast = q0 + F8_BM - 1 < S - 1 ? q0 + F8_BM - 1 : S - 1;
  const int kt_hi = (p.causal ? qlast : S - 1) / F8_BN + 1;
  // Tiles every row of the workgroup sees in full need no mask.
  const int k_full = p.causal ? q0 : S;  // keys [0, k_full) are allowed for every row

  const uint8_t* qb = (const uint8_t*)p.q + (int64_t)bh * S * D;
  const uint8_t* kb = (const uint8_t*)p.k + (int64_t)bh * S * D;
  const uint8_t* vb = (const uint8_t*)p.v + (int64_t)bh * S * D;

  // Tile loader: item n of this thread is a 16-byte K chunk (row n / (D/16),
  // chunk n % (D/16)) and a 4 x 4 block of V (keys 4 (n / (D/4)) .., dims
  // 4 (n % (D/4)) ..).  Rows past S re-read row S - 1 (masked, or weighted 0).
  u32x4 kr[T::NPT];
  uint32_t vr[T::NPT][4];
  auto fetch = [&](int t) {
    const int k0 = t * F8_BN;
#pragma unroll
    for (int i = 0; i < T::NPT; ++i) {
      const int n = tid + i * F8_NT;
      if (n < T::NITEM) {
        const int kr_row = n / (D / 16), kr_c = n % (D / 16);
        const int key = min(k0 + kr_row, S - 1);
        kr[i] = *reinterpret_cast<const u32x4*>(kb + (int64_t)key * D + 16 * kr_c);
        const int kq = n / (D / 4), dq = n % (D / 4);
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int vk = min(k0 + 4 * kq + j, S - 1);
          vr[i][j] = *reinterpret_cast<const uint32_t*>(vb + (int64_t)vk * D + 4 * dq);
        }
      }
    }
  };
  auto store = [&](uint8_t* buf) {
#pragma unroll
    for (int i = 0; i < T::NPT; ++i) {
      const int n = tid + i * F8_NT;
      if (n < T::NITEM) {
        const int kr_row = n / (D / 16), kr_c = n % (D / 16);
        *reinterpret_cast<u32x4*>(buf + kr_row * T::KS + 16 * kr_c) = kr[i];
        // 4 x 4 byte transpose: out[d] = byte d of keys 0..3.
        const uint32_t w0 = vr[i][0], w1 = vr[i][1], w2 = vr[i][2], w3 = vr[i][3];
        const uint32_t a_lo = __builtin_amdgcn_perm(w1, w0, 0x05010400u);  // w0.0 w1.0 w0.1 w1.1
        const uint32_t a_hi = __builtin_amdgcn_perm(w1, w0, 0x07030602u);  // w0.2 w1.2 w0.3 w1.3
        const uint32_t b_lo = __builtin_amdgcn_perm(w3, w2, 0x05010400u);
        const uint32_t b_hi = __builtin_amdgcn_perm(w3, w2, 0x07030602u);
        const uint32_t o0 = __builtin_amdgcn_perm(b_lo, a_lo, 0x05040100u);
        const uint32_t o1 = __builtin_amdgcn_perm(b_lo, a_lo, 0x07060302u);
        const uint32_t o2 = __builtin_amdgcn_perm(b_hi, a_hi, 0x05040100u);
        const uint32_t o3 = __builtin_amdgcn_perm(b_hi, a_hi, 0x07060302u);
        // Keys 4 kq .. 4 kq + 3 sit at byte (half) 32 + 16 b + 4 g of each V^T row,
        // with key = 32 b + 8 g + 4 half + (0..3).
        const int kq = n / (D / 4), dq = n % (D / 4);
        const int key = 4 * kq;
        const int pos = 32 * ((key >> 2) & 1) + 16 * (key >> 5) + 4 * ((key >> 3) & 3);
        uint8_t* vrow = buf + T::KBYTES + (4 * dq) * T::VS + pos;
        *reinterpret_cast<uint32_t*>(vrow) = o0;
        *reinterpret_cast<uint32_t*>(vrow + T::VS) = o1;
        *reinterpret_cast<uint32_t*>(vrow + 2 * T::VS) = o2;
        *reinterpret_cast<uint32_t*>(vrow + 3 * T::VS) = o3;
      }
    }
  };

  fetch(0);

  // Q~ of this lane's row as the B operand: step c holds dims 64 c + 32 hh .. +31.
  i32x8 qop[T::NC];
  {
    const uint8_t* qrow = qb + (int64_t)qc * D;
#pragma unroll
    for (int c = 0; c < T::NC; ++c) {
      const int d0 = 64 * c + 32 * hh;
      if (d0 < D) {
        const u32x4 x = *reinterpret_cast<const u32x4*>(qrow + d0);
        const u32x4 y = *reinterpret_cast<const u32x4*>(qrow + d0 + 16);
        qop[c] = i32x8{(int)x[0], (int)x[1], (int)x[2], (int)x[3],
                       (int)y[0], (int)y[1], (int)y[2], (int)y[3]};
      } else {
        qop[c] = i32x8{0, 0, 0, 0, 0, 0, 0, 0};
      }
    }
  }

  store(lds);
  if (kt_hi > 1) fetch(1);

  const float c2 = p.scale_log2;
  float m = -INFINITY, l = 0.0f;
  f32x16 oacc[D / 32];
#pragma unroll
  for (int db = 0; db < D / 32; ++db) oacc[db] = f32x16{};

  for (int t = 0; t < kt_hi; ++t) {
    __syncthreads();  // tile t is in LDS; every wave is done with buffer (t + 1) % 2
    const uint8_t* buf = lds + (t & 1) * T::BUF;
    const int k0 = t * F8_BN;

    // K~ operands (key block kb2, 64-dim step c), read one MFMA ahead (D <= 96).
    f32x16 sacc[2] = {f32x16{}, f32x16{}};
    auto kread = [&](int i) {
      const int kb2 = i / T::NC, c = i % T::NC;
      const int d0 = 64 * c + 32 * hh;
      return d0 < D ? lds_read32(buf + (kb2 * 32 + ql) * T::KS + d0)
                    : i32x8{0, 0, 0, 0, 0, 0, 0, 0};
    };
    if constexpr (D <= 96) {
      i32x8 kcur = kread(0);
#pragma unroll
      for (int i = 0; i < 2 * T::NC; ++i) {
        const i32x8 knext = i + 1 < 2 * T::NC ? kread(i + 1) : kcur;
        __builtin_amdgcn_sched_barrier(0);  // keep the next read ahead of this MFMA
        sacc[i / T::NC] = mfma_f8(kcur, qop[i % T::NC], sacc[i / T::NC]);
        kcur = knext;
      }
    } else {  // D = 128: no registers to spare for reading ahead
#pragma unroll
      for (int i = 0; i < 2 * T::NC; ++i)
        sacc[i / T::NC] = mfma_f8(kread(i), qop[i % T::NC], sacc[i / T::NC]);
    }
    // Next tile into the other buffer (its readers finished before this barrier).
    if (t + 1 < kt_hi) {
      store(lds + ((t + 1) & 1) * T::BUF);
      if (t + 2 < kt_hi) fetch(t + 2);
    }

    // Scores in the exp2 domain; mask keys past the row's last allowed key.
    float s[32];
    const bool full = k0 + F8_BN <= k_full;
#pragma unroll
    for (int kb2 = 0; kb2 < 2; ++kb2)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int key = k0 + 32 * kb2 + 8 * (r >> 2) + 4 * hh + (r & 3);
        const float x = sacc[kb2][r] * c2;
        s[16 * kb2 + r] = (full || key <= hi) ? x : -INFINITY;
      }
    // 2^4 P in E4M3, four per dword, in the score registers' key order, taken
    // against the running max without finding the tile max first.  This lane's
    // sum over its 32 keys bounds each value: a sum above 2^8 (or a row
    // without a reference yet) takes the exact path, which raises the running
    // max to the tile max, rescales O and the row sum and converts again, so
    // every stored 2^4 P stays <= 2^8 (E4M3 reaches 448).
    i32x8 pop;
    float ts = 0.0f;
    auto expo = [&](float mref) {
      const float mo = mref - kPShift;
      ts = 0.0f;
#pragma unroll
      for (int w = 0; w < 8; ++w) {
        const float p0 = fast_exp2(s[4 * w] - mo), p1 = fast_exp2(s[4 * w + 1] - mo);
        const float p2 = fast_exp2(s[4 * w + 2] - mo), p3 = fast_exp2(s[4 * w + 3] - mo);
        ts += (p0 + p1) + (p2 + p3);
        int d = __builtin_amdgcn_cvt_pk_fp8_f32(p0, p1, 0, false);
        d = __builtin_amdgcn_cvt_pk_fp8_f32(p2, p3, d, true);
        pop[w] = d;
      }
    };
    if constexpr (D > 96) {
      // D = 128: the two paths do not fit the register budget; find the tile
      // max every tile and raise the running max lazily (by more than 2^4).
      float mx = s[0];
#pragma unroll
      for (int j = 1; j < 32; ++j) mx = fmaxf(mx, s[j]);
      mx = fmaxf(mx, __shfl_xor(mx, 32));
      if (mx > m + kPShift) {
        const float corr = fast_exp2(m - mx);
        l *= corr;
#pragma unroll
        for (int db = 0; db < D / 32; ++db) oacc[db] *= corr;
        m = mx;
      }
      expo(m);
      l += ts;
    } else {
    bool exact = __any(m == -INFINITY);
    if (!exact) {
      expo(m);
      exact = __any(ts > kF8SumLimit);
    }
    if (exact) {
      float mx = s[0];
#pragma unroll
      for (int j = 1; j < 32; ++j) mx = fmaxf(mx, s[j]);
      mx = fmaxf(mx, __shfl_xor(mx, 32));  // the other half holds the row's other keys
      const float m_new = fmaxf(m, mx);
      const float corr = m_new == -INFINITY ? 1.0f : fast_exp2(m - m_new);
      l *= corr;
#pragma unroll
      for (int db = 0; db < D / 32; ++db) oacc[db] *= corr;
      m = m_new;
      expo(m == -INFINITY ? 0.0f : m);
    }
    l += ts;
    }
    auto vread = [&](int db) {
      return lds_read32(buf + T::KBYTES + (db * 32 + ql) * T::VS + 32 * hh);
    };
    if constexpr (D <= 96) {
      i32x8 vcur = vread(0);
#pragma unroll
      for (int db = 0; db < D / 32; ++db) {
        const i32x8 vnext = db + 1 < D / 32 ? vread(db + 1) : vcur;
        __builtin_amdgcn_sched_barrier(0);  // keep the next read ahead of this MFMA
        oacc[db] = mfma_f8(vcur, pop, oacc[db]);
        vcur = vnext;
      }
    } else {
#pragma unroll
      for (int db = 0; db < D / 32; ++db) oacc[db] = mfma_f8(vread(db), pop, oacc[db]);
    }
  }

  // o = O v_scale / l (the 2^4 of P cancels); lse = (m - 4 + log2 l) ln 2.
  const float l_tot = l + __shfl_xor(l, 32);
  if (qi < S) {
    const float mul = p.v_scale / l_tot;
#pragma unroll
    for (int db = 0; db < D / 32; ++db)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int d0 = db * 32 + 8 * g + 4 * hh;
        const float x0 = oacc[db][4 * g] * mul, x1 = oacc[db][4 * g + 1] * mul;
        const float x2 = oacc[db][4 * g + 2] * mul, x3 = oacc[db][4 * g + 3] * mul;
        if (p.out_f32) {
          float* orow = (float*)p.o + ((int64_t)bh * S + qi) * D + d0;
          *reinterpret_cast<f32x4*>(orow) = f32x4{x0, x1, x2, x3};
        } else {
          uint16_t* orow = (uint16_t*)p.o + ((int64_t)bh * S + qi) * D + d0;
          bf16x2 a2, b2;
          a2[0] = (__bf16)x0;
          a2[1] = (__bf16)x1;
          b2[0] = (__bf16)x2;
          b2[1] = (__bf16)x3;
          *reinterpret_cast<u32x2*>(orow) =
              u32x2{__builtin_bit_cast(uint32_t, a2), __builtin_bit_cast(uint32_t, b2)};
        }
      }
    if (hh == 0) p.lse[(int64_t)bh * S + qi] = (m - kPShift + __log2f(l_tot)) * kLn2;
  }
}

template <int D>
hipError_t launch_fp8_d(const Fp8FwdParams& p, hipStream_t st) {
  const int nqt = (p.S + F8_BM - 1) / F8_BM;
  hipLaunchKernelGGL((fwd_fp8_kernel<D>), dim3((unsigned)(nqt * p.B * p.H)), dim3(F8_NT), 0, st,
                     p);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_fwd_fp8(const Fp8FwdParams& p, hipStream_t st) {
  switch (p.D) {
    case 64: return launch_fp8_d<64>(p, st);
    case 96: return launch_fp8_d<96>(p, st);
    case 128: return launch_fp8_d<128>(p, st);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace neox
