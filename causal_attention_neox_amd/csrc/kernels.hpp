// Internal interface between the C-ABI host code and the gfx950 kernels.
// Parameter blocks are passed by value to the kernels; every pointer in them is
// a device pointer.  Launchers return the hipError_t of the launch.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace neox {

// Element strides of one [B, H, S, D] tensor (head dim contiguous).
struct Strides {
  int64_t b, h, s;
};

struct AttnShape {
  int B, H, S, D;
  int rd;                 // rotary dims (0 = none)
  const float2* rope;     // [S][rd/2] (cos, sin) or null when rd == 0
  float scale;            // softmax scale
  float scale_log2;       // softmax scale * log2(e)
  int causal;
  int alibi;              // 1: add -slope*(i-j)
  const float* slopes;    // [H] or null (then 2^(-8(h+1)/H))
  const int32_t* docs;    // [B][n_docs+1] or null
  int n_docs;
};

struct FwdParams {
  AttnShape a;
  const void* q;
  const void* k;
  const void* v;
  void* o;
  float* lse;
  Strides sq, sk, sv, so;
  int out_f32;     // o stored as fp32
  uint16_t* qrot;  // 16-bit [B][H][S][D] workspace parts for q~ = R q and k~ = R k,
  uint16_t* krot;  // or null (16-bit paths; rotation then happens in the kernel)
};

struct BwdParams {
  AttnShape a;
  const void* q;
  const void* k;
  const void* v;
  const void* o;
  const void* dout;
  const float* lse;
  void* dq;
  void* dk;
  void* dv;
  float* dq_acc;   // [B][H][S][D] fp32 workspace (contiguous; fp32 path only)
  float* delta;    // [B][H][S] fp32 workspace: dO_i . o_i
  float* nlse;     // [B][H][S] fp32 workspace: -lse_i * log2(e) (ALiBi: also - slope * log2(e) * i)
  uint16_t* qrot;  // [B][H][S][D] 16-bit workspace: rotated q (16-bit paths with rotary)
  uint16_t* krot;  // [B][H][S][D] 16-bit workspace: rotated k
  Strides sq, sk, sv, so, sdo, sdq, sdk, sdv;
  int out_f32;     // dq, dk, dv stored as fp32
  int qk_ready;    // qrot / krot already hold R q and R k (written by the forward)
};

// One decoding step: the new token of every (batch, head) against its cache.
struct DecodeParams {
  int B, H, D, cap;       // cache rows hold positions 0 .. cap-1
  int rd;                 // rotary dims (0 = none)
  const float2* rope;     // [cap][rd/2] (cos, sin) or null when rd == 0
  float scale_log2;       // softmax scale * log2(e)
  int dtype;              // storage: 0 fp32, 1 bf16, 2 fp16 (the NEOX_* codes)
  int chunk;              // cache rows per split workgroup (a multiple of decode_tile_rows())
  int nsplit;             // chunks per (batch, head) = ceil(cap / chunk)
  const int32_t* lens;    // [B] tokens already cached = position of the new token
  const void* q;          // [B][H][D] new token, raw
  const void* k;
  const void* v;
  void* k_cache;          // [B][H][cap][D], keys stored rotated
  void* v_cache;
  void* o;                // [B][H][D]
  float* lse;             // [B][H]
  float* part;            // [B][H][nsplit][D + 4] fp32 workspace: m, l, 2 unused, o[D] per chunk
                          // (unused when nsplit == 1)
};

// FP8 (E4M3) forward: q~, k~ (already rotated) and v as E4M3 codes [B][H][S][D],
// contiguous; value = code x per-tensor scale.
struct Fp8FwdParams {
  int B, H, S, D;
  const void* q;
  const void* k;
  const void* v;
  void* o;           // [B][H][S][D] bf16, or fp32 when out_f32
  float* lse;        // [B][H][S]
  float scale_log2;  // softmax scale * q scale * k scale * log2(e)
  float v_scale;
  int causal;
  int out_f32;
};

hipError_t launch_fwd_fp8(const Fp8FwdParams& p, hipStream_t st);

int decode_tile_rows();
void decode_plan(int BH, int cap, int* chunk, int* nsplit);
hipError_t launch_decode(const DecodeParams& p, hipStream_t st);
// Device address of the fixed decode scratch array on `dev` (the current device).
hipError_t decode_scratch(int dev, float** out);

hipError_t launch_rope_table(float2* table, int S, int rd, double base, hipStream_t st);

// Which kernel forms a 16-bit call launches: decided here, on the host, and
// used both by the launchers and by neox_attn_plan.
struct FwdPlan {
  int rotation_pass;  // q~, k~ row pass into the workspace, then the rotation-free kernel
  int rot_mode;       // K staging of the attention kernel: 0 plain or pre-rotated, 1 rotary
                      // pairs 8 wide (rd % 16 == 0), 2 pairs 4 wide (rd % 8 == 0), 3 every
                      // chunk through registers
  int rotate_q;       // the attention kernel rotates Q~ as it loads it
  int alibi;
};
inline FwdPlan fwd_plan16(int rd, bool alibi, bool workspace) {
  FwdPlan f{0, 0, 0, alibi ? 1 : 0};
  if (alibi || rd == 0) return f;
  if (workspace) {
    f.rotation_pass = 1;
    return f;
  }
  f.rotate_q = 1;
  f.rot_mode = rd % 16 == 0 ? 1 : (rd % 8 == 0 ? 2 : 3);
  return f;
}
struct BwdPlan {
  int rotation_pass;  // the backward rotates q and k into the workspace itself
  int alibi;
};
inline BwdPlan bwd_plan16(int rd, bool alibi, bool qk_ready) {
  return BwdPlan{(rd > 0 && !qk_ready) ? 1 : 0, alibi ? 1 : 0};
}

// `ev` is null or 3 events: [0] is recorded by the caller before the call;
// the launcher records [1] after the q/k rotation pass (before the attention
// kernel when there is none); the caller records [2] after the call.
hipError_t launch_fwd_bf16(const FwdParams& p, hipStream_t st, const hipEvent_t* ev);
hipError_t launch_fwd_f16(const FwdParams& p, hipStream_t st, const hipEvent_t* ev);
hipError_t launch_fwd_f32(const FwdParams& p, hipStream_t st);

// `ev` is null or 4 events: before the first kernel, after the preprocess
// kernel (if any), after the dQ kernel (16-bit paths: dQ runs first and also
// writes Delta and nlse) or the fp32 main kernels, and at the end.
hipError_t launch_bwd_bf16(const BwdParams& p, hipStream_t st, const hipEvent_t* ev);
hipError_t launch_bwd_f16(const BwdParams& p, hipStream_t st, const hipEvent_t* ev);
hipError_t launch_bwd_f32(const BwdParams& p, hipStream_t st, const hipEvent_t* ev);

inline hipError_t record_event(const hipEvent_t* ev, int i, hipStream_t st) {
  return ev ? hipEventRecord(ev[i], st) : hipSuccess;
}

}  // namespace neox
