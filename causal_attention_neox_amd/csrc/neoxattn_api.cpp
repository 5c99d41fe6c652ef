// Host side of libneoxattn: argument validation, kernel dispatch and the
// per-device rotary cos/sin table cache.  Every exported function is declared
// in include/neoxattn.h, which documents arguments, ownership and errors.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdint>
#include <cstring>
#include <mutex>
#include <vector>

#include "../../include/neoxattn.h"
#include "kernels.hpp"

namespace {

constexpr int64_t kMaxRows = (int64_t)1 << 31;  // B*H*S must stay below 2^31

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }
bool finite_pos(float x) { return std::isfinite(x) && x > 0.0f; }
size_t round256(size_t x) { return (x + 255u) & ~(size_t)255u; }

// ---------------------------------------------------------------- device check

struct DeviceInfo {
  bool checked = false;
  bool ok = false;
};

std::mutex g_mu;
std::vector<DeviceInfo> g_devices;

int check_device(int* dev_out) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return NEOX_E_DEVICE;
  std::lock_guard<std::mutex> lk(g_mu);
  if ((int)g_devices.size() <= dev) g_devices.resize(dev + 1);
  DeviceInfo& info = g_devices[dev];
  if (!info.checked) {
    hipDeviceProp_t prop;
    info.checked = true;
    info.ok = hipGetDeviceProperties(&prop, dev) == hipSuccess &&
              std::strncmp(prop.gcnArchName, "gfx950", 6) == 0;
  }
  *dev_out = dev;
  return info.ok ? NEOX_OK : NEOX_E_DEVICE;
}

// ---------------------------------------------------------------- rotary tables

struct RopeTable {
  int dev;
  int rd;
  uint32_t base_bits;
  int cap;  // positions 0..cap-1
  float2* ptr;
};

std::vector<RopeTable> g_tables;  // never freed: kernels in flight may read them

uint32_t float_bits(float f) {
  uint32_t u;
  std::memcpy(&u, &f, 4);
  return u;
}

// The prepared table of this device covering positions 0..S-1, or
// NEOX_E_NOT_PREPARED.  Compute calls only look tables up: they never
// allocate or wait.
int find_rope_table(int dev, int S, int rd, float base, const float2** out) {
  std::lock_guard<std::mutex> lk(g_mu);
  const uint32_t bb = float_bits(base);
  for (const RopeTable& t : g_tables) {
    if (t.dev == dev && t.rd == rd && t.base_bits == bb && t.cap >= S) {
      *out = t.ptr;
      return NEOX_OK;
    }
  }
  return NEOX_E_NOT_PREPARED;
}

// Builds (allocating) a table covering at least positions 0..S-1 on the null
// stream and waits for it; called by neox_rope_table_prepare only.
int build_rope_table(int dev, int S, int rd, float base, const float2** out) {
  std::lock_guard<std::mutex> lk(g_mu);
  const uint32_t bb = float_bits(base);
  hipStream_t st = nullptr;
  int cap = S;
  for (const RopeTable& t : g_tables) {
    if (t.dev != dev || t.rd != rd || t.base_bits != bb) continue;
    if (t.cap >= S) {
      *out = t.ptr;
      return NEOX_OK;
    }
    if (2 * t.cap > cap) cap = 2 * t.cap;
  }
  cap = (cap + 255) & ~255;
  float2* ptr = nullptr;
  if (hipMalloc(&ptr, (size_t)cap * (size_t)(rd / 2) * sizeof(float2)) != hipSuccess) {
    (void)hipGetLastError();
    return NEOX_E_ALLOC;
  }
  if (neox::launch_rope_table(ptr, cap, rd, (double)base, st) != hipSuccess) return NEOX_E_LAUNCH;
  if (hipStreamSynchronize(st) != hipSuccess) return NEOX_E_DEVICE;
  g_tables.push_back(RopeTable{dev, rd, bb, cap, ptr});
  *out = ptr;
  return NEOX_OK;
}

// ---------------------------------------------------------------- validation

// The backward may take q~, k~ from a workspace the forward left them in.
bool qk_ready(const neox_attn_args* a) {
  return a->reuse_rotated_qk && a->dtype != NEOX_F32 && a->pos == NEOX_POS_ROPE &&
         a->rotary_dim > 0;
}

int validate_common(const neox_attn_args* a) {
  if (!a) return NEOX_E_ARG;
  if (a->B < 1 || a->H < 1 || a->S < 1 || a->D < 1) return NEOX_E_ARG;
  if ((int64_t)a->B * a->H * a->S >= kMaxRows) return NEOX_E_ARG;
  if (a->dtype != NEOX_F32 && a->dtype != NEOX_BF16 && a->dtype != NEOX_F16) return NEOX_E_ARG;
  if (a->pos != NEOX_POS_NONE && a->pos != NEOX_POS_ROPE && a->pos != NEOX_POS_ALIBI)
    return NEOX_E_ARG;
  if (!finite_pos(a->softmax_scale)) return NEOX_E_ARG;
  if (a->out_dtype != NEOX_OUT_SAME && a->out_dtype != NEOX_OUT_F32) return NEOX_E_ARG;
  if (a->pos == NEOX_POS_ROPE) {
    if (a->rotary_dim < 0 || a->rotary_dim > a->D || (a->rotary_dim & 1)) return NEOX_E_ARG;
    if (!finite_pos(a->rope_base)) return NEOX_E_ARG;
  } else if (a->rotary_dim != 0) {
    return NEOX_E_ARG;
  }
  if (a->alibi_slopes && a->pos != NEOX_POS_ALIBI) return NEOX_E_ARG;
  if (a->reuse_rotated_qk != 0 && a->reuse_rotated_qk != 1) return NEOX_E_ARG;
  if (a->doc_offsets) {
    if (a->n_docs < 1 || a->n_docs > (1 << 24)) return NEOX_E_ARG;
    if ((reinterpret_cast<uintptr_t>(a->doc_offsets) & 3u) != 0) return NEOX_E_ALIGN;
  } else if (a->n_docs != 0) {
    return NEOX_E_ARG;
  }
  if (a->alibi_slopes && (reinterpret_cast<uintptr_t>(a->alibi_slopes) & 3u) != 0)
    return NEOX_E_ALIGN;
  if (a->D != 64 && a->D != 96 && a->D != 128) return NEOX_E_UNSUPPORTED;
  return NEOX_OK;
}

// Checks one tensor: pointer present and 16-byte aligned, strides non-negative
// and multiples of the 16-byte unit (`unit` elements), row stride at most 2^22
// elements.
int check_tensor(const void* p, const neox_strides& s, int unit) {
  if (!p) return NEOX_E_ARG;
  if (s.batch < 0 || s.head < 0 || s.seq < 0) return NEOX_E_ARG;
  if (!aligned16(p)) return NEOX_E_ALIGN;
  if (s.batch % unit || s.head % unit || s.seq % unit) return NEOX_E_ALIGN;
  // tile loads address up to 128 rows from a tile's first row with 32-bit
  // byte offsets
  if (s.seq > ((int64_t)1 << 22)) return NEOX_E_UNSUPPORTED;
  return NEOX_OK;
}

neox_strides contiguous(const neox_attn_args* a) {
  const int64_t sd = a->D;
  return neox_strides{(int64_t)a->H * a->S * sd, (int64_t)a->S * sd, sd};
}

neox::Strides to_internal(const neox_strides& s) { return neox::Strides{s.batch, s.head, s.seq}; }

int fill_shape(const neox_attn_args* a, const float2* rope, neox::AttnShape* sh) {
  sh->B = a->B;
  sh->H = a->H;
  sh->S = a->S;
  sh->D = a->D;
  sh->rd = a->pos == NEOX_POS_ROPE ? a->rotary_dim : 0;
  sh->rope = rope;
  sh->scale = a->softmax_scale;
  sh->scale_log2 = a->softmax_scale * 1.4426950408889634f;
  sh->causal = a->causal != 0;
  sh->alibi = a->pos == NEOX_POS_ALIBI;
  sh->slopes = a->alibi_slopes;
  sh->docs = a->doc_offsets;
  sh->n_docs = a->doc_offsets ? a->n_docs : 0;
  return NEOX_OK;
}

int lookup_rope(const neox_attn_args* a, int dev, const float2** rope) {
  *rope = nullptr;
  if (a->pos == NEOX_POS_ROPE && a->rotary_dim > 0)
    return find_rope_table(dev, a->S, a->rotary_dim, a->rope_base, rope);
  return NEOX_OK;
}

// Backward workspace: the rotated 16-bit q and k [rows][D] each (first, at the
// offsets the forward workspace uses, so one buffer can serve both calls; used
// by the 16-bit paths) or, over the same bytes, the fp32 dq accumulator
// [rows][D] (used by the fp32 path only); then fp32 Delta [rows] and fp32
// -lse*log2e [rows]; 256-byte aligned pieces, rows = B*H*S.
struct BwdWorkspace {
  size_t dq_acc, delta, nlse, qrot, krot, total;
};

bool bwd_workspace_layout(int B, int H, int S, int D, BwdWorkspace* w) {
  if (B < 1 || H < 1 || S < 1 || D < 1) return false;
  const int64_t rows = (int64_t)B * H * S;
  if (rows >= kMaxRows || D > 4096) return false;
  size_t off = 0;
  w->qrot = off;
  w->dq_acc = off;
  off += round256((size_t)rows * (size_t)D * 2u);
  w->krot = off;
  off += round256((size_t)rows * (size_t)D * 2u);
  const size_t acc_end = round256((size_t)rows * (size_t)D * 4u);
  if (acc_end > off) off = acc_end;
  w->delta = off;
  off += round256((size_t)rows * 4u);
  w->nlse = off;
  off += round256((size_t)rows * 4u);
  w->total = off;
  return true;
}

}  // namespace

extern "C" {

size_t neox_rope_attn_bwd_workspace_size(int B, int H, int S, int D) {
  BwdWorkspace w;
  return bwd_workspace_layout(B, H, S, D, &w) ? w.total : 0;
}

size_t neox_rope_attn_fwd_workspace_size(int B, int H, int S, int D) {
  if (B < 1 || H < 1 || S < 1 || D < 1 || D > 4096) return 0;
  const int64_t rows = (int64_t)B * H * S;
  if (rows >= kMaxRows) return 0;
  return 2 * round256((size_t)rows * (size_t)D * 2u);
}

size_t neox_rope_attn_decode_workspace_size(int B, int H, int D, int cap) {
  if (B < 1 || H < 1 || D < 1 || D > 4096 || cap < 1) return 0;
  const int64_t bh = (int64_t)B * H;
  if (bh * cap >= kMaxRows) return 0;
  const int tile = neox::decode_tile_rows();  // the smallest chunk
  const int64_t nsplit = (cap + tile - 1) / tile;
  return round256((size_t)bh * (size_t)nsplit * (size_t)(D + 4) * 4u);
}

const char* neox_status_str(int status) {
  switch (status) {
    case NEOX_OK: return "ok";
    case NEOX_E_ARG: return "invalid argument";
    case NEOX_E_UNSUPPORTED: return "unsupported configuration";
    case NEOX_E_ALIGN: return "misaligned pointer or stride";
    case NEOX_E_WORKSPACE: return "workspace missing or too small";
    case NEOX_E_LAUNCH: return "kernel launch failed";
    case NEOX_E_DEVICE: return "no usable gfx950 device or HIP runtime error";
    case NEOX_E_ALLOC: return "rotary table allocation failed";
    case NEOX_E_TOO_LARGE:
      return "problem larger than the fixed scratch of the no-allocation entry point "
             "(NEOX_DECODE_SCRATCH_BYTES)";
    case NEOX_E_NOT_PREPARED:
      return "rotary table not prepared for this rotary_dim, rope_base and length "
             "(call neox_rope_table_prepare first)";
    default: return "unknown status";
  }
}

int neox_attn_fwd_ex(const neox_attn_args* a, const void* q, const void* k, const void* v,
                     void* o, float* lse, void* workspace, size_t workspace_bytes,
                     void* stream) {
  int st = validate_common(a);
  if (st != NEOX_OK) return st;
  const neox_strides def = contiguous(a);
  const neox_strides* s = a->strides;
  const bool half16 = a->dtype != NEOX_F32;  // bf16 or fp16 storage
  const int unit_in = half16 ? 8 : 4;
  const int unit_out = (half16 && a->out_dtype == NEOX_OUT_SAME) ? 8 : 4;
  if ((st = check_tensor(q, s ? s[0] : def, unit_in)) != NEOX_OK) return st;
  if ((st = check_tensor(k, s ? s[1] : def, unit_in)) != NEOX_OK) return st;
  if ((st = check_tensor(v, s ? s[2] : def, unit_in)) != NEOX_OK) return st;
  if ((st = check_tensor(o, s ? s[3] : def, unit_out)) != NEOX_OK) return st;
  if (!lse) return NEOX_E_ARG;
  if (!aligned16(lse)) return NEOX_E_ALIGN;
  if (workspace) {
    if (workspace_bytes < neox_rope_attn_fwd_workspace_size(a->B, a->H, a->S, a->D))
      return NEOX_E_WORKSPACE;
    if ((reinterpret_cast<uintptr_t>(workspace) & 255u) != 0) return NEOX_E_ALIGN;
  }

  int dev = 0;
  if ((st = check_device(&dev)) != NEOX_OK) return st;
  hipStream_t hs = reinterpret_cast<hipStream_t>(stream);
  const float2* rope = nullptr;
  if ((st = lookup_rope(a, dev, &rope)) != NEOX_OK) return st;

  neox::FwdParams p;
  fill_shape(a, rope, &p.a);
  p.q = q;
  p.k = k;
  p.v = v;
  p.o = o;
  p.lse = lse;
  p.sq = to_internal(s ? s[0] : def);
  p.sk = to_internal(s ? s[1] : def);
  p.sv = to_internal(s ? s[2] : def);
  p.so = to_internal(s ? s[3] : def);
  p.out_f32 = (a->dtype == NEOX_F32 || a->out_dtype == NEOX_OUT_F32) ? 1 : 0;
  p.qrot = reinterpret_cast<uint16_t*>(workspace);
  p.krot = workspace ? reinterpret_cast<uint16_t*>(
                           reinterpret_cast<char*>(workspace) +
                           round256((size_t)a->B * a->H * a->S * (size_t)a->D * 2u))
                     : nullptr;
  const hipEvent_t* ev = reinterpret_cast<const hipEvent_t*>(a->phase_events);
  if (neox::record_event(ev, 0, hs) != hipSuccess) return NEOX_E_LAUNCH;
  hipError_t e;
  if (a->dtype != NEOX_F32) {
    e = a->dtype == NEOX_BF16 ? neox::launch_fwd_bf16(p, hs, ev) : neox::launch_fwd_f16(p, hs, ev);
  } else {
    e = neox::record_event(ev, 1, hs);
    if (e == hipSuccess) e = neox::launch_fwd_f32(p, hs);
  }
  if (e != hipSuccess) return NEOX_E_LAUNCH;
  return neox::record_event(ev, 2, hs) == hipSuccess ? NEOX_OK : NEOX_E_LAUNCH;
}

int neox_attn_bwd_ex(const neox_attn_args* a, const void* q, const void* k, const void* v,
                     const void* o, const void* dout, const float* lse, void* dq, void* dk,
                     void* dv, void* workspace, size_t workspace_bytes, void* stream) {
  int st = validate_common(a);
  if (st != NEOX_OK) return st;
  const neox_strides def = contiguous(a);
  const neox_strides* s = a->strides;
  const bool half16 = a->dtype != NEOX_F32;  // bf16 or fp16 storage
  const int unit_in = half16 ? 8 : 4;
  const int unit_out = (half16 && a->out_dtype == NEOX_OUT_SAME) ? 8 : 4;
  const void* ins[5] = {q, k, v, o, dout};
  for (int t = 0; t < 5; ++t)
    if ((st = check_tensor(ins[t], s ? s[t] : def, unit_in)) != NEOX_OK) return st;
  void* outs[3] = {dq, dk, dv};
  for (int t = 0; t < 3; ++t)
    if ((st = check_tensor(outs[t], s ? s[5 + t] : def, unit_out)) != NEOX_OK) return st;
  if (!lse) return NEOX_E_ARG;
  if (!aligned16(lse)) return NEOX_E_ALIGN;
  for (int t = 0; t < 3; ++t)
    for (int u = 0; u < 5; ++u)
      if (outs[t] == ins[u]) return NEOX_E_ARG;
  const size_t need = neox_rope_attn_bwd_workspace_size(a->B, a->H, a->S, a->D);
  if (!workspace || workspace_bytes < need) return NEOX_E_WORKSPACE;
  if ((reinterpret_cast<uintptr_t>(workspace) & 255u) != 0) return NEOX_E_ALIGN;

  int dev = 0;
  if ((st = check_device(&dev)) != NEOX_OK) return st;
  hipStream_t hs = reinterpret_cast<hipStream_t>(stream);
  const float2* rope = nullptr;
  if ((st = lookup_rope(a, dev, &rope)) != NEOX_OK) return st;

  neox::BwdParams p;
  fill_shape(a, rope, &p.a);
  p.q = q;
  p.k = k;
  p.v = v;
  p.o = o;
  p.dout = dout;
  p.lse = lse;
  p.dq = dq;
  p.dk = dk;
  p.dv = dv;
  BwdWorkspace wl;
  bwd_workspace_layout(a->B, a->H, a->S, a->D, &wl);
  char* ws = reinterpret_cast<char*>(workspace);
  p.dq_acc = reinterpret_cast<float*>(ws + wl.dq_acc);
  p.delta = reinterpret_cast<float*>(ws + wl.delta);
  p.nlse = reinterpret_cast<float*>(ws + wl.nlse);
  p.qrot = reinterpret_cast<uint16_t*>(ws + wl.qrot);
  p.krot = reinterpret_cast<uint16_t*>(ws + wl.krot);
  p.sq = to_internal(s ? s[0] : def);
  p.sk = to_internal(s ? s[1] : def);
  p.sv = to_internal(s ? s[2] : def);
  p.so = to_internal(s ? s[3] : def);
  p.sdo = to_internal(s ? s[4] : def);
  p.sdq = to_internal(s ? s[5] : def);
  p.sdk = to_internal(s ? s[6] : def);
  p.sdv = to_internal(s ? s[7] : def);
  p.qk_ready = qk_ready(a) ? 1 : 0;
  p.out_f32 = (a->dtype == NEOX_F32 || a->out_dtype == NEOX_OUT_F32) ? 1 : 0;
  const hipEvent_t* ev = reinterpret_cast<const hipEvent_t*>(a->phase_events);
  const hipError_t e = a->dtype == NEOX_BF16  ? neox::launch_bwd_bf16(p, hs, ev)
                       : a->dtype == NEOX_F16 ? neox::launch_bwd_f16(p, hs, ev)
                                              : neox::launch_bwd_f32(p, hs, ev);
  return e == hipSuccess ? NEOX_OK : NEOX_E_LAUNCH;
}

int neox_rope_attn_fwd(const void* q, const void* k, const void* v, void* o, float* lse, int B,
                       int H, int S, int D, int rotary_dim, float rope_base, int causal,
                       float softmax_scale, int dtype, void* workspace, size_t workspace_bytes,
                       void* stream) {
  neox_attn_args a;
  std::memset(&a, 0, sizeof(a));
  a.B = B;
  a.H = H;
  a.S = S;
  a.D = D;
  a.dtype = dtype;
  a.pos = NEOX_POS_ROPE;
  a.rotary_dim = rotary_dim;
  a.rope_base = rope_base;
  a.causal = causal;
  a.softmax_scale = softmax_scale;
  a.out_dtype = NEOX_OUT_SAME;
  return neox_attn_fwd_ex(&a, q, k, v, o, lse, workspace, workspace_bytes, stream);
}

int neox_rope_attn_bwd(const void* q, const void* k, const void* v, const void* o,
                       const void* dout, const float* lse, void* dq, void* dk, void* dv, int B,
                       int H, int S, int D, int rotary_dim, float rope_base, int causal,
                       float softmax_scale, int dtype, void* workspace, size_t workspace_bytes,
                       void* stream) {
  neox_attn_args a;
  std::memset(&a, 0, sizeof(a));
  a.B = B;
  a.H = H;
  a.S = S;
  a.D = D;
  a.dtype = dtype;
  a.pos = NEOX_POS_ROPE;
  a.rotary_dim = rotary_dim;
  a.rope_base = rope_base;
  a.causal = causal;
  a.softmax_scale = softmax_scale;
  a.out_dtype = NEOX_OUT_SAME;
  return neox_attn_bwd_ex(&a, q, k, v, o, dout, lse, dq, dk, dv, workspace, workspace_bytes,
                          stream);
}

}  // extern "C"

namespace {

// Argument checks shared by both decode entry points (no device work).
int validate_decode(const void* q, const void* k, const void* v, const void* k_cache,
                    const void* v_cache, const int32_t* cache_lens, const void* o,
                    const float* lse, int B, int H, int D, int cap, int rotary_dim,
                    float rope_base, float softmax_scale, int dtype) {
  if (B < 1 || H < 1 || D < 1 || cap < 1) return NEOX_E_ARG;
  if ((int64_t)B * H * cap >= kMaxRows) return NEOX_E_ARG;
  if (dtype != NEOX_F32 && dtype != NEOX_BF16 && dtype != NEOX_F16) return NEOX_E_ARG;
  if (rotary_dim < 0 || rotary_dim > D || (rotary_dim & 1)) return NEOX_E_ARG;
  if (rotary_dim > 0 && !finite_pos(rope_base)) return NEOX_E_ARG;
  if (!finite_pos(softmax_scale)) return NEOX_E_ARG;
  const void* ptrs[] = {q, k, v, k_cache, v_cache, cache_lens, o, lse};
  for (const void* ptr : ptrs) {
    if (!ptr) return NEOX_E_ARG;
    if (!aligned16(ptr)) return NEOX_E_ALIGN;
  }
  if (o == q || o == k || o == v || o == k_cache || o == v_cache) return NEOX_E_ARG;
  if (D != 64 && D != 96 && D != 128) return NEOX_E_UNSUPPORTED;
  return NEOX_OK;
}

// Enqueues one decoding step with chunk partials in `part` (validated
// arguments; `dev` is the current device).  Without a scratch pointer
// (part == nullptr) the per-device fixed array is used.
int run_decode(int dev, const void* q, const void* k, const void* v, void* k_cache,
               void* v_cache, const int32_t* cache_lens, void* o, float* lse, int B, int H,
               int D, int cap, int rotary_dim, float rope_base, float softmax_scale, int dtype,
               float* part, hipStream_t hs) {
  int st = NEOX_OK;
  const float2* rope = nullptr;
  if (rotary_dim > 0 && (st = find_rope_table(dev, cap, rotary_dim, rope_base, &rope)) != NEOX_OK)
    return st;

  neox::DecodeParams p;
  p.B = B;
  p.H = H;
  p.D = D;
  p.cap = cap;
  p.rd = rotary_dim;
  p.rope = rope;
  p.scale_log2 = softmax_scale * 1.4426950408889634f;
  p.dtype = dtype;
  neox::decode_plan(B * H, cap, &p.chunk, &p.nsplit);
  p.lens = cache_lens;
  p.q = q;
  p.k = k;
  p.v = v;
  p.k_cache = k_cache;
  p.v_cache = v_cache;
  p.o = o;
  p.lse = lse;
  if (part == nullptr && p.nsplit > 1 && neox::decode_scratch(dev, &part) != hipSuccess) {
    (void)hipGetLastError();
    return NEOX_E_DEVICE;
  }
  p.part = part;
  return neox::launch_decode(p, hs) == hipSuccess ? NEOX_OK : NEOX_E_LAUNCH;
}

}  // namespace

extern "C" {

int neox_rope_attn_decode(const void* q, const void* k, const void* v, void* k_cache,
                          void* v_cache, const int32_t* cache_lens, void* o, float* lse, int B,
                          int H, int D, int cap, int rotary_dim, float rope_base,
                          float softmax_scale, int dtype, void* workspace,
                          size_t workspace_bytes, void* stream) {
  int st = validate_decode(q, k, v, k_cache, v_cache, cache_lens, o, lse, B, H, D, cap,
                           rotary_dim, rope_base, softmax_scale, dtype);
  if (st != NEOX_OK) return st;
  const size_t need = neox_rope_attn_decode_workspace_size(B, H, D, cap);
  if (!workspace || workspace_bytes < need) return NEOX_E_WORKSPACE;
  if ((reinterpret_cast<uintptr_t>(workspace) & 255u) != 0) return NEOX_E_ALIGN;
  int dev = 0;
  if ((st = check_device(&dev)) != NEOX_OK) return st;
  return run_decode(dev, q, k, v, k_cache, v_cache, cache_lens, o, lse, B, H, D, cap,
                    rotary_dim, rope_base, softmax_scale, dtype, static_cast<float*>(workspace),
                    reinterpret_cast<hipStream_t>(stream));
}

int neox_rope_attn_decode_noalloc(const void* q, const void* k, const void* v, void* k_cache,
                                  void* v_cache, const int32_t* cache_lens, void* o, float* lse,
                                  int B, int H, int D, int cap, int rotary_dim, float rope_base,
                                  float softmax_scale, int dtype, void* stream) {
  int st = validate_decode(q, k, v, k_cache, v_cache, cache_lens, o, lse, B, H, D, cap,
                           rotary_dim, rope_base, softmax_scale, dtype);
  if (st != NEOX_OK) return st;
  if (neox_rope_attn_decode_workspace_size(B, H, D, cap) > NEOX_DECODE_SCRATCH_BYTES)
    return NEOX_E_TOO_LARGE;
  int dev = 0;
  if ((st = check_device(&dev)) != NEOX_OK) return st;
  return run_decode(dev, q, k, v, k_cache, v_cache, cache_lens, o, lse, B, H, D, cap,
                    rotary_dim, rope_base, softmax_scale, dtype, nullptr,
                    reinterpret_cast<hipStream_t>(stream));
}

int neox_attn_fwd_fp8(const void* q8, const void* k8, const void* v8, float q_scale,
                      float k_scale, float v_scale, void* o, float* lse, int B, int H, int S,
                      int D, int causal, float softmax_scale, int out_dtype, void* stream) {
  if (B < 1 || H < 1 || S < 1 || D < 1) return NEOX_E_ARG;
  if ((int64_t)B * H * S >= kMaxRows) return NEOX_E_ARG;
  if (!finite_pos(q_scale) || !finite_pos(k_scale) || !finite_pos(v_scale)) return NEOX_E_ARG;
  if (!finite_pos(softmax_scale)) return NEOX_E_ARG;
  if (out_dtype != NEOX_OUT_SAME && out_dtype != NEOX_OUT_F32) return NEOX_E_ARG;
  const void* ptrs[] = {q8, k8, v8, o, lse};
  for (const void* ptr : ptrs) {
    if (!ptr) return NEOX_E_ARG;
    if (!aligned16(ptr)) return NEOX_E_ALIGN;
  }
  if (o == q8 || o == k8 || o == v8) return NEOX_E_ARG;
  if (D != 64 && D != 96 && D != 128) return NEOX_E_UNSUPPORTED;
  int dev = 0;
  const int st = check_device(&dev);
  if (st != NEOX_OK) return st;
  neox::Fp8FwdParams p;
  p.B = B;
  p.H = H;
  p.S = S;
  p.D = D;
  p.q = q8;
  p.k = k8;
  p.v = v8;
  p.o = o;
  p.lse = lse;
  p.scale_log2 = softmax_scale * q_scale * k_scale * 1.4426950408889634f;
  p.v_scale = v_scale;
  p.causal = causal ? 1 : 0;
  p.out_f32 = out_dtype == NEOX_OUT_F32 ? 1 : 0;
  return neox::launch_fwd_fp8(p, reinterpret_cast<hipStream_t>(stream)) == hipSuccess
             ? NEOX_OK
             : NEOX_E_LAUNCH;
}

int neox_check_doc_offsets(const int32_t* host_offsets, int B, int n_docs, int S) {
  if (!host_offsets || B < 1 || n_docs < 1 || S < 1) return NEOX_E_ARG;
  for (int b = 0; b < B; ++b) {
    const int32_t* row = host_offsets + (int64_t)b * (n_docs + 1);
    if (row[0] != 0 || row[n_docs] != S) return NEOX_E_ARG;
    for (int d = 0; d < n_docs; ++d)
      if (row[d + 1] < row[d]) return NEOX_E_ARG;
  }
  return NEOX_OK;
}

int neox_attn_plan(const neox_attn_args* a, int fwd_workspace, neox_plan* out) {
  if (!out) return NEOX_E_ARG;
  const int st = validate_common(a);
  if (st != NEOX_OK) return st;
  if (fwd_workspace != 0 && fwd_workspace != 1) return NEOX_E_ARG;
  *out = neox_plan{};
  out->fp32_path = a->dtype == NEOX_F32;
  if (out->fp32_path) {
    out->alibi = a->pos == NEOX_POS_ALIBI;
    return NEOX_OK;
  }
  const int rd = a->pos == NEOX_POS_ROPE ? a->rotary_dim : 0;
  const neox::FwdPlan f = neox::fwd_plan16(rd, a->pos == NEOX_POS_ALIBI, fwd_workspace != 0);
  const neox::BwdPlan b = neox::bwd_plan16(rd, a->pos == NEOX_POS_ALIBI, qk_ready(a));
  out->fwd_rotation_pass = f.rotation_pass;
  out->fwd_k_staging = f.rot_mode;
  out->fwd_rotate_q = f.rotate_q;
  out->alibi = f.alibi;
  out->bwd_rotation_pass = b.rotation_pass;
  return NEOX_OK;
}

int neox_rope_table_prepare(int max_S, int rotary_dim, float rope_base) {
  if (max_S < 1 || rotary_dim < 0 || (rotary_dim & 1) || !finite_pos(rope_base))
    return NEOX_E_ARG;
  if (rotary_dim == 0) return NEOX_OK;
  int dev = 0;
  int st = check_device(&dev);
  if (st != NEOX_OK) return st;
  const float2* rope = nullptr;
  return build_rope_table(dev, max_S, rotary_dim, rope_base, &rope);
}

}  // extern "C"
