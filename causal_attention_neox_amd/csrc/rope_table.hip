// Rotary cos/sin table: table[t * half + p] = (cos theta, sin theta) with
// theta = t * base^(-2p / rotary_dim), p < half = rotary_dim / 2 (one entry per
// rotary pair: the attention.rotary_emb.inv_freq frequencies listed among the
// GPT-NeoX checkpoint tensors in "FasterTransformer GPT-NeoX 推理指南").
// Angles and trigonometric values are computed in double and rounded to fp32
// once, so large positions keep full fp32 accuracy.
#include "kernels.hpp"

namespace neox {
namespace {

__global__ __launch_bounds__(256) void rope_table_kernel(float2* table, int S, int half, double base,
                                                          int rd) {
  const int64_t it = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (it >= (int64_t)S * half) return;
  const int t = (int)(it / half), pidx = (int)(it % half);
  const double inv_freq = pow(base, -2.0 * (double)pidx / (double)rd);
  const double theta = (double)t * inv_freq;
  double sn, cs;
  sincos(theta, &sn, &cs);
  table[it] = make_float2((float)cs, (float)sn);
}

}  // namespace

hipError_t launch_rope_table(float2* table, int S, int rd, double base, hipStream_t st) {
  const int half = rd / 2;
  const int64_t n = (int64_t)S * half;
  if (n == 0) return hipSuccess;
  hipLaunchKernelGGL(rope_table_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, st, table,
                     S, half, base, rd);
  return hipGetLastError();
}

}  // namespace neox
