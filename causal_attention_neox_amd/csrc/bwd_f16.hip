// Backward attention for IEEE half storage: the 16-bit backward kernels of
// bwd_bf16.hip compiled with half elements (v_mfma_f32_32x32x16_f16, fp32
// accumulation; round-to-nearest-even conversions).
#define NEOX_ELEM_F16 1
#include "bwd_bf16.hip"
