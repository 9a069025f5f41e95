// Dense forward kernels at d = 64: the kernels of attn_fwd_bf16.hip, instantiated
// here alone so that this translation unit can be built with matrix-instruction
// accumulators in VGPRs (a whole-compilation option).  At d = 64 that frees the
// AGPRs the O accumulators held and lifts occupancy (three waves per SIMD at 32
// rows per wave, two at 64): causal B2 H32 N8192 d64 +12%, H32 N16384 d64 +16%.  At
// d = 128, where the score accumulators are already in VGPRs and O belongs in AGPRs,
// the same option costs 2-8%, so the d = 128 kernels stay in attn_fwd_bf16.hip.
#define ATTN_FWD_D64_TU 1
#include "attn_fwd_bf16.hip"
