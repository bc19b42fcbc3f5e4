// Internal interface between the C-ABI host code and the gfx950 kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#define AWQ_MOE_KMAX_TOKENS 8

namespace awq_moe {

// Everything a stage kernel needs besides its activation input and output.
struct StageArgs {
  const uint8_t* bank;
  uint64_t expert_bytes;
  uint64_t w13_off, w13_meta_off, w2_off, w2_meta_off;
  int H, I, RB, M, topk;
  const int32_t* active_ids;
  const int32_t* offsets;
  const int32_t* sorted_slots;
  const int32_t* num_active;
};

hipError_t launch_route_compact(const int32_t* ids, int n, int E, int32_t* active_ids,
                                int32_t* offsets, int32_t* sorted_slots, int32_t* num_active,
                                uint32_t* status, hipStream_t stream);
hipError_t launch_w13_swiglu(const StageArgs& a, const uint16_t* x, uint16_t* act, hipStream_t stream);
hipError_t launch_w2_reduce(const StageArgs& a, const uint16_t* act, const float* topk_w,
                            uint16_t* out, hipStream_t stream);
hipError_t launch_dequant(const uint8_t* bank, uint64_t expert_bytes, uint64_t units_off,
                          uint64_t meta_off, int RB, int which, int K, int N, int expert_begin,
                          int expert_count, float* out, hipStream_t stream);
int w2_segment_slots(int I);
size_t w2_lds_bytes(int M, int I);

}  // namespace awq_moe
