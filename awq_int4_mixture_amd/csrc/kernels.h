// Internal interface between the C-ABI host code and the gfx950 kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#define AWQ_MOE_KMAX_TOKENS 8
#define AWQ_MOE_KMAX_SLOTS 256
#define AWQ_MOE_KMAX_TOPK 32
#define AWQ_MOE_KMAX_ROUTER_E 4096
#define AWQ_MOE_KMAX_HIDDEN 8192
#define AWQ_MOE_STATUS_BAD_ID_BIT 1u
// decode workspace: status word, then fp16 act [M*topk][I]
#define AWQ_MOE_KWS_STATUS_OFFSET 0
#define AWQ_MOE_KWS_ACT_OFFSET 256
// fixed decode scratch of the no-allocation entry point: status word and act
#define AWQ_MOE_KNOALLOC_SCRATCH_BYTES (256 + 512 * 1024)

namespace awq_moe {

// Everything a stage kernel needs besides its activation input and output.
// Passed by value as a kernel argument.
struct StageArgs {
  const uint8_t* bank;
  uint64_t expert_bytes;
  uint64_t w13_off, w13_meta_off, w2_off, w2_meta_off;
  const int32_t* topk_ids;  // [M][topk]
  int H, I, RB, M, topk, E;
};

// Where the compacted routing arrays go (all null: not written).
struct RouteOut {
  int32_t* active_ids;
  int32_t* offsets;
  int32_t* sorted_slots;
  int32_t* num_active;
  uint32_t* status;
};

hipError_t launch_route_compact(const int32_t* ids, int n, int E, const RouteOut& o, hipStream_t stream);
// Kernel forms of the two decode stages. Form 0 lets the tactic table choose.
enum W13Form : int { kW13Table = 0, kW13Pair = 1, kW13Single = 2, kW13Single2 = 3, kW13FormCount = 4 };
enum W2Form : int { kW2Table = 0, kW2SegMost = 1, kW2SegFewer = 2, kW2FormCount = 3 };
// The forms the table chooses for a shape (always valid for it).
void decode_table(int H, int I, int topk, int M, int RB, int* w13_form, int* w2_form);
// Whether a form (other than 0) can run a shape.
bool w13_form_valid(int form, int H, int I, int topk, int M);
bool w2_form_valid(int form, int H, int I, int topk, int M);

// ws: the decode workspace (status word and act at the offsets above).
// norm: x is a residual row r and the stage consumes r / rms(r) (eps).
hipError_t launch_w13_swiglu(const StageArgs& a, const uint16_t* x, void* ws, bool norm, float eps, int form,
                             hipStream_t stream);
// resid non-null: out receives fp16(resid + fp16(result)).
hipError_t launch_w2_reduce(const StageArgs& a, const uint16_t* act, const float* topk_w, uint16_t* out,
                            const uint16_t* resid, int form, hipStream_t stream);
hipError_t launch_router_topk(const float* logits, int M, int E, int k, int32_t* ids, float* w, hipStream_t stream);
// r_next and x may not alias r or delta.
hipError_t launch_residual_rmsnorm(const uint16_t* r, const uint16_t* delta, int M, int H, float eps,
                                   uint16_t* r_next, uint16_t* x, hipStream_t stream);
hipError_t launch_router_residual(const float* logits, int M, int E, int k, int32_t* ids, float* w,
                                  const uint16_t* r, const uint16_t* delta, int H, float eps, uint16_t* r_next,
                                  uint16_t* x, hipStream_t stream);
// Residual update + RMS norm of M rows, then fp32 logits = x . wr^T
// (wr fp16 [E][H]).
hipError_t launch_router_gemv(const uint16_t* r, const uint16_t* delta, int M, int H, float eps, const uint16_t* wr,
                              int E, uint16_t* r_next, uint16_t* x, float* logits, hipStream_t stream);
// Indexed prefill workspace (all device pointers inside the caller's workspace).
struct PrefillWs {
  uint32_t* status;
  int32_t* num_items;
  int32_t* slot_row;  // [n] row of each slot, -1 for an invalid id
  int32_t* row_slot;  // [n] slot of each row
  int32_t* items;     // [max_items][2] {expert, row0 | rows << 24}, rows <= 32
  int32_t* num_witems;
  int32_t* witems;    // [max_wide_items][2] the same with rows <= 64
  int32_t* route_cnt;  // [route blocks][E] slots per expert in each routing workgroup's slice
  int32_t* route_bad;  // [route blocks] the slice holds an id outside [0, E)
  uint16_t* act;      // fp16 [n][I] by row
  float* y;           // fp32 [n][H] by row
};
// Upper bound on the number of work items (expert row chunks of 32) for n slots.
int prefill_max_items(int n, int E);
// The same for wide work items (chunks of 64 rows).
int prefill_max_wide_items(int n, int E);
// Workgroups of the routing launches for n slots and E experts.
int prefill_route_blocks(int n, int E);
hipError_t launch_prefill(const StageArgs& a, const uint16_t* x, const float* topk_w, uint16_t* out,
                          const PrefillWs& w, hipStream_t stream);
// Address of this device's copy of the library's fixed decode scratch (the
// workspace of the no-allocation entry point), AWQ_MOE_KNOALLOC_SCRATCH_BYTES
// bytes, 256-byte aligned. Taken once per device with that device current.
hipError_t noalloc_scratch(void** ptr);
hipError_t launch_dequant(const uint8_t* bank, uint64_t expert_bytes, uint64_t units_off,
                          uint64_t meta_off, int RB, int which, int H, int I, int expert_begin,
                          int expert_count, float* out, hipStream_t stream);

}  // namespace awq_moe
