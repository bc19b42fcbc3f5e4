// Host side of the C ABI declared in include/awq_moe.h: argument checks
// (fail closed before any write or launch), the bank packer, layout and
// workspace queries, and the kernel launch sequence of the decode stage.

#include <cfloat>
#include <hip/hip_runtime.h>

#include <atomic>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <string>

#include "../../include/awq_moe.h"
#include "kernels.h"

namespace {

thread_local std::string g_err;

int fail(int code, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_err = buf;
  return code;
}

int ok() {
  g_err.clear();
  return AWQ_MOE_OK;
}

uint64_t pad256(uint64_t n) { return (n + 255u) / 256u * 256u; }

bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

int check_dims(const awq_moe_dims* d) {
  if (!d) return fail(AWQ_MOE_EINVAL, "dims is null");
  if (d->group_size != 32) return fail(AWQ_MOE_EUNSUPPORTED, "group_size %d: only 32 is served", d->group_size);
  if (d->meta_bytes != 3 && d->meta_bytes != 4)
    return fail(AWQ_MOE_EUNSUPPORTED, "meta_bytes %d: only 3 or 4", d->meta_bytes);
  if (d->num_experts < 1) return fail(AWQ_MOE_EINVAL, "num_experts %d < 1", d->num_experts);
  if (d->hidden < 32 || d->hidden % 32 || d->hidden > AWQ_MOE_MAX_HIDDEN)
    return fail(AWQ_MOE_EUNSUPPORTED, "hidden %d: must be a multiple of 32 in [32, %d]", d->hidden,
                AWQ_MOE_MAX_HIDDEN);
  if (d->inter < 32 || d->inter % 32 || d->inter > AWQ_MOE_MAX_INTER)
    return fail(AWQ_MOE_EUNSUPPORTED, "inter %d: must be a multiple of 32 in [32, %d]", d->inter, AWQ_MOE_MAX_INTER);
  return AWQ_MOE_OK;
}

struct Layout {
  uint64_t w13_units, w13_meta, w2_units, w2_meta;
  awq_moe_bank_layout pub;
};

Layout make_layout(const awq_moe_dims* d) {
  const uint64_t H = (uint64_t)d->hidden, I = (uint64_t)d->inter, RB = (uint64_t)d->meta_bytes;
  Layout L;
  L.w13_units = (H / 32) * (2 * I) * 16;
  L.w13_meta = (H / 32) * (2 * I) * RB;
  L.w2_units = (I / 32) * H * 16;
  L.w2_meta = (I / 32) * H * RB;
  L.pub.w13_off = 0;
  L.pub.w13_meta_off = pad256(L.w13_units);
  L.pub.w2_off = L.pub.w13_meta_off + pad256(L.w13_meta);
  L.pub.w2_meta_off = L.pub.w2_off + pad256(L.w2_units);
  L.pub.expert_bytes = L.pub.w2_meta_off + pad256(L.w2_meta);
  L.pub.total_bytes = L.pub.expert_bytes * (uint64_t)d->num_experts;
  return L;
}

// Workspace: [status u32 | pad] [fp16 act[n][I]].
static_assert(AWQ_MOE_WS_ACT_OFFSET % 256 == 0, "act must stay 256-byte aligned");
static_assert(AWQ_MOE_NOALLOC_SCRATCH_BYTES == AWQ_MOE_KNOALLOC_SCRATCH_BYTES,
              "header and kernels agree on the fixed scratch size");
static_assert(AWQ_MOE_WS_ACT_OFFSET == AWQ_MOE_KWS_ACT_OFFSET && AWQ_MOE_WS_STATUS_OFFSET == AWQ_MOE_KWS_STATUS_OFFSET,
              "kernels and header agree on the workspace layout");

uint64_t ws_total(const awq_moe_dims* d, int max_tokens, int topk) {
  const uint64_t n = (uint64_t)max_tokens * (uint64_t)topk;
  return AWQ_MOE_WS_ACT_OFFSET + pad256(n * (uint64_t)d->inter * 2);
}

int check_tokens(int M, int topk) {
  if (M < 1 || M > AWQ_MOE_MAX_TOKENS) return fail(AWQ_MOE_EINVAL, "M %d outside [1, %d]", M, AWQ_MOE_MAX_TOKENS);
  if (topk < 1 || topk > AWQ_MOE_MAX_TOPK) return fail(AWQ_MOE_EINVAL, "topk %d outside [1, %d]", topk, AWQ_MOE_MAX_TOPK);
  return AWQ_MOE_OK;
}

// The kernels are built for gfx950 only; remember the answer per device.
std::atomic<int> g_arch_state[64];  // 0 unknown, 1 gfx950, 2 other

int check_device() {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return fail(AWQ_MOE_EHIP, "hipGetDevice: %s", hipGetErrorString(e));
  if (dev < 0 || dev >= 64) return fail(AWQ_MOE_EUNSUPPORTED, "device index %d", dev);
  int st = g_arch_state[dev].load(std::memory_order_relaxed);
  if (st == 0) {
    hipDeviceProp_t prop;
    e = hipGetDeviceProperties(&prop, dev);
    if (e != hipSuccess) return fail(AWQ_MOE_EHIP, "hipGetDeviceProperties: %s", hipGetErrorString(e));
    st = (std::strncmp(prop.gcnArchName, "gfx950", 6) == 0) ? 1 : 2;
    g_arch_state[dev].store(st, std::memory_order_relaxed);
    if (st == 2) return fail(AWQ_MOE_EUNSUPPORTED, "device %d is %s; kernels are built for gfx950", dev, prop.gcnArchName);
  }
  if (st == 2) return fail(AWQ_MOE_EUNSUPPORTED, "device %d is not gfx950", dev);
  return AWQ_MOE_OK;
}

int hip_status(hipError_t e, const char* what) {
  if (e != hipSuccess) return fail(AWQ_MOE_EHIP, "%s: %s", what, hipGetErrorString(e));
  return ok();
}

awq_moe::StageArgs stage_args(const awq_moe_dims* d, const void* bank, const int32_t* topk_ids, int M,
                              int topk) {
  const Layout L = make_layout(d);
  awq_moe::StageArgs a;
  a.bank = static_cast<const uint8_t*>(bank);
  a.expert_bytes = L.pub.expert_bytes;
  a.w13_off = L.pub.w13_off;
  a.w13_meta_off = L.pub.w13_meta_off;
  a.w2_off = L.pub.w2_off;
  a.w2_meta_off = L.pub.w2_meta_off;
  a.topk_ids = topk_ids;
  a.H = d->hidden;
  a.I = d->inter;
  a.RB = d->meta_bytes;
  a.M = M;
  a.topk = topk;
  a.E = d->num_experts;
  return a;
}

int check_route_ptrs(const int32_t* ids, const int32_t* offsets, const int32_t* slots, const int32_t* na) {
  if (!ids || !offsets || !slots || !na) return fail(AWQ_MOE_EINVAL, "routing array is null");
  if (!aligned(ids, 4) || !aligned(offsets, 4) || !aligned(slots, 4) || !aligned(na, 4))
    return fail(AWQ_MOE_EINVAL, "routing arrays must be 4-byte aligned");
  return AWQ_MOE_OK;
}

int check_router_args(const float* logits, int32_t M, int32_t num_experts, int32_t topk, const int32_t* topk_ids,
                      const float* topk_w, int32_t max_rows = AWQ_MOE_MAX_TOKENS) {
  if (M < 1 || M > max_rows) return fail(AWQ_MOE_EINVAL, "M %d outside [1, %d]", M, max_rows);
  if (num_experts < 1 || num_experts > AWQ_MOE_MAX_ROUTER_EXPERTS)
    return fail(AWQ_MOE_EINVAL, "num_experts %d outside [1, %d]", num_experts, AWQ_MOE_MAX_ROUTER_EXPERTS);
  if (topk < 1 || topk > AWQ_MOE_MAX_TOPK || topk > num_experts)
    return fail(AWQ_MOE_EINVAL, "topk %d outside [1, min(%d, num_experts)]", topk, AWQ_MOE_MAX_TOPK);
  if (!logits || !aligned(logits, 4)) return fail(AWQ_MOE_EINVAL, "logits null or misaligned");
  if (!topk_ids || !aligned(topk_ids, 4)) return fail(AWQ_MOE_EINVAL, "topk_ids null or misaligned");
  if (!topk_w || !aligned(topk_w, 4)) return fail(AWQ_MOE_EINVAL, "topk_w null or misaligned");
  return AWQ_MOE_OK;
}

int check_residual_args(const uint16_t* r, const uint16_t* delta, int32_t M, int32_t hidden, float eps,
                        const uint16_t* r_next, const uint16_t* x) {
  if (M < 1 || M > AWQ_MOE_MAX_TOKENS) return fail(AWQ_MOE_EINVAL, "M %d outside [1, %d]", M, AWQ_MOE_MAX_TOKENS);
  if (hidden < 8 || hidden > AWQ_MOE_MAX_HIDDEN || hidden % 8)
    return fail(AWQ_MOE_EINVAL, "hidden %d: a multiple of 8 in [8, %d]", hidden, AWQ_MOE_MAX_HIDDEN);
  // a normal float: 1/sqrt(mean + eps) is formed with the hardware
  // reciprocal square root, whose argument is then never subnormal
  if (!(eps >= FLT_MIN) || eps > 1.f) return fail(AWQ_MOE_EINVAL, "eps must be a normal float in [2^-126, 1]");
  if (!r || !r_next || !x || !aligned(r, 16) || !aligned(r_next, 16) || !aligned(x, 16) ||
      (delta && !aligned(delta, 16)))
    return fail(AWQ_MOE_EINVAL, "row pointer null or not 16-byte aligned");
  const uint64_t nb = (uint64_t)M * hidden * 2;
  auto overlap = [nb](const void* a, const void* b) {
    const uintptr_t pa = reinterpret_cast<uintptr_t>(a), pb = reinterpret_cast<uintptr_t>(b);
    return b && pa < pb + nb && pb < pa + nb;
  };
  if (overlap(r_next, r) || overlap(r_next, delta) || overlap(x, r) || overlap(x, delta) || overlap(x, r_next))
    return fail(AWQ_MOE_EINVAL, "r_next and x must not overlap r, delta or each other");
  return AWQ_MOE_OK;
}

// The bank must hold every expert block of dims: the kernels index experts
// by id up to num_experts - 1 and never see the allocation's size.
int check_bank(const awq_moe_dims* dims, const void* bank, uint64_t bank_bytes) {
  if (!bank || !aligned(bank, 256)) return fail(AWQ_MOE_EINVAL, "bank null or not 256-byte aligned");
  const uint64_t need = make_layout(dims).pub.total_bytes;
  if (bank_bytes < need)
    return fail(AWQ_MOE_ENOSPC, "bank_bytes %llu < %llu (the layout of dims)", (unsigned long long)bank_bytes,
                (unsigned long long)need);
  return AWQ_MOE_OK;
}

int check_stage(const awq_moe_dims* dims, const void* bank, uint64_t bank_bytes, int32_t M, int32_t topk,
                const void* workspace, uint64_t workspace_bytes) {
  int rc = check_dims(dims);
  if (rc) return rc;
  if ((rc = check_tokens(M, topk))) return rc;
  if ((rc = check_bank(dims, bank, bank_bytes))) return rc;
  if (!workspace || !aligned(workspace, 256)) return fail(AWQ_MOE_EINVAL, "workspace null or not 256-byte aligned");
  const uint64_t need = ws_total(dims, M, topk);
  if (workspace_bytes < need)
    return fail(AWQ_MOE_ENOSPC, "workspace_bytes %llu < %llu", (unsigned long long)workspace_bytes,
                (unsigned long long)need);
  return AWQ_MOE_OK;
}

struct WsPtrs {
  uint32_t* status;
  uint16_t* act;
};

WsPtrs ws_ptrs(const void* workspace) {
  uint8_t* ws = static_cast<uint8_t*>(const_cast<void*>(workspace));
  return WsPtrs{reinterpret_cast<uint32_t*>(ws + AWQ_MOE_WS_STATUS_OFFSET),
                reinterpret_cast<uint16_t*>(ws + AWQ_MOE_WS_ACT_OFFSET)};
}

}  // namespace

extern "C" {

const char* awq_moe_last_error(void) { return g_err.c_str(); }

int awq_moe_bank_layout_query(const awq_moe_dims* dims, awq_moe_bank_layout* out) {
  int rc = check_dims(dims);
  if (rc) return rc;
  if (!out) return fail(AWQ_MOE_EINVAL, "out is null");
  *out = make_layout(dims).pub;
  return ok();
}

int awq_moe_workspace_bytes(const awq_moe_dims* dims, int32_t max_tokens, int32_t topk, uint64_t* out) {
  int rc = check_dims(dims);
  if (rc) return rc;
  if ((rc = check_tokens(max_tokens, topk))) return rc;
  if (!out) return fail(AWQ_MOE_EINVAL, "out is null");
  *out = ws_total(dims, max_tokens, topk);
  return ok();
}

int awq_moe_prepare(const awq_moe_dims* dims, const uint8_t* q_gate, const uint8_t* q_up,
                    const uint8_t* q_down, const uint16_t* s_gate, const uint16_t* s_up,
                    const uint16_t* s_down, const uint8_t* z_gate, const uint8_t* z_up,
                    const uint8_t* z_down, void* bank, uint64_t bank_bytes) {
  int rc = check_dims(dims);
  if (rc) return rc;
  if (!q_gate || !q_up || !q_down || !s_gate || !s_up || !s_down || !z_gate || !z_up || !z_down || !bank)
    return fail(AWQ_MOE_EINVAL, "null input or bank pointer");
  const Layout L = make_layout(dims);
  if (bank_bytes < L.pub.total_bytes)
    return fail(AWQ_MOE_ENOSPC, "bank_bytes %llu < %llu", (unsigned long long)bank_bytes,
                (unsigned long long)L.pub.total_bytes);
  const uint64_t E = (uint64_t)dims->num_experts, H = (uint64_t)dims->hidden, I = (uint64_t)dims->inter;
  const int RB = dims->meta_bytes;
  // validate everything before writing anything
  const uint64_t nq13 = E * H * I, nq2 = E * I * H;
  for (uint64_t i = 0; i < nq13; ++i)
    if (q_gate[i] > 15 || q_up[i] > 15) return fail(AWQ_MOE_EINVAL, "q_gate/q_up value > 15 at %llu", (unsigned long long)i);
  for (uint64_t i = 0; i < nq2; ++i)
    if (q_down[i] > 15) return fail(AWQ_MOE_EINVAL, "q_down value > 15 at %llu", (unsigned long long)i);
  const uint64_t ns13 = E * (H / 32) * I, ns2 = E * (I / 32) * H;
  auto finite = [](uint16_t b) { return (b & 0x7C00u) != 0x7C00u; };
  for (uint64_t i = 0; i < ns13; ++i)
    if (!finite(s_gate[i]) || !finite(s_up[i])) return fail(AWQ_MOE_EINVAL, "non-finite W13 scale at %llu", (unsigned long long)i);
  for (uint64_t i = 0; i < ns2; ++i)
    if (!finite(s_down[i])) return fail(AWQ_MOE_EINVAL, "non-finite W2 scale at %llu", (unsigned long long)i);

  uint8_t* out = static_cast<uint8_t*>(bank);
  std::memset(out, 0, L.pub.total_bytes);
  const uint64_t G13 = H / 32, L13 = 4 * G13, G2 = I / 32, L2 = 4 * G2;

  // Pack 32 values v(k), k = 0..31 into a 16-byte unit.
  auto put_unit = [](uint8_t* dst, auto value_at) {
    for (int d = 0; d < 4; ++d) {
      uint32_t w = 0;
      for (int p = 0; p < 8; ++p) w |= (uint32_t)value_at(8 * d + p) << (4 * (p >> 1) + 16 * (p & 1));
      dst[4 * d + 0] = (uint8_t)(w);
      dst[4 * d + 1] = (uint8_t)(w >> 8);
      dst[4 * d + 2] = (uint8_t)(w >> 16);
      dst[4 * d + 3] = (uint8_t)(w >> 24);
    }
  };
  auto put_record = [RB](uint8_t* dst, uint16_t s, uint8_t z) {
    dst[0] = (uint8_t)(s & 0xFF);
    dst[1] = (uint8_t)(s >> 8);
    dst[2] = z;
    if (RB == 4) dst[3] = 0;
  };

  for (uint64_t e = 0; e < E; ++e) {
    uint8_t* blk = out + e * L.pub.expert_bytes;
    const uint8_t* qg = q_gate + e * H * I;
    const uint8_t* qu = q_up + e * H * I;
    const uint8_t* qd = q_down + e * I * H;
    const uint16_t* sg = s_gate + e * G13 * I;
    const uint16_t* su = s_up + e * G13 * I;
    const uint16_t* sd = s_down + e * G2 * H;
    const uint8_t* zg = z_gate + e * G13 * I;
    const uint8_t* zu = z_up + e * G13 * I;
    const uint8_t* zd = z_down + e * G2 * H;
    // W13: column n = 2i (gate i) or 2i + 1 (up i)
    for (uint64_t n = 0; n < 2 * I; ++n) {
      const uint64_t i = n >> 1;
      const bool up = n & 1;
      const uint8_t* q = up ? qu : qg;
      const uint64_t nt = n / 16, c = n % 16, quad = c / 4, j = c % 4;
      for (uint64_t g = 0; g < G13; ++g) {
        const uint64_t t = 4 * g + quad;
        put_unit(blk + L.pub.w13_off + nt * 256 * G13 + (j * L13 + t) * 16,
                 [&](int k) { return q[(32 * g + k) * I + i]; });
        put_record(blk + L.pub.w13_meta_off + nt * 16 * G13 * RB + (4 * t + j) * RB,
                   (up ? su : sg)[g * I + i], (up ? zu : zg)[g * I + i]);
      }
    }
    // W2: column n of hidden
    for (uint64_t n = 0; n < H; ++n) {
      const uint64_t nt = n / 16, c = n % 16, quad = c / 4, j = c % 4;
      for (uint64_t g = 0; g < G2; ++g) {
        const uint64_t t = 4 * g + quad;
        put_unit(blk + L.pub.w2_off + nt * 256 * G2 + (j * L2 + t) * 16,
                 [&](int k) { return qd[(32 * g + k) * H + n]; });
        put_record(blk + L.pub.w2_meta_off + nt * 16 * G2 * RB + (4 * t + j) * RB, sd[g * H + n], zd[g * H + n]);
      }
    }
  }
  return ok();
}

int awq_moe_route_compact(const int32_t* topk_ids, int32_t M, int32_t topk, int32_t num_experts,
                          int32_t* active_expert_ids, int32_t* active_expert_offsets,
                          int32_t* sorted_slots, int32_t* num_active, uint32_t* status, void* stream) {
  int rc = check_tokens(M, topk);
  if (rc) return rc;
  if (num_experts < 1) return fail(AWQ_MOE_EINVAL, "num_experts %d < 1", num_experts);
  if (!topk_ids || !aligned(topk_ids, 4)) return fail(AWQ_MOE_EINVAL, "topk_ids null or misaligned");
  if ((rc = check_route_ptrs(active_expert_ids, active_expert_offsets, sorted_slots, num_active))) return rc;
  if (!status || !aligned(status, 4)) return fail(AWQ_MOE_EINVAL, "status null or misaligned");
  if ((rc = check_device())) return rc;
  const awq_moe::RouteOut o{active_expert_ids, active_expert_offsets, sorted_slots, num_active, status};
  return hip_status(awq_moe::launch_route_compact(topk_ids, M * topk, num_experts, o, static_cast<hipStream_t>(stream)),
                    "route_compact launch");
}

int awq_moe_router_topk(const float* logits, int32_t M, int32_t num_experts, int32_t topk, int32_t* topk_ids,
                        float* topk_w, void* stream) {
  int rc = check_router_args(logits, M, num_experts, topk, topk_ids, topk_w, AWQ_MOE_MAX_ROUTER_ROWS);
  if (rc) return rc;
  if ((rc = check_device())) return rc;
  return hip_status(awq_moe::launch_router_topk(logits, M, num_experts, topk, topk_ids, topk_w,
                                                static_cast<hipStream_t>(stream)),
                    "router launch");
}

int awq_moe_residual_rmsnorm(const uint16_t* r, const uint16_t* delta, int32_t M, int32_t hidden, float eps,
                             uint16_t* r_next, uint16_t* x, void* stream) {
  int rc = check_residual_args(r, delta, M, hidden, eps, r_next, x);
  if (rc) return rc;
  if ((rc = check_device())) return rc;
  return hip_status(awq_moe::launch_residual_rmsnorm(r, delta, M, hidden, eps, r_next, x,
                                                     static_cast<hipStream_t>(stream)),
                    "residual_rmsnorm launch");
}

int awq_moe_router_residual(const float* logits, int32_t M, int32_t num_experts, int32_t topk, int32_t* topk_ids,
                            float* topk_w, const uint16_t* r, const uint16_t* delta, int32_t hidden, float eps,
                            uint16_t* r_next, uint16_t* x, void* stream) {
  int rc = check_router_args(logits, M, num_experts, topk, topk_ids, topk_w);
  if (rc) return rc;
  if ((rc = check_residual_args(r, delta, M, hidden, eps, r_next, x))) return rc;
  if ((rc = check_device())) return rc;
  return hip_status(awq_moe::launch_router_residual(logits, M, num_experts, topk, topk_ids, topk_w, r, delta, hidden,
                                                    eps, r_next, x, static_cast<hipStream_t>(stream)),
                    "router_residual launch");
}

int awq_moe_router_gemv(const uint16_t* r, const uint16_t* delta, int32_t M, int32_t hidden, float eps,
                        const uint16_t* router_w, int32_t num_experts, uint16_t* r_next, uint16_t* x, float* logits,
                        void* stream) {
  int rc = check_residual_args(r, delta, M, hidden, eps, r_next, x);
  if (rc) return rc;
  if (num_experts < 1 || num_experts > AWQ_MOE_MAX_ROUTER_EXPERTS)
    return fail(AWQ_MOE_EINVAL, "num_experts %d outside [1, %d]", num_experts, AWQ_MOE_MAX_ROUTER_EXPERTS);
  if (!router_w || !aligned(router_w, 16)) return fail(AWQ_MOE_EINVAL, "router_w null or not 16-byte aligned");
  if (!logits || !aligned(logits, 4)) return fail(AWQ_MOE_EINVAL, "logits null or misaligned");
  if ((rc = check_device())) return rc;
  return hip_status(awq_moe::launch_router_gemv(r, delta, M, hidden, eps, router_w, num_experts, r_next, x, logits,
                                                static_cast<hipStream_t>(stream)),
                    "router_gemv launch");
}

int awq_moe_w13_swiglu(const awq_moe_dims* dims, const void* bank, uint64_t bank_bytes, const uint16_t* x,
                       const int32_t* topk_ids, int32_t M, int32_t topk, void* workspace, uint64_t workspace_bytes,
                       void* stream) {
  int rc = check_stage(dims, bank, bank_bytes, M, topk, workspace, workspace_bytes);
  if (rc) return rc;
  if (!x || !aligned(x, 16)) return fail(AWQ_MOE_EINVAL, "x null or not 16-byte aligned");
  if (!topk_ids || !aligned(topk_ids, 4)) return fail(AWQ_MOE_EINVAL, "topk_ids null or misaligned");
  if ((rc = check_device())) return rc;
  return hip_status(awq_moe::launch_w13_swiglu(stage_args(dims, bank, topk_ids, M, topk), x, workspace, false, 0.f, 0,
                                               static_cast<hipStream_t>(stream)),
                    "w13 launch");
}

int awq_moe_w2_reduce(const awq_moe_dims* dims, const void* bank, uint64_t bank_bytes, const int32_t* topk_ids,
                      const float* topk_w, int32_t M, int32_t topk, const void* workspace, uint64_t workspace_bytes,
                      uint16_t* out, void* stream) {
  int rc = check_stage(dims, bank, bank_bytes, M, topk, workspace, workspace_bytes);
  if (rc) return rc;
  if (!topk_ids || !aligned(topk_ids, 4)) return fail(AWQ_MOE_EINVAL, "topk_ids null or misaligned");
  if (!topk_w || !aligned(topk_w, 4)) return fail(AWQ_MOE_EINVAL, "topk_w null or misaligned");
  if (!out || !aligned(out, 16)) return fail(AWQ_MOE_EINVAL, "out null or not 16-byte aligned");
  if ((rc = check_device())) return rc;
  const WsPtrs w = ws_ptrs(workspace);
  return hip_status(awq_moe::launch_w2_reduce(stage_args(dims, bank, topk_ids, M, topk), w.act, topk_w, out, nullptr, 0,
                                              static_cast<hipStream_t>(stream)),
                    "w2 launch");
}

namespace {

struct PrefillLayout {
  uint64_t slot_row, row_slot, items, witems, route_cnt, route_bad, act, y, total;
};

PrefillLayout prefill_layout(const awq_moe_dims* d, int M, int topk) {
  const uint64_t n = (uint64_t)M * (uint64_t)topk;
  const uint64_t mi = (uint64_t)awq_moe::prefill_max_items((int)n, d->num_experts);
  const uint64_t mw = (uint64_t)awq_moe::prefill_max_wide_items((int)n, d->num_experts);
  PrefillLayout L;
  uint64_t off = 256;  // status u32 at 0, num_items i32 at 4, num wide items i32 at 8
  L.slot_row = off;
  off += pad256(n * 4);
  L.row_slot = off;
  off += pad256(n * 4);
  L.items = off;
  off += pad256(mi * 8);
  L.witems = off;
  off += pad256(mw * 8);
  const uint64_t nb = (uint64_t)awq_moe::prefill_route_blocks((int)n, d->num_experts);
  L.route_cnt = off;
  off += pad256(nb * (uint64_t)d->num_experts * 4);
  L.route_bad = off;
  off += pad256(nb * 4);
  L.act = off;
  off += pad256(n * (uint64_t)d->inter * 2);
  L.y = off;
  off += pad256(n * (uint64_t)d->hidden * 4);
  L.total = off;
  return L;
}

int check_prefill_shape(const awq_moe_dims* dims, int M, int topk) {
  int rc = check_dims(dims);
  if (rc) return rc;
  if (dims->num_experts > AWQ_MOE_PREFILL_MAX_EXPERTS)
    return fail(AWQ_MOE_EUNSUPPORTED, "num_experts %d > %d for prefill", dims->num_experts,
                AWQ_MOE_PREFILL_MAX_EXPERTS);
  if (M < AWQ_MOE_PREFILL_MIN_TOKENS || M > AWQ_MOE_PREFILL_MAX_TOKENS)
    return fail(AWQ_MOE_EINVAL, "M %d outside [%d, %d] (1..8 tokens go to awq_moe_decode)", M,
                AWQ_MOE_PREFILL_MIN_TOKENS, AWQ_MOE_PREFILL_MAX_TOKENS);
  if (topk < 1 || topk > AWQ_MOE_MAX_TOPK) return fail(AWQ_MOE_EINVAL, "topk %d outside [1, %d]", topk, AWQ_MOE_MAX_TOPK);
  return AWQ_MOE_OK;
}

}  // namespace

int awq_moe_prefill_workspace_bytes(const awq_moe_dims* dims, int32_t max_tokens, int32_t topk, uint64_t* out) {
  int rc = check_prefill_shape(dims, max_tokens, topk);
  if (rc) return rc;
  if (!out) return fail(AWQ_MOE_EINVAL, "out is null");
  *out = prefill_layout(dims, max_tokens, topk).total;
  return ok();
}

int awq_moe_prefill(const awq_moe_dims* dims, const void* bank, uint64_t bank_bytes, const uint16_t* x,
                    const int32_t* topk_ids, const float* topk_w, int32_t M, int32_t topk, uint16_t* out,
                    void* workspace, uint64_t workspace_bytes, void* stream) {
  int rc = check_prefill_shape(dims, M, topk);
  if (rc) return rc;
  if ((rc = check_bank(dims, bank, bank_bytes))) return rc;
  if (!workspace || !aligned(workspace, 256)) return fail(AWQ_MOE_EINVAL, "workspace null or not 256-byte aligned");
  const PrefillLayout L = prefill_layout(dims, M, topk);
  if (workspace_bytes < L.total)
    return fail(AWQ_MOE_ENOSPC, "workspace_bytes %llu < %llu", (unsigned long long)workspace_bytes,
                (unsigned long long)L.total);
  if (!x || !aligned(x, 16)) return fail(AWQ_MOE_EINVAL, "x null or not 16-byte aligned");
  if (!topk_ids || !aligned(topk_ids, 4)) return fail(AWQ_MOE_EINVAL, "topk_ids null or misaligned");
  if (!topk_w || !aligned(topk_w, 4)) return fail(AWQ_MOE_EINVAL, "topk_w null or misaligned");
  if (!out || !aligned(out, 16)) return fail(AWQ_MOE_EINVAL, "out null or not 16-byte aligned");
  if ((rc = check_device())) return rc;
  uint8_t* ws = static_cast<uint8_t*>(workspace);
  awq_moe::PrefillWs w;
  w.status = reinterpret_cast<uint32_t*>(ws);
  w.num_items = reinterpret_cast<int32_t*>(ws + 4);
  w.slot_row = reinterpret_cast<int32_t*>(ws + L.slot_row);
  w.row_slot = reinterpret_cast<int32_t*>(ws + L.row_slot);
  w.items = reinterpret_cast<int32_t*>(ws + L.items);
  w.num_witems = reinterpret_cast<int32_t*>(ws + 8);
  w.witems = reinterpret_cast<int32_t*>(ws + L.witems);
  w.route_cnt = reinterpret_cast<int32_t*>(ws + L.route_cnt);
  w.route_bad = reinterpret_cast<int32_t*>(ws + L.route_bad);
  w.act = reinterpret_cast<uint16_t*>(ws + L.act);
  w.y = reinterpret_cast<float*>(ws + L.y);
  return hip_status(awq_moe::launch_prefill(stage_args(dims, bank, topk_ids, M, topk), x, topk_w, out, w,
                                            static_cast<hipStream_t>(stream)),
                    "prefill launch");
}

int awq_moe_decode(const awq_moe_dims* dims, const void* bank, uint64_t bank_bytes, const uint16_t* x,
                   const int32_t* topk_ids, const float* topk_w, int32_t M, int32_t topk, uint16_t* out,
                   void* workspace, uint64_t workspace_bytes, void* stream) {
  int rc = check_stage(dims, bank, bank_bytes, M, topk, workspace, workspace_bytes);
  if (rc) return rc;
  if (!x || !aligned(x, 16)) return fail(AWQ_MOE_EINVAL, "x null or not 16-byte aligned");
  if (!topk_ids || !aligned(topk_ids, 4)) return fail(AWQ_MOE_EINVAL, "topk_ids null or misaligned");
  if (!topk_w || !aligned(topk_w, 4)) return fail(AWQ_MOE_EINVAL, "topk_w null or misaligned");
  if (!out || !aligned(out, 16)) return fail(AWQ_MOE_EINVAL, "out null or not 16-byte aligned");
  if ((rc = check_device())) return rc;
  const WsPtrs w = ws_ptrs(workspace);
  hipStream_t s = static_cast<hipStream_t>(stream);
  const awq_moe::StageArgs a = stage_args(dims, bank, topk_ids, M, topk);
  hipError_t e = awq_moe::launch_w13_swiglu(a, x, workspace, false, 0.f, 0, s);
  if (e != hipSuccess) return hip_status(e, "w13 launch");
  return hip_status(awq_moe::launch_w2_reduce(a, w.act, topk_w, out, nullptr, 0, s), "w2 launch");
}

int awq_moe_decode_rmsnorm_residual(const awq_moe_dims* dims, const void* bank, uint64_t bank_bytes,
                                    const uint16_t* r, float eps, const int32_t* topk_ids, const float* topk_w,
                                    int32_t M, int32_t topk, uint16_t* r_next, void* workspace,
                                    uint64_t workspace_bytes, void* stream) {
  int rc = check_stage(dims, bank, bank_bytes, M, topk, workspace, workspace_bytes);
  if (rc) return rc;
  // a normal float: 1/sqrt(mean + eps) is formed with the hardware
  // reciprocal square root, whose argument is then never subnormal
  if (!(eps >= FLT_MIN) || eps > 1.f) return fail(AWQ_MOE_EINVAL, "eps must be a normal float in [2^-126, 1]");
  if (!r || !r_next || !aligned(r, 16) || !aligned(r_next, 16))
    return fail(AWQ_MOE_EINVAL, "r or r_next null or not 16-byte aligned");
  const uint64_t nb = (uint64_t)M * dims->hidden * 2;
  const uintptr_t pa = reinterpret_cast<uintptr_t>(r), pb = reinterpret_cast<uintptr_t>(r_next);
  if (pa < pb + nb && pb < pa + nb) return fail(AWQ_MOE_EINVAL, "r_next must not overlap r");
  if (!topk_ids || !aligned(topk_ids, 4)) return fail(AWQ_MOE_EINVAL, "topk_ids null or misaligned");
  if (!topk_w || !aligned(topk_w, 4)) return fail(AWQ_MOE_EINVAL, "topk_w null or misaligned");
  if ((rc = check_device())) return rc;
  const WsPtrs w = ws_ptrs(workspace);
  hipStream_t s = static_cast<hipStream_t>(stream);
  const awq_moe::StageArgs a = stage_args(dims, bank, topk_ids, M, topk);
  hipError_t e = awq_moe::launch_w13_swiglu(a, r, workspace, true, eps, 0, s);
  if (e != hipSuccess) return hip_status(e, "w13 launch");
  return hip_status(awq_moe::launch_w2_reduce(a, w.act, topk_w, r_next, r, 0, s), "w2 launch");
}

int awq_moe_decode_table(const awq_moe_dims* dims, int32_t M, int32_t topk, int32_t* w13_form, int32_t* w2_form) {
  int rc = check_dims(dims);
  if (rc) return rc;
  if ((rc = check_tokens(M, topk))) return rc;
  if (!w13_form || !w2_form) return fail(AWQ_MOE_EINVAL, "null output pointer");
  int a = 0, b = 0;
  awq_moe::decode_table(dims->hidden, dims->inter, topk, M, dims->meta_bytes, &a, &b);
  *w13_form = a;
  *w2_form = b;
  return ok();
}

int awq_moe_decode_forms(const awq_moe_dims* dims, const void* bank, uint64_t bank_bytes, const uint16_t* x,
                         const int32_t* topk_ids, const float* topk_w, int32_t M, int32_t topk, uint16_t* out,
                         void* workspace, uint64_t workspace_bytes, int32_t w13_form, int32_t w2_form,
                         int32_t stages, void* stream) {
  int rc = check_stage(dims, bank, bank_bytes, M, topk, workspace, workspace_bytes);
  if (rc) return rc;
  if (stages < 1 || stages > 3) return fail(AWQ_MOE_EINVAL, "stages %d: 1 (W13), 2 (W2) or 3 (both)", stages);
  if (w13_form < 0 || w13_form >= awq_moe::kW13FormCount || w2_form < 0 || w2_form >= awq_moe::kW2FormCount)
    return fail(AWQ_MOE_EINVAL, "form out of range (w13 %d, w2 %d)", w13_form, w2_form);
  if (w13_form && !awq_moe::w13_form_valid(w13_form, dims->hidden, dims->inter, topk, M))
    return fail(AWQ_MOE_EUNSUPPORTED, "W13 form %d does not fit hidden %d", w13_form, dims->hidden);
  if (w2_form && !awq_moe::w2_form_valid(w2_form, dims->hidden, dims->inter, topk, M))
    return fail(AWQ_MOE_EUNSUPPORTED, "W2 form %d does not fit inter %d", w2_form, dims->inter);
  if ((stages & 1) && (!x || !aligned(x, 16))) return fail(AWQ_MOE_EINVAL, "x null or not 16-byte aligned");
  if (!topk_ids || !aligned(topk_ids, 4)) return fail(AWQ_MOE_EINVAL, "topk_ids null or misaligned");
  if (stages & 2) {
    if (!topk_w || !aligned(topk_w, 4)) return fail(AWQ_MOE_EINVAL, "topk_w null or misaligned");
    if (!out || !aligned(out, 16)) return fail(AWQ_MOE_EINVAL, "out null or not 16-byte aligned");
  }
  if ((rc = check_device())) return rc;
  const WsPtrs w = ws_ptrs(workspace);
  hipStream_t s = static_cast<hipStream_t>(stream);
  const awq_moe::StageArgs a = stage_args(dims, bank, topk_ids, M, topk);
  if (stages & 1) {
    hipError_t e = awq_moe::launch_w13_swiglu(a, x, workspace, false, 0.f, w13_form, s);
    if (e != hipSuccess) return hip_status(e, "w13 launch");
  }
  if (stages & 2) return hip_status(awq_moe::launch_w2_reduce(a, w.act, topk_w, out, nullptr, w2_form, s), "w2 launch");
  return ok();
}

int awq_moe_decode_noalloc(const awq_moe_dims* dims, const void* bank, uint64_t bank_bytes, const uint16_t* x,
                           const int32_t* topk_ids, const float* topk_w, int32_t M, int32_t topk, uint16_t* out,
                           uint32_t* status, void* stream) {
  int rc = check_dims(dims);
  if (rc) return rc;
  if ((rc = check_tokens(M, topk))) return rc;
  if ((rc = check_bank(dims, bank, bank_bytes))) return rc;
  const uint64_t need = ws_total(dims, M, topk);
  if (need > AWQ_MOE_NOALLOC_SCRATCH_BYTES)
    return fail(AWQ_MOE_ENOSPC, "M*topk*inter = %lld needs %llu bytes of scratch; the library holds %llu",
                (long long)M * topk * dims->inter, (unsigned long long)need,
                (unsigned long long)AWQ_MOE_NOALLOC_SCRATCH_BYTES);
  if (!x || !aligned(x, 16)) return fail(AWQ_MOE_EINVAL, "x null or not 16-byte aligned");
  if (!topk_ids || !aligned(topk_ids, 4)) return fail(AWQ_MOE_EINVAL, "topk_ids null or misaligned");
  if (!topk_w || !aligned(topk_w, 4)) return fail(AWQ_MOE_EINVAL, "topk_w null or misaligned");
  if (!out || !aligned(out, 16)) return fail(AWQ_MOE_EINVAL, "out null or not 16-byte aligned");
  if (status && !aligned(status, 4)) return fail(AWQ_MOE_EINVAL, "status misaligned");
  if ((rc = check_device())) return rc;
  void* ws = nullptr;
  hipError_t e = awq_moe::noalloc_scratch(&ws);
  if (e != hipSuccess) return hip_status(e, "scratch address");
  const WsPtrs w = ws_ptrs(ws);
  hipStream_t s = static_cast<hipStream_t>(stream);
  const awq_moe::StageArgs a = stage_args(dims, bank, topk_ids, M, topk);
  e = awq_moe::launch_w13_swiglu(a, x, ws, false, 0.f, 0, s);
  if (e != hipSuccess) return hip_status(e, "w13 launch");
  e = awq_moe::launch_w2_reduce(a, w.act, topk_w, out, nullptr, 0, s);
  if (e != hipSuccess) return hip_status(e, "w2 launch");
  if (status) return hip_status(hipMemcpyAsync(status, w.status, 4, hipMemcpyDeviceToDevice, s), "status copy");
  return ok();
}

int awq_moe_dequant(const awq_moe_dims* dims, const void* bank, uint64_t bank_bytes, int32_t expert_begin,
                    int32_t expert_count, int32_t which, float* out, void* stream) {
  int rc = check_dims(dims);
  if (rc) return rc;
  if ((rc = check_bank(dims, bank, bank_bytes))) return rc;
  if (!out || !aligned(out, 4)) return fail(AWQ_MOE_EINVAL, "out null or misaligned");
  if (which != 0 && which != 1) return fail(AWQ_MOE_EINVAL, "which %d: 0 (W13) or 1 (W2)", which);
  if (expert_count < 1 || expert_begin < 0 || (int64_t)expert_begin + expert_count > dims->num_experts)
    return fail(AWQ_MOE_EINVAL, "expert range [%d, %d) outside [0, %d)", expert_begin,
                expert_begin + expert_count, dims->num_experts);
  if ((rc = check_device())) return rc;
  const Layout L = make_layout(dims);
  const uint64_t uo = which == 0 ? L.pub.w13_off : L.pub.w2_off;
  const uint64_t mo = which == 0 ? L.pub.w13_meta_off : L.pub.w2_meta_off;
  return hip_status(awq_moe::launch_dequant(static_cast<const uint8_t*>(bank), L.pub.expert_bytes, uo, mo,
                                            dims->meta_bytes, which, dims->hidden, dims->inter, expert_begin, expert_count, out,
                                            static_cast<hipStream_t>(stream)),
                    "dequant launch");
}

}  // extern "C"
