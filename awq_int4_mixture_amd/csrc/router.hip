// gfx950 kernels of the per-layer steps around the expert stage in a stack
// of layers: the router top-k + softmax, the residual update + RMS norm, and
// the router GEMV. The pages leave the router unchanged (fork PR #12,
// Purpose and stack); these exist so that a many-layer decode step runs
// entirely on the device.

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "device_util.h"
#include "kernels.h"

namespace awq_moe {
// ---------------------------------------------------------------------------
// Router top-k + softmax (the layer-stack workload's per-layer router; the
// pages leave the router unchanged, fork PR #12, Purpose and stack).
// One workgroup per token. Each logit becomes a 64-bit key that orders by
// value (exact fp32 order, -0 == +0, NaN below every number) and then by
// lower id:  key = ord(value) << 32 | (0xFFFFFFFF - id), ord mapping the
// float bit pattern to an order-preserving uint32. Keys are distinct, so
// the number of larger keys is an element's rank. The softmax over the k
// winners is fp32, summed in rank order.
// ---------------------------------------------------------------------------
__device__ __forceinline__ uint64_t router_key(float v, int id) {
  uint32_t ord;
  if (v != v) {
    ord = 0u;  // NaN: below every number
  } else {
    const uint32_t u = __builtin_bit_cast(uint32_t, v == 0.f ? 0.f : v);
    ord = (u & 0x80000000u) ? ~u : (u | 0x80000000u);
  }
  return ((uint64_t)ord << 32) | (uint64_t)(0xFFFFFFFFu - (uint32_t)id);
}

__device__ __forceinline__ uint64_t readlane_u64(uint64_t v, int lane) {
  const uint32_t lo = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)v, lane);
  const uint32_t hi = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)(v >> 32), lane);
  return ((uint64_t)hi << 32) | lo;
}

// Two stages. (1) Each wave ranks the keys of a 64-element chunk among
// themselves with lane reads (no memory round trips) and keeps its k best
// as candidates at fixed places chunk*k + rank. (2) Each candidate is
// ranked among all candidates in LDS; rank < k is the answer.
__device__ void router_topk_row(const float* __restrict__ lg, int E, int k, int32_t* __restrict__ ids,
                                float* __restrict__ w) {
  __shared__ uint64_t cand[AWQ_MOE_KMAX_ROUTER_E / 64 * AWQ_MOE_KMAX_TOPK];
  __shared__ float cand_v[AWQ_MOE_KMAX_ROUTER_E / 64 * AWQ_MOE_KMAX_TOPK];
  __shared__ float sel_v[AWQ_MOE_KMAX_TOPK];
  const int t = threadIdx.x, nt = blockDim.x;
  const int lane = t & 63, wave = t >> 6, nwaves = nt >> 6;
  const int nchunks = (E + 63) >> 6;
  const int ncand = nchunks * k;
  // the wave's first chunk is requested before anything waits
  const int i0 = wave * 64 + lane;
  float v0 = 0.f;
  if (i0 < E) v0 = lg[i0];
  for (int c = t; c < ncand; c += nt) cand[c] = 0;  // 0 sorts below every key
  __syncthreads();
  for (int chunk = wave; chunk < nchunks; chunk += nwaves) {
    const int i = chunk * 64 + lane;
    const float v = chunk == wave ? v0 : (i < E ? lg[i] : 0.f);
    const uint64_t key = i < E ? router_key(v, i) : 0;
    int r = 0;
#pragma unroll
    for (int j = 0; j < 64; ++j) r += readlane_u64(key, j) > key;
    if (i < E && r < k) {
      cand[chunk * k + r] = key;
      cand_v[chunk * k + r] = v;
    }
  }
  __syncthreads();
  for (int c = t; c < ncand; c += nt) {
    const uint64_t kc = cand[c];
    if (kc == 0) continue;
    int r = 0;
#pragma unroll 8
    for (int j = 0; j < ncand; ++j) r += cand[j] > kc;
    if (r < k) {
      ids[r] = (int)(0xFFFFFFFFu - (uint32_t)kc);
      sel_v[r] = cand_v[c];
    }
  }
  __syncthreads();
  if (t < 64) {
    const float m = sel_v[0];
    const float p = t < k ? expf(sel_v[t] - m) : 0.f;
    float sum = 0.f;  // in rank order, from the lanes' registers
    for (int r = 0; r < k; ++r) sum += __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, p), r));
    if (t < k) w[t] = p / sum;
  }
}

__global__ __launch_bounds__(1024) void router_topk_kernel(const float* __restrict__ logits, int E, int k,
                                                           int32_t* __restrict__ ids, float* __restrict__ w) {
  const int tok = blockIdx.x;
  router_topk_row(logits + (uint64_t)tok * E, E, k, ids + tok * k, w + tok * k);
}

// ---------------------------------------------------------------------------
// Residual update and parameter-free RMS norm for the layer-stack workload:
// r_next = fp16(r + delta) (delta may be null: r_next = r), and
// x = fp16(r_next / sqrt(mean(r_next^2) + eps)), all in fp32. One workgroup
// per row; each thread owns runs of 8 values (16-byte loads and stores) and
// keeps them in registers across the reduction.
// ---------------------------------------------------------------------------
// One run of 8 values per thread (blockDim >= H/8, H <= 8192, H % 8 == 0).
struct ResRow {
  h8_t a, b;
};

// Issue the loads of row r (and delta) for this thread's run.
__device__ __forceinline__ ResRow residual_load(const uint16_t* __restrict__ r, const uint16_t* __restrict__ delta,
                                                int H) {
  ResRow rr;
  const int i = threadIdx.x;
  if (i < (H >> 3)) {
    rr.a = *reinterpret_cast<const h8_t*>(r + 8 * i);
    if (delta) rr.b = *reinterpret_cast<const h8_t*>(delta + 8 * i);
  }
  return rr;
}

// 1/sqrt(tot / H + eps) with the hardware reciprocal and reciprocal square
// root (about 1 ulp each): the step sits between the row's last barrier and
// its first use, where an IEEE division and square root lengthen every
// workgroup's critical path. Both kernels that normalise a row use it, so
// their x agree bit for bit.
__device__ __forceinline__ float inv_rms_row(float tot, int H, float eps) {
  return __builtin_amdgcn_rsqf(fmaf(tot, __builtin_amdgcn_rcpf((float)H), eps));
}

__device__ void residual_finish(const ResRow& rr, bool has_delta, int H, float eps, uint16_t* __restrict__ r_next,
                                uint16_t* __restrict__ x) {
  __shared__ float part[16];
  const int t = threadIdx.x;
  const bool on = t < (H >> 3);
  h8_t a = rr.a;
  float ss = 0.f;
  if (on) {
    if (has_delta) {
#pragma unroll
      for (int e = 0; e < 8; ++e) a[e] = (_Float16)((float)a[e] + (float)rr.b[e]);
    }
    *reinterpret_cast<h8_t*>(r_next + 8 * t) = a;
#pragma unroll
    for (int e = 0; e < 8; ++e) ss = fmaf((float)a[e], (float)a[e], ss);
  }
  ss = wave_sum_xor_order(ss);
  if ((t & 63) == 0) part[t >> 6] = ss;
  __syncthreads();
  float tot = 0.f;
  for (int i = 0; i < (int)(blockDim.x >> 6); ++i) tot += part[i];
  const float inv = inv_rms_row(tot, H, eps);
  if (on) {
    h8_t o;
#pragma unroll
    for (int e = 0; e < 8; ++e) o[e] = (_Float16)((float)a[e] * inv);
    *reinterpret_cast<h8_t*>(x + 8 * t) = o;
  }
}

__global__ __launch_bounds__(1024) void residual_rmsnorm_kernel(const uint16_t* __restrict__ r,
                                                                const uint16_t* __restrict__ delta, int H, float eps,
                                                                uint16_t* __restrict__ r_next,
                                                                uint16_t* __restrict__ x) {
  const uint64_t o = (uint64_t)blockIdx.x * H;
  const ResRow rr = residual_load(r + o, delta ? delta + o : nullptr, H);
  residual_finish(rr, delta != nullptr, H, eps, r_next + o, x + o);
}

// Both per-token steps between two stacked layers in one launch, as two
// workgroups per token (blockIdx.y: 0 the router, 1 the residual update and
// norm) so that the two chains run side by side. The block is the same for
// both roles; the norm's extra waves add zero partial sums, so its result is
// bit-identical to residual_rmsnorm_kernel's.
__global__ __launch_bounds__(1024) void router_residual_kernel(const float* __restrict__ logits, int E, int k,
                                                               int32_t* __restrict__ ids, float* __restrict__ w,
                                                               const uint16_t* __restrict__ r,
                                                               const uint16_t* __restrict__ delta, int H, float eps,
                                                               uint16_t* __restrict__ r_next,
                                                               uint16_t* __restrict__ x) {
  const int tok = blockIdx.x;
  if (blockIdx.y == 0) {
    router_topk_row(logits + (uint64_t)tok * E, E, k, ids + tok * k, w + tok * k);
  } else {
    const uint64_t o = (uint64_t)tok * H;
    const ResRow rr = residual_load(r + o, delta ? delta + o : nullptr, H);
    residual_finish(rr, delta != nullptr, H, eps, r_next + o, x + o);
  }
}

// ---------------------------------------------------------------------------
// Router GEMV for a stack of layers: the residual update and RMS norm of a
// row (bit-identical to residual_rmsnorm_kernel), then fp32 logits =
// x . wr^T for kGemvExperts experts (wr fp16 [E][H]). One workgroup per
// (expert chunk, token row), one thread per run of 8 values as in
// residual_finish: a workgroup normalises only its own row (from L2), and
// the M workgroups of a chunk read its router weights, which come from HBM
// once and from L2 after that when they share an XCD (the chunk count is
// rounded up to a multiple of 8 so that they do). The weights are loaded
// before the norm, which does not depend on them.
// ---------------------------------------------------------------------------
constexpr int kGemvExperts = 16;

// One step of a wave reduce-scatter over the lane pairing of a DPP control
// (lanes with `up` keep the upper half of the n values in v[0..n)); with
// n == 1 it is a plain pairwise sum.
template <int CTRL, int n, int N>
__device__ __forceinline__ void rs_dpp(float (&v)[N], bool up) {
  if constexpr (n > 1) {
#pragma unroll
    for (int i = 0; i < n / 2; ++i) {
      const float keep = up ? v[i + n / 2] : v[i];
      const float send = up ? v[i] : v[i + n / 2];
      v[i] = keep + dpp<CTRL>(send);
    }
  } else {
    v[0] += dpp<CTRL>(v[0]);
  }
}
template <int OFF, int n, int N>
__device__ __forceinline__ void rs_shfl(float (&v)[N], bool up) {
  if constexpr (n > 1) {
#pragma unroll
    for (int i = 0; i < n / 2; ++i) {
      const float keep = up ? v[i + n / 2] : v[i];
      const float send = up ? v[i] : v[i + n / 2];
      v[i] = keep + __shfl_xor(send, OFF);
    }
  } else {
    v[0] += __shfl_xor(v[0], OFF);
  }
}
constexpr int rs_n(int N, int s) { return (N >> s) > 0 ? (N >> s) : 1; }

// Wave sums of N = 2^b values per lane: a reduce-scatter over lane bits
// 0..b-1, plain sums over the others. Lane l ends with the wave's sum of
// value index bitreverse_b(l mod N). The quad permutes and row rotations
// pair lanes within a 16-lane row (a rotation by 4 after the quad steps
// still pairs lanes that hold the same index subset), the shuffles across rows.
template <int N>
__device__ __forceinline__ float wave_reduce_scatter(float (&v)[N]) {
  const int lane = threadIdx.x & 63;
  rs_dpp<kQuadSwap1, rs_n(N, 0)>(v, lane & 1);
  rs_dpp<kQuadSwap2, rs_n(N, 1)>(v, lane & 2);
  rs_dpp<kRowRor4, rs_n(N, 2)>(v, lane & 4);
  rs_dpp<kRowRor8, rs_n(N, 3)>(v, lane & 8);
  rs_shfl<16, rs_n(N, 4)>(v, lane & 16);
  rs_shfl<32, rs_n(N, 5)>(v, lane & 32);
  return v[0];
}

__global__ __launch_bounds__(1024) void router_gemv_kernel(const uint16_t* __restrict__ r,
                                                           const uint16_t* __restrict__ delta, int H, float eps,
                                                           const uint16_t* __restrict__ wr, int E,
                                                           uint16_t* __restrict__ r_next, uint16_t* __restrict__ x,
                                                           float* __restrict__ logits) {
  constexpr int NV = kGemvExperts;
  constexpr int LOGN = 4;
  static_assert(NV == 1 << LOGN, "expert count per workgroup");
  __shared__ float part[16];
  __shared__ float dot_part[16][NV];
  const int e0 = blockIdx.x * kGemvExperts;
  if (e0 >= E) return;  // chunk-count padding
  const int t = threadIdx.x, lane = t & 63, wave = t >> 6, nwaves = blockDim.x >> 6;
  const int nv = H >> 3;
  const int ir = min(t, nv - 1);
  const int m = blockIdx.y;

  uint4 wv[NV];
#pragma unroll
  for (int j = 0; j < NV; ++j)
    wv[j] = *reinterpret_cast<const uint4*>(wr + (uint64_t)min(e0 + j, E - 1) * H + 8 * ir);
  const uint64_t o = (uint64_t)m * H;
  ResRow rr;
  rr.a = *reinterpret_cast<const h8_t*>(r + o + 8 * ir);
  if (delta) rr.b = *reinterpret_cast<const h8_t*>(delta + o + 8 * ir);

  // residual_finish's arithmetic, in registers
  const bool on = t < nv;
  h8_t a = rr.a;
  if (delta) {
#pragma unroll
    for (int e = 0; e < 8; ++e) a[e] = (_Float16)((float)a[e] + (float)rr.b[e]);
  }
  float ss = 0.f;
  if (!on) a = h8_t{};
#pragma unroll
  for (int e = 0; e < 8; ++e) ss = fmaf((float)a[e], (float)a[e], ss);
  ss = wave_sum_xor_order(ss);
  if (lane == 0) part[wave] = ss;
  __syncthreads();
  float tot = 0.f;
  for (int i = 0; i < nwaves; ++i) tot += part[i];
  const float inv = inv_rms_row(tot, H, eps);
  h8_t xo;
#pragma unroll
  for (int e = 0; e < 8; ++e) xo[e] = (_Float16)((float)a[e] * inv);
  if (blockIdx.x == 0 && on) {
    *reinterpret_cast<h8_t*>(r_next + o + 8 * t) = a;
    *reinterpret_cast<h8_t*>(x + o + 8 * t) = xo;
  }
  const uint4 xv = __builtin_bit_cast(uint4, xo);
  float acc[NV];
#pragma unroll
  for (int j = 0; j < NV; ++j) {
    float c = dot2(wv[j].x, xv.x, 0.f);
    c = dot2(wv[j].y, xv.y, c);
    c = dot2(wv[j].z, xv.z, c);
    acc[j] = dot2(wv[j].w, xv.w, c);
  }
  const float p = wave_reduce_scatter<NV>(acc);
  if (lane < NV) dot_part[wave][lane] = p;
  __syncthreads();
  if (t < NV) {
    float sum = 0.f;
    for (int w = 0; w < nwaves; ++w) sum += dot_part[w][t];
    const int e = e0 + (int)(__builtin_bitreverse32((uint32_t)t) >> (32 - LOGN));
    if (e < E) logits[(uint64_t)m * E + e] = sum;
  }
}

hipError_t launch_router_gemv(const uint16_t* r, const uint16_t* delta, int M, int H, float eps, const uint16_t* wr,
                              int E, uint16_t* r_next, uint16_t* x, float* logits, hipStream_t stream) {
  // chunk-major workgroup ids: the M rows of a chunk are 8 * k apart in
  // dispatch order and land on one XCD
  const int chunks = ((E + kGemvExperts - 1) / kGemvExperts + 7) / 8 * 8;
  const int threads = ((H / 8 + 63) / 64) * 64;
  hipLaunchKernelGGL(router_gemv_kernel, dim3(chunks, M), dim3(threads), 0, stream, r, delta, H, eps, wr, E, r_next,
                     x, logits);
  return hipGetLastError();
}

hipError_t launch_router_topk(const float* logits, int M, int E, int k, int32_t* ids, float* w, hipStream_t stream) {
  // E <= 4096 over at most 1024 threads: at most 4 keys per thread
  int threads = ((E + 63) / 64) * 64;
  if (threads > 1024) threads = 1024;
  hipLaunchKernelGGL(router_topk_kernel, dim3(M), dim3(threads), 0, stream, logits, E, k, ids, w);
  return hipGetLastError();
}

hipError_t launch_residual_rmsnorm(const uint16_t* r, const uint16_t* delta, int M, int H, float eps,
                                   uint16_t* r_next, uint16_t* x, hipStream_t stream) {
  int threads = ((H / 8 + 63) / 64) * 64;
  if (threads > 1024) threads = 1024;
  hipLaunchKernelGGL(residual_rmsnorm_kernel, dim3(M), dim3(threads), 0, stream, r, delta, H, eps, r_next, x);
  return hipGetLastError();
}

hipError_t launch_router_residual(const float* logits, int M, int E, int k, int32_t* ids, float* w,
                                  const uint16_t* r, const uint16_t* delta, int H, float eps, uint16_t* r_next,
                                  uint16_t* x, hipStream_t stream) {
  int threads = ((E + 63) / 64) * 64;
  const int rt = ((H / 8 + 63) / 64) * 64;
  if (rt > threads) threads = rt;
  if (threads > 1024) threads = 1024;
  hipLaunchKernelGGL(router_residual_kernel, dim3(M, 2), dim3(threads), 0, stream, logits, E, k, ids, w, r, delta, H,
                     eps, r_next, x);
  return hipGetLastError();
}

}  // namespace awq_moe
