// gfx950 kernels of the AWQ int4 MoE expert stage for small-batch decode.
//
// The stage follows PR #520 "[Perf][SM70] Narrow Qwen3.8 AWQ active grouped
// decode" (Purpose, Implementation): one offsets-based launch per stage over
// multi-row active-expert segments; W13 (gate/up interleaved) + SwiGLU; W2
// with the router-weighted reduction. Records are {fp16 scale, u8 zero},
// 3 or 4 bytes (PR #522 "Coalesce AWQ QPN W13 compact metadata loads...",
// Purpose). The pages' SM70 warp/shuffle/MMA kernels are prior art only;
// these kernels are built around 64-lane wavefronts streaming 16-byte loads:
//
//  * a lane owns one 32-value group of four adjacent output columns, so its
//    four weight loads are dwordx4 loads that are contiguous across lanes,
//    and its four records are one aligned 12- or 16-byte load (the bank
//    layout places them so; no cross-lane redistribution is needed);
//  * 4-bit values become fp16 by OR-ing them into the mantissa of 1024.0 or
//    64.0, and v_dot2_f32_f16 multiplies two of them with two fp16
//    activations per instruction into an fp32 accumulator; the constant
//    offsets and the zero point are removed once per group through the
//    per-group activation sums S = sum x and C = sum offset_k * x_k:
//        sum_k x_k (q_k - z) = acc - (C + z S),   group result = s * that;
//  * K is reduced inside the workgroup (wave shuffles, then LDS) in a fixed
//    order, so results are run-to-run deterministic and independent of the
//    order of a token's top-k pairs.

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "kernels.h"

namespace awq_moe {

typedef _Float16 h2_t __attribute__((ext_vector_type(2)));
typedef uint32_t u32x3_a4 __attribute__((ext_vector_type(3), aligned(4)));

// Bit pattern constants of the nibble -> fp16 conversion.
constexpr uint32_t kLoMask = 0x000F000Fu;   // values at bits 0 and 16
constexpr uint32_t kHiMask = 0x00F000F0u;   // values at bits 4 and 20
constexpr uint32_t kMagic1024 = 0x64006400u; // fp16 1024.0 twice: mantissa ulp 1
constexpr uint32_t kMagic64 = 0x54005400u;   // fp16 64.0 twice: ulp 1/16, so bits 4..7 count 1 each

__device__ __forceinline__ h2_t as_h2(uint32_t v) { return __builtin_bit_cast(h2_t, v); }

__device__ __forceinline__ float dot2(uint32_t a, uint32_t b, float c) {
  return __builtin_amdgcn_fdot2(as_h2(a), as_h2(b), c, false);
}

// Records of a lane's four columns: scale (fp16 -> fp32, exact) and zero.
template <int RB>
struct Records {
  float s[4];
  float z[4];
};

__device__ __forceinline__ void decode_record(uint32_t r, float& s, float& z) {
  _Float16 h = __builtin_bit_cast(_Float16, (uint16_t)(r & 0xFFFFu));
  s = (float)h;
  z = (float)((r >> 16) & 0xFFu);
}

template <int RB>
__device__ __forceinline__ Records<RB> load_records(const uint8_t* p) {
  Records<RB> out;
  uint32_t r[4];
  if constexpr (RB == 4) {
    uint4 v = *reinterpret_cast<const uint4*>(p);
    r[0] = v.x; r[1] = v.y; r[2] = v.z; r[3] = v.w;
  } else {
    u32x3_a4 v = *reinterpret_cast<const u32x3_a4*>(p);
    r[0] = v.x;
    r[1] = __builtin_amdgcn_alignbyte(v.y, v.x, 3);
    r[2] = __builtin_amdgcn_alignbyte(v.z, v.y, 2);
    r[3] = v.z >> 8;
  }
#pragma unroll
  for (int j = 0; j < 4; ++j) decode_record(r[j], out.s[j], out.z[j]);
  return out;
}

// 32 fp16 activations of one group as 16 packed pairs: px[4d + p] holds
// (x[8d + 2p], x[8d + 2p + 1]).
struct Act32 {
  uint32_t px[16];
};

__device__ __forceinline__ Act32 load_act32(const uint16_t* p) {
  Act32 a;
  const uint4* q = reinterpret_cast<const uint4*>(p);
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    uint4 v = q[i];
    a.px[4 * i + 0] = v.x; a.px[4 * i + 1] = v.y; a.px[4 * i + 2] = v.z; a.px[4 * i + 3] = v.w;
  }
  return a;
}

// Per-group sums: S = sum x, C = 1024 * (x at 1024-offset slots) + 64 * (x at 64-offset slots).
__device__ __forceinline__ void group_sums(const Act32& a, float& S, float& C) {
  const uint32_t one2 = 0x3C003C00u;  // fp16 (1.0, 1.0)
  float s1024 = 0.f, s64 = 0.f;
#pragma unroll
  for (int d = 0; d < 4; ++d) {
    s1024 = dot2(a.px[4 * d + 0], one2, s1024);
    s64 = dot2(a.px[4 * d + 1], one2, s64);
    s1024 = dot2(a.px[4 * d + 2], one2, s1024);
    s64 = dot2(a.px[4 * d + 3], one2, s64);
  }
  S = s1024 + s64;
  C = fmaf(1024.f, s1024, 64.f * s64);
}

// acc = sum_k x_k * (offset_k + q_k) over one unit (4 dwords = 32 values).
__device__ __forceinline__ float unit_dot(const uint4& w, const Act32& a) {
  float acc = 0.f;
  const uint32_t wd[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
  for (int d = 0; d < 4; ++d) {
    const uint32_t v = wd[d];
    const uint32_t v8 = v >> 8;
    acc = dot2(a.px[4 * d + 0], (v & kLoMask) | kMagic1024, acc);
    acc = dot2(a.px[4 * d + 1], (v & kHiMask) | kMagic64, acc);
    acc = dot2(a.px[4 * d + 2], (v8 & kLoMask) | kMagic1024, acc);
    acc = dot2(a.px[4 * d + 3], (v8 & kHiMask) | kMagic64, acc);
  }
  return acc;
}

__device__ __forceinline__ float silu_mul(float g, float u) {
  return g / (1.0f + __expf(-g)) * u;
}

// ---------------------------------------------------------------------------
// routing compaction: one workgroup, one thread per slot (n <= 256)
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void route_compact_kernel(
    const int32_t* __restrict__ ids, int n, int E, int32_t* __restrict__ active_ids,
    int32_t* __restrict__ offsets, int32_t* __restrict__ sorted_slots,
    int32_t* __restrict__ num_active, uint32_t* __restrict__ status) {
  __shared__ int key[256];    // id of a valid slot, -1 for an invalid one
  __shared__ int first[256];  // 1 when the slot is the first valid slot of its id
  const int s = threadIdx.x;
  int id = -1;
  if (s < n) {
    const int v = ids[s];
    id = (v >= 0 && v < E) ? v : -1;
    key[s] = id;
  }
  __syncthreads();
  int before = 0, inv_before = 0, nvalid = 0, is_first = 1;
  for (int s2 = 0; s2 < n; ++s2) {
    const int k2 = key[s2];
    nvalid += (k2 >= 0);
    if (id >= 0) {
      before += (k2 >= 0) && (k2 < id || (k2 == id && s2 < s));
      if (k2 == id && s2 < s) is_first = 0;
    } else {
      inv_before += (k2 < 0) && (s2 < s);
    }
  }
  if (s < n) first[s] = (id >= 0) && is_first;
  __syncthreads();
  int seg = 0, nseg = 0;
  for (int s2 = 0; s2 < n; ++s2) {
    const int f = first[s2];
    nseg += f;
    seg += f && (key[s2] < id);
  }
  if (s < n) {
    if (id >= 0) {
      sorted_slots[before] = s;
      if (is_first) {
        active_ids[seg] = id;
        offsets[seg] = before;
      }
    } else {
      sorted_slots[nvalid + inv_before] = s;
    }
    if (s >= nseg) active_ids[s] = -1;
  }
  for (int i = s; i <= n; i += blockDim.x)
    if (i >= nseg) offsets[i] = nvalid;
  if (s == 0) {
    *num_active = nseg;
    *status = (nvalid == n) ? 0u : 1u;
  }
}

// ---------------------------------------------------------------------------
// W13 + SwiGLU: grid (2I/16 column tiles, n segment slots); one workgroup
// streams one 16-column tile of one active expert over all of K once and
// applies it to every row of the segment.
// ---------------------------------------------------------------------------
template <int RB>
__global__ __launch_bounds__(1024) void w13_swiglu_kernel(
    const uint8_t* __restrict__ bank, uint64_t expert_bytes, uint64_t w13_off,
    uint64_t w13_meta_off, int H, int I, const uint16_t* __restrict__ x, int topk,
    const int32_t* __restrict__ active_ids, const int32_t* __restrict__ offsets,
    const int32_t* __restrict__ sorted_slots, const int32_t* __restrict__ num_active,
    uint16_t* __restrict__ act) {
  constexpr int R = 4;  // rows per pass
  __shared__ float red[16][R][16];  // [wave][row][column]
  const int seg = blockIdx.y;
  if (seg >= *num_active) return;
  const int nt = blockIdx.x;
  const int e = active_ids[seg];
  const int r_begin = offsets[seg], r_end = offsets[seg + 1];
  const int G = H >> 5;
  const int L = 4 * G;
  const int t = threadIdx.x;
  const int lane = t & 63, wave = t >> 6, nwaves = blockDim.x >> 6;
  const bool active = t < L;
  const int g = t >> 2;

  const uint8_t* blk = bank + (uint64_t)e * expert_bytes;
  uint4 w[4];
  Records<RB> rec;
  if (active) {
    const uint8_t* units = blk + w13_off + (uint64_t)nt * 256u * G;
#pragma unroll
    for (int j = 0; j < 4; ++j) w[j] = *reinterpret_cast<const uint4*>(units + ((uint64_t)j * L + t) * 16u);
    rec = load_records<RB>(blk + w13_meta_off + (uint64_t)nt * 16u * G * RB + (uint64_t)t * 4u * RB);
  }

  for (int r0 = r_begin; r0 < r_end; r0 += R) {
    float part[R][4];
#pragma unroll
    for (int rr = 0; rr < R; ++rr) {
#pragma unroll
      for (int j = 0; j < 4; ++j) part[rr][j] = 0.f;
      if (active && r0 + rr < r_end) {
        const int tok = sorted_slots[r0 + rr] / topk;
        const Act32 a = load_act32(x + (uint64_t)tok * H + 32 * g);
        float S, C;
        group_sums(a, S, C);
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const float acc = unit_dot(w[j], a);
          part[rr][j] = rec.s[j] * (acc - fmaf(rec.z[j], S, C));
        }
      }
    }
    // reduce over the 16 groups of this wave: lanes with equal (lane & 3)
#pragma unroll
    for (int rr = 0; rr < R; ++rr)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        float v = part[rr][j];
        v += __shfl_xor(v, 4);
        v += __shfl_xor(v, 8);
        v += __shfl_xor(v, 16);
        v += __shfl_xor(v, 32);
        part[rr][j] = v;
      }
    if (lane < 4) {
#pragma unroll
      for (int rr = 0; rr < R; ++rr)
#pragma unroll
        for (int j = 0; j < 4; ++j) red[wave][rr][4 * lane + j] = part[rr][j];
    }
    __syncthreads();
    if (t < 16 * R) {
      const int col = t & 15, rr = t >> 4;
      float h = 0.f;
      for (int wv = 0; wv < nwaves; ++wv) h += red[wv][rr][col];
      const float other = __shfl_xor(h, 1);  // partner column: gate <-> up
      if (!(col & 1) && r0 + rr < r_end) {
        const float v = silu_mul(h, other);
        act[(uint64_t)(r0 + rr) * I + nt * 8 + (col >> 1)] = __builtin_bit_cast(uint16_t, (_Float16)v);
      }
    }
    __syncthreads();
  }
}

// ---------------------------------------------------------------------------
// W2 + router-weighted reduction: grid (H/8 column tiles); one workgroup owns
// 8 output columns for all tokens and walks every active segment, so a
// token's sum over its experts never leaves the workgroup.
// ---------------------------------------------------------------------------
template <int RB>
__global__ __launch_bounds__(512) void w2_reduce_kernel(
    const uint8_t* __restrict__ bank, uint64_t expert_bytes, uint64_t w2_off,
    uint64_t w2_meta_off, int H, int I, const uint16_t* __restrict__ act,
    const float* __restrict__ topk_w, int M, int topk, int SS,
    const int32_t* __restrict__ active_ids, const int32_t* __restrict__ offsets,
    const int32_t* __restrict__ sorted_slots, const int32_t* __restrict__ num_active,
    uint16_t* __restrict__ out) {
  extern __shared__ float red[];  // [M][8][SS*G2] then [M][8][G2]
  const int nt = blockIdx.x;
  const int G2 = I >> 5;
  const int L2 = 2 * G2;
  const int t = threadIdx.x;
  const int sl = t / L2, tl = t - sl * L2;
  const int g = tl >> 1, quad = tl & 1;
  const int nseg = *num_active;

  float acc[AWQ_MOE_KMAX_TOKENS][4];
#pragma unroll
  for (int tt = 0; tt < AWQ_MOE_KMAX_TOKENS; ++tt)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[tt][j] = 0.f;

  if (sl < SS) {
    for (int seg = sl; seg < nseg; seg += SS) {
      const int e = active_ids[seg];
      const uint8_t* blk = bank + (uint64_t)e * expert_bytes;
      const uint8_t* units = blk + w2_off + (uint64_t)nt * 128u * G2;
      uint4 w[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) w[j] = *reinterpret_cast<const uint4*>(units + ((uint64_t)j * L2 + tl) * 16u);
      const Records<RB> rec =
          load_records<RB>(blk + w2_meta_off + (uint64_t)nt * 8u * G2 * RB + (uint64_t)tl * 4u * RB);
      const int r_end = offsets[seg + 1];
      for (int r = offsets[seg]; r < r_end; ++r) {
        const int slot = sorted_slots[r];
        const int tok = slot / topk;
        const float wr = topk_w[slot];
        const Act32 a = load_act32(act + (uint64_t)r * I + 32 * g);
        float S, C;
        group_sums(a, S, C);
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const float y = rec.s[j] * (unit_dot(w[j], a) - fmaf(rec.z[j], S, C));
#pragma unroll
          for (int tt = 0; tt < AWQ_MOE_KMAX_TOKENS; ++tt)
            if (tt == tok) acc[tt][j] = fmaf(wr, y, acc[tt][j]);
        }
      }
    }
  }
  // reduction over (segment slot, group) in a fixed order
  const int P = SS * G2;
  float* red2 = red + (size_t)M * 8 * P;
  if (sl < SS) {
#pragma unroll
    for (int tt = 0; tt < AWQ_MOE_KMAX_TOKENS; ++tt)
      if (tt < M) {
#pragma unroll
        for (int j = 0; j < 4; ++j) red[((size_t)tt * 8 + 4 * quad + j) * P + sl * G2 + g] = acc[tt][j];
      }
  }
  __syncthreads();
  for (int i = t; i < M * 8 * G2; i += blockDim.x) {
    const int gg = i % G2, tc = i / G2;  // tc = token*8 + column
    float v = 0.f;
    for (int s2 = 0; s2 < SS; ++s2) v += red[(size_t)tc * P + s2 * G2 + gg];
    red2[(size_t)tc * G2 + gg] = v;
  }
  __syncthreads();
  for (int i = t; i < M * 8; i += blockDim.x) {
    float v = 0.f;
    for (int gg = 0; gg < G2; ++gg) v += red2[(size_t)i * G2 + gg];
    const int tt = i >> 3, col = i & 7;
    out[(uint64_t)tt * H + nt * 8 + col] = __builtin_bit_cast(uint16_t, (_Float16)v);
  }
}

// ---------------------------------------------------------------------------
// dequantisation (diagnostic): one thread per unit, writes 32 fp32 values
// ---------------------------------------------------------------------------
template <int RB>
__global__ void dequant_kernel(const uint8_t* __restrict__ bank, uint64_t expert_bytes,
                               uint64_t units_off, uint64_t meta_off, int which, int K, int N,
                               int expert_begin, int expert_count, float* __restrict__ out) {
  const int G = K >> 5;
  const uint64_t per_expert = (uint64_t)G * N;
  const uint64_t idx = (uint64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (idx >= per_expert * (uint64_t)expert_count) return;
  const int el = (int)(idx / per_expert);
  const int rem = (int)(idx - (uint64_t)el * per_expert);
  const int g = rem / N, n = rem - g * N;
  uint64_t uo, ro;
  if (which == 0) {
    const int L = 4 * G, nt = n >> 4, c = n & 15, quad = c >> 2, j = c & 3, t = 4 * g + quad;
    uo = (uint64_t)nt * 256u * G + ((uint64_t)j * L + t) * 16u;
    ro = (uint64_t)nt * 16u * G * RB + (uint64_t)(4 * t + j) * RB;
  } else {
    const int L = 2 * G, nt = n >> 3, c = n & 7, quad = c >> 2, j = c & 3, t = 2 * g + quad;
    uo = (uint64_t)nt * 128u * G + ((uint64_t)j * L + t) * 16u;
    ro = (uint64_t)nt * 8u * G * RB + (uint64_t)(4 * t + j) * RB;
  }
  const uint8_t* blk = bank + (uint64_t)(expert_begin + el) * expert_bytes;
  const uint4 w = *reinterpret_cast<const uint4*>(blk + units_off + uo);
  const uint8_t* rp = blk + meta_off + ro;
  const uint32_t r = (uint32_t)rp[0] | ((uint32_t)rp[1] << 8) | ((uint32_t)rp[2] << 16);
  float s, z;
  decode_record(r, s, z);
  const uint32_t wd[4] = {w.x, w.y, w.z, w.w};
  float* o = out + (uint64_t)el * K * N;
#pragma unroll
  for (int d = 0; d < 4; ++d)
#pragma unroll
    for (int p = 0; p < 8; ++p) {
      const uint32_t q = (wd[d] >> (4 * (p >> 1) + 16 * (p & 1))) & 0xFu;
      o[(uint64_t)(32 * g + 8 * d + p) * N + n] = ((float)q - z) * s;
    }
}

// ---------------------------------------------------------------------------
// launchers
// ---------------------------------------------------------------------------
hipError_t launch_route_compact(const int32_t* ids, int n, int E, int32_t* active_ids,
                                int32_t* offsets, int32_t* sorted_slots, int32_t* num_active,
                                uint32_t* status, hipStream_t stream) {
  hipLaunchKernelGGL(route_compact_kernel, dim3(1), dim3(256), 0, stream, ids, n, E, active_ids,
                     offsets, sorted_slots, num_active, status);
  return hipGetLastError();
}

hipError_t launch_w13_swiglu(const StageArgs& a, const uint16_t* x, uint16_t* act, hipStream_t stream) {
  const int L = 4 * (a.H / 32);
  const dim3 block(((L + 63) / 64) * 64);
  const dim3 grid((2 * a.I) / 16, a.M * a.topk);
  if (a.RB == 4)
    hipLaunchKernelGGL(w13_swiglu_kernel<4>, grid, block, 0, stream, a.bank, a.expert_bytes,
                       a.w13_off, a.w13_meta_off, a.H, a.I, x, a.topk, a.active_ids, a.offsets,
                       a.sorted_slots, a.num_active, act);
  else
    hipLaunchKernelGGL(w13_swiglu_kernel<3>, grid, block, 0, stream, a.bank, a.expert_bytes,
                       a.w13_off, a.w13_meta_off, a.H, a.I, x, a.topk, a.active_ids, a.offsets,
                       a.sorted_slots, a.num_active, act);
  return hipGetLastError();
}

int w2_segment_slots(int I) {
  const int L2 = 2 * (I / 32);
  int ss = 320 / L2;
  if (ss > 32) ss = 32;
  if (ss < 1) ss = 1;
  return ss;
}

size_t w2_lds_bytes(int M, int I) {
  const int G2 = I / 32;
  const int SS = w2_segment_slots(I);
  return (size_t)M * 8 * (SS * G2 + G2) * sizeof(float);
}

hipError_t launch_w2_reduce(const StageArgs& a, const uint16_t* act, const float* topk_w,
                            uint16_t* out, hipStream_t stream) {
  const int SS = w2_segment_slots(a.I);
  const int L2 = 2 * (a.I / 32);
  const dim3 block(((SS * L2 + 63) / 64) * 64);
  const dim3 grid(a.H / 8);
  const size_t lds = w2_lds_bytes(a.M, a.I);
  if (a.RB == 4)
    hipLaunchKernelGGL(w2_reduce_kernel<4>, grid, block, lds, stream, a.bank, a.expert_bytes,
                       a.w2_off, a.w2_meta_off, a.H, a.I, act, topk_w, a.M, a.topk, SS,
                       a.active_ids, a.offsets, a.sorted_slots, a.num_active, out);
  else
    hipLaunchKernelGGL(w2_reduce_kernel<3>, grid, block, lds, stream, a.bank, a.expert_bytes,
                       a.w2_off, a.w2_meta_off, a.H, a.I, act, topk_w, a.M, a.topk, SS,
                       a.active_ids, a.offsets, a.sorted_slots, a.num_active, out);
  return hipGetLastError();
}

hipError_t launch_dequant(const uint8_t* bank, uint64_t expert_bytes, uint64_t units_off,
                          uint64_t meta_off, int RB, int which, int K, int N, int expert_begin,
                          int expert_count, float* out, hipStream_t stream) {
  const uint64_t total = (uint64_t)(K / 32) * N * expert_count;
  const dim3 block(256);
  const dim3 grid((unsigned)((total + 255) / 256));
  if (RB == 4)
    hipLaunchKernelGGL(dequant_kernel<4>, grid, block, 0, stream, bank, expert_bytes, units_off,
                       meta_off, which, K, N, expert_begin, expert_count, out);
  else
    hipLaunchKernelGGL(dequant_kernel<3>, grid, block, 0, stream, bank, expert_bytes, units_off,
                       meta_off, which, K, N, expert_begin, expert_count, out);
  return hipGetLastError();
}

}  // namespace awq_moe
