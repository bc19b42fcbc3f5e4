// gfx950 kernels of the indexed prefill stage: the same expert computation
// as the decode stage for M >= 9 tokens (PR #520 "[Perf][SM70] Narrow
// Qwen3.8 AWQ active grouped decode", Tests: indexed prefill is admitted
// from 9 tokens, disjoint from the grouped decode's 1..8).
//
// With many tokens an expert serves several rows, so the work is expert-major
// and the products run on the matrix cores:
//
//  * route: one workgroup counts the slots per expert, lays the experts'
//    rows out in ascending expert order and cuts each expert's rows into
//    work items of at most 32 rows (two 16-row MFMA tiles);
//  * W13 + SwiGLU: one workgroup per (work item, 16-column tile); each
//    group of 32 K values is one v_mfma_f32_16x16x32_f16 whose B operand is
//    the exact integer (q - z) in fp16 (|q - z| <= 255), so the dequantised
//    weight is never rounded; the group's fp32 result is scaled by s and
//    accumulated in fp32;
//  * W2: the same per (work item, 8 column tiles), writing fp32 row results;
//  * reduce: per token, the router-weighted fp32 sum of its rows in
//    ascending (expert id, slot) order, rounded once to fp16, as the decode
//    stage does.
//
// A row's result depends only on its token and expert, not on the other
// rows of its tile, so the order in which rows are placed inside an
// expert's segment (LDS atomics) does not change any output.

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "device_util.h"
#include "kernels.h"

namespace awq_moe {

typedef float f4_t __attribute__((ext_vector_type(4)));

constexpr int kItemRows = 32;

// ---------------------------------------------------------------------------
// routing: counts, row offsets per expert, work items, row of every slot.
// Thread t owns experts [4t, 4t + 4) in the scans (E <= 4096).
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(1024) void prefill_route_kernel(const int32_t* __restrict__ ids, int n, int E,
                                                             int32_t* __restrict__ slot_row,
                                                             int32_t* __restrict__ row_slot,
                                                             int32_t* __restrict__ items,
                                                             int32_t* __restrict__ num_items,
                                                             uint32_t* __restrict__ status) {
  __shared__ int cnt[AWQ_MOE_KMAX_ROUTER_E];
  __shared__ int cur[AWQ_MOE_KMAX_ROUTER_E];
  __shared__ int wsum[16][2];
  __shared__ int bad;
  const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
  for (int e = t; e < E; e += 1024) cnt[e] = 0;
  if (t == 0) bad = 0;
  __syncthreads();
  for (int s = t; s < n; s += 1024) {
    const int e = ids[s];
    if (e >= 0 && e < E)
      atomicAdd(&cnt[e], 1);
    else
      bad = 1;
  }
  __syncthreads();
  int c4[4], r4[4], i4[4], rs = 0, is = 0;
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const int e = 4 * t + q;
    c4[q] = e < E ? cnt[e] : 0;
    r4[q] = rs;
    i4[q] = is;
    rs += c4[q];
    is += (c4[q] + kItemRows - 1) / kItemRows;
  }
  int ri = rs, ii = is;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const int a = __shfl_up(ri, off), b = __shfl_up(ii, off);
    if (lane >= off) {
      ri += a;
      ii += b;
    }
  }
  if (lane == 63) {
    wsum[wave][0] = ri;
    wsum[wave][1] = ii;
  }
  __syncthreads();
  int rb = ri - rs, ib = ii - is;  // exclusive bases of this thread
  for (int w = 0; w < wave; ++w) {
    rb += wsum[w][0];
    ib += wsum[w][1];
  }
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const int e = 4 * t + q;
    if (e >= E) break;
    const int row0 = rb + r4[q], it0 = ib + i4[q];
    cur[e] = row0;
    for (int p = 0; p * kItemRows < c4[q]; ++p) {
      items[2 * (it0 + p)] = e;
      items[2 * (it0 + p) + 1] = (row0 + kItemRows * p) | (min(kItemRows, c4[q] - kItemRows * p) << 24);
    }
  }
  if (t == 1023) *num_items = ib + is;
  if (t == 0) *status = bad ? AWQ_MOE_STATUS_BAD_ID_BIT : 0u;
  __syncthreads();
  for (int s = t; s < n; s += 1024) {
    const int e = ids[s];
    if (e >= 0 && e < E) {
      const int r = atomicAdd(&cur[e], 1);
      slot_row[s] = r;
      row_slot[r] = s;
    } else {
      slot_row[s] = -1;
    }
  }
}

// ---------------------------------------------------------------------------
// MFMA operands. Lane l of a wave covers column c = l % 16 of a 16-column
// tile and K block kb = l / 16 (K values 8kb .. 8kb + 7 of a 32-value
// group) for B, and row l % 16 with the same K block for A; the result
// holds rows 4kb .. 4kb + 3 of column c.
// ---------------------------------------------------------------------------
template <int RB>
__device__ __forceinline__ uint32_t load_record1(const uint8_t* p) {
  if constexpr (RB == 4) {
    return *reinterpret_cast<const uint32_t*>(p);
  } else {
    return (uint32_t)p[0] | ((uint32_t)p[1] << 8) | ((uint32_t)p[2] << 16);
  }
}

// Eight (q - z) values in fp16 from one dword of a unit (value p of the dword
// at bits 4*(p/2) + 16*(p%2)) and the record's zero point. The nibbles become
// 1024 + q or 64 + q by OR-ing them into those numbers' mantissas; subtracting
// 1024 + z or 64 + z (integers below 2048, exact in fp16) leaves q - z exactly.
__device__ __forceinline__ h8_t qz_operand(uint32_t w, uint32_t z) {
  const _Float16 z1024 = (_Float16)(-(1024.0f + (float)z));
  const _Float16 z64 = (_Float16)(-(64.0f + (float)z));
  const h2_t c1024 = {z1024, z1024}, c64 = {z64, z64};
  const h2_t p0 = as_h2((w & 0x000F000Fu) | 0x64006400u) + c1024;
  const h2_t p1 = as_h2((w & 0x00F000F0u) | 0x54005400u) + c64;
  const h2_t p2 = as_h2(((w >> 8) & 0x000F000Fu) | 0x64006400u) + c1024;
  const h2_t p3 = as_h2(((w >> 8) & 0x00F000F0u) | 0x54005400u) + c64;
  return h8_t{p0[0], p0[1], p1[0], p1[1], p2[0], p2[1], p3[0], p3[1]};
}

__device__ __forceinline__ f4_t mfma16(const h8_t& a, const h8_t& b) {
  const f4_t zero = {0.f, 0.f, 0.f, 0.f};
  return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, zero, 0, 0, 0);
}

__device__ __forceinline__ void scale_add(f4_t& acc, float s, const f4_t& d) {
#pragma unroll
  for (int i = 0; i < 4; ++i) acc[i] = fmaf(s, d[i], acc[i]);
}

__device__ __forceinline__ void item_of(const int32_t* __restrict__ items, int it, int& e, int& row0, int& rows) {
  e = items[2 * it];
  const int rp = items[2 * it + 1];
  row0 = rp & 0xFFFFFF;
  rows = rp >> 24;
}

// ---------------------------------------------------------------------------
// W13 + SwiGLU: grid (2I/16 column tiles, work items), 4 waves; wave w takes
// the groups g = w, w + 4, ... and the waves' partial tiles are summed in
// LDS in wave order. Gate and up of intermediate i are columns 2i and 2i + 1,
// i.e. neighbouring lanes of the result.
// ---------------------------------------------------------------------------
template <int RB, int NRT>
__device__ __forceinline__ void w13_groups(const uint8_t* __restrict__ ub, const uint8_t* __restrict__ rbp,
                                           const uint16_t* __restrict__ xr0, const uint16_t* __restrict__ xr1,
                                           int G, int wave, int kb, f4_t (&acc)[2]) {
#pragma unroll 4
  for (int g = wave; g < G; g += 4) {
    const uint32_t w = *reinterpret_cast<const uint32_t*>(ub + 64 * g);
    const uint32_t r = load_record1<RB>(rbp + 16 * g * RB);
    const float s = (float)__builtin_bit_cast(_Float16, (uint16_t)(r & 0xFFFFu));
    const h8_t b = qz_operand(w, (r >> 16) & 0xFFu);
    const h8_t a0 = *reinterpret_cast<const h8_t*>(xr0 + 32 * g + 8 * kb);
    scale_add(acc[0], s, mfma16(a0, b));
    if constexpr (NRT == 2) {
      const h8_t a1 = *reinterpret_cast<const h8_t*>(xr1 + 32 * g + 8 * kb);
      scale_add(acc[1], s, mfma16(a1, b));
    }
  }
}

template <int RB>
__global__ __launch_bounds__(256) void prefill_w13_kernel(const int32_t* __restrict__ items,
                                                          const int32_t* __restrict__ num_items,
                                                          const int32_t* __restrict__ row_slot,
                                                          const uint8_t* __restrict__ bank,
                                                          const uint16_t* __restrict__ x, uint64_t expert_bytes,
                                                          uint64_t units_off, uint64_t meta_off, int H, int I,
                                                          int topk, uint16_t* __restrict__ act) {
  __shared__ f4_t red[4][2][64];
  const int it = blockIdx.y;
  if (it >= *num_items) return;
  int e, row0, rows;
  item_of(items, it, e, row0, rows);
  const int nt = blockIdx.x, G = H >> 5;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int c = lane & 15, kb = lane >> 4, quad = c >> 2, j = c & 3;
  const uint8_t* blk = bank + (uint64_t)e * expert_bytes;
  // unit (g, column c) dword kb at nt*256G + (j*4G + 4g + quad)*16 + 4kb
  const uint8_t* ub = blk + units_off + (uint64_t)nt * 256 * G + (uint64_t)j * 64 * G + 16 * quad + 4 * kb;
  // record (g, column c) at nt*16G*RB + (16g + 4quad + j)*RB
  const uint8_t* rbp = blk + meta_off + (uint64_t)nt * 16 * G * RB + (uint64_t)(4 * quad + j) * RB;
  const int ra = min(c, rows - 1), rb = min(16 + c, rows - 1);
  const uint16_t* xr0 = x + (uint64_t)(row_slot[row0 + ra] / topk) * H;
  const uint16_t* xr1 = x + (uint64_t)(row_slot[row0 + rb] / topk) * H;
  f4_t acc[2] = {{0.f, 0.f, 0.f, 0.f}, {0.f, 0.f, 0.f, 0.f}};
  if (rows > 16)
    w13_groups<RB, 2>(ub, rbp, xr0, xr1, G, wave, kb, acc);
  else
    w13_groups<RB, 1>(ub, rbp, xr0, xr1, G, wave, kb, acc);
  red[wave][0][lane] = acc[0];
  red[wave][1][lane] = acc[1];
  __syncthreads();
  if (wave != 0) return;
  const int nrt = rows > 16 ? 2 : 1;
  for (int rt = 0; rt < nrt; ++rt) {
    const f4_t d = red[0][rt][lane] + red[1][rt][lane] + red[2][rt][lane] + red[3][rt][lane];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float up = dpp<kQuadSwap1>(d[i]);  // column c ^ 1
      const int row = 16 * rt + 4 * kb + i;
      if (!(c & 1) && row < rows) {
        const float g = d[i];
        const float a = g / (1.0f + __expf(-g)) * up;
        act[(uint64_t)(row0 + row) * I + nt * 8 + (c >> 1)] = __builtin_bit_cast(uint16_t, (_Float16)a);
      }
    }
  }
}

// ---------------------------------------------------------------------------
// W2: grid (ceil(H/16 / 8) column blocks, work items), 4 waves; wave w takes
// column tiles 8b + w and 8b + w + 4 over all I/32 groups; fp32 row results.
// ---------------------------------------------------------------------------
template <int RB, int NRT>
__device__ __forceinline__ void w2_tiles(const uint8_t* __restrict__ blk, uint64_t units_off, uint64_t meta_off,
                                         const uint16_t* __restrict__ ar0, const uint16_t* __restrict__ ar1, int G,
                                         int NT, int nt0, int lane, f4_t (&acc)[2][2]) {
  const int c = lane & 15, kb = lane >> 4, quad = c >> 2, j = c & 3;
  for (int g = 0; g < G; ++g) {
    const h8_t a0 = *reinterpret_cast<const h8_t*>(ar0 + 32 * g + 8 * kb);
    h8_t a1;
    if constexpr (NRT == 2) a1 = *reinterpret_cast<const h8_t*>(ar1 + 32 * g + 8 * kb);
#pragma unroll
    for (int q = 0; q < 2; ++q) {
      const int nt = nt0 + 4 * q;
      if (nt < NT) {
        const uint32_t w = *reinterpret_cast<const uint32_t*>(
            blk + units_off + (uint64_t)nt * 256 * G + (uint64_t)j * 64 * G + 64 * g + 16 * quad + 4 * kb);
        const uint32_t r =
            load_record1<RB>(blk + meta_off + (uint64_t)nt * 16 * G * RB + (uint64_t)(16 * g + 4 * quad + j) * RB);
        const float s = (float)__builtin_bit_cast(_Float16, (uint16_t)(r & 0xFFFFu));
        const h8_t b = qz_operand(w, (r >> 16) & 0xFFu);
        scale_add(acc[q][0], s, mfma16(a0, b));
        if constexpr (NRT == 2) scale_add(acc[q][1], s, mfma16(a1, b));
      }
    }
  }
}

template <int RB>
__global__ __launch_bounds__(256) void prefill_w2_kernel(const int32_t* __restrict__ items,
                                                         const int32_t* __restrict__ num_items,
                                                         const uint8_t* __restrict__ bank, uint64_t expert_bytes,
                                                         uint64_t units_off, uint64_t meta_off, int H, int I,
                                                         const uint16_t* __restrict__ act, float* __restrict__ y) {
  const int it = blockIdx.y;
  if (it >= *num_items) return;
  int e, row0, rows;
  item_of(items, it, e, row0, rows);
  const int G = I >> 5, NT = H >> 4;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int c = lane & 15, kb = lane >> 4;
  const int nt0 = blockIdx.x * 8 + wave;
  if (nt0 >= NT) return;
  const uint8_t* blk = bank + (uint64_t)e * expert_bytes;
  const uint16_t* ar0 = act + (uint64_t)(row0 + min(c, rows - 1)) * I;
  const uint16_t* ar1 = act + (uint64_t)(row0 + min(16 + c, rows - 1)) * I;
  f4_t acc[2][2] = {};
  if (rows > 16)
    w2_tiles<RB, 2>(blk, units_off, meta_off, ar0, ar1, G, NT, nt0, lane, acc);
  else
    w2_tiles<RB, 1>(blk, units_off, meta_off, ar0, ar1, G, NT, nt0, lane, acc);
  const int nrt = rows > 16 ? 2 : 1;
#pragma unroll
  for (int q = 0; q < 2; ++q) {
    const int nt = nt0 + 4 * q;
    if (nt >= NT) break;
    for (int rt = 0; rt < nrt; ++rt) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int row = 16 * rt + 4 * kb + i;
        if (row < rows) y[(uint64_t)(row0 + row) * H + nt * 16 + c] = acc[q][rt][i];
      }
    }
  }
}

// ---------------------------------------------------------------------------
// reduce: grid (ceil(H/512), M), one wave; lane l sums columns 8l .. 8l + 7 of
// a 512-column block. The token's valid slots are ranked by (expert id,
// slot) with lane reads, then summed in that order: acc = fma(w, y, acc)
// from +0, rounded once to fp16.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(64) void prefill_reduce_kernel(const int32_t* __restrict__ ids,
                                                            const float* __restrict__ topk_w,
                                                            const int32_t* __restrict__ slot_row,
                                                            const float* __restrict__ y, int H, int topk, int E,
                                                            uint16_t* __restrict__ out) {
  __shared__ int order_row[AWQ_MOE_KMAX_TOPK];
  __shared__ float order_w[AWQ_MOE_KMAX_TOPK];
  const int tok = blockIdx.y, lane = threadIdx.x;
  const int s = tok * topk + lane;
  int id = lane < topk ? ids[s] : -1;
  const bool valid = lane < topk && id >= 0 && id < E;
  const int key = valid ? id * 32 + lane : 0x7FFFFFFF;
  int rank = 0;
  for (int jj = 0; jj < topk; ++jj) rank += __builtin_amdgcn_readlane(key, jj) < key;
  if (valid) {
    order_row[rank] = slot_row[s];
    order_w[rank] = topk_w[s];
  }
  const int nvalid = __popcll(__ballot(valid));
  __syncthreads();
  const int col = blockIdx.x * 512 + 8 * lane;
  if (col >= H) return;
  float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  for (int r = 0; r < nvalid; ++r) {
    const float w = order_w[r];
    const float* yr = y + (uint64_t)order_row[r] * H + col;
    const float4 v0 = *reinterpret_cast<const float4*>(yr);
    const float4 v1 = *reinterpret_cast<const float4*>(yr + 4);
    acc[0] = fmaf(w, v0.x, acc[0]);
    acc[1] = fmaf(w, v0.y, acc[1]);
    acc[2] = fmaf(w, v0.z, acc[2]);
    acc[3] = fmaf(w, v0.w, acc[3]);
    acc[4] = fmaf(w, v1.x, acc[4]);
    acc[5] = fmaf(w, v1.y, acc[5]);
    acc[6] = fmaf(w, v1.z, acc[6]);
    acc[7] = fmaf(w, v1.w, acc[7]);
  }
  h8_t o;
#pragma unroll
  for (int i = 0; i < 8; ++i) o[i] = (_Float16)acc[i];
  *reinterpret_cast<h8_t*>(out + (uint64_t)tok * H + col) = o;
}

// ---------------------------------------------------------------------------
// launchers
// ---------------------------------------------------------------------------
int prefill_max_items(int n, int E) { return (n + kItemRows - 1) / kItemRows + (E < n ? E : n); }

hipError_t launch_prefill(const StageArgs& a, const uint16_t* x, const float* topk_w, uint16_t* out,
                          const PrefillWs& w, hipStream_t stream) {
  const int n = a.M * a.topk;
  const int max_items = prefill_max_items(n, a.E);
  hipLaunchKernelGGL(prefill_route_kernel, dim3(1), dim3(1024), 0, stream, a.topk_ids, n, a.E, w.slot_row,
                     w.row_slot, w.items, w.num_items, w.status);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;
  const dim3 g13((2 * a.I) / 16, max_items), g2(((a.H / 16) + 7) / 8, max_items);
  if (a.RB == 4) {
    hipLaunchKernelGGL(prefill_w13_kernel<4>, g13, dim3(256), 0, stream, w.items, w.num_items, w.row_slot, a.bank, x,
                       a.expert_bytes, a.w13_off, a.w13_meta_off, a.H, a.I, a.topk, w.act);
  } else {
    hipLaunchKernelGGL(prefill_w13_kernel<3>, g13, dim3(256), 0, stream, w.items, w.num_items, w.row_slot, a.bank, x,
                       a.expert_bytes, a.w13_off, a.w13_meta_off, a.H, a.I, a.topk, w.act);
  }
  if ((err = hipGetLastError()) != hipSuccess) return err;
  if (a.RB == 4) {
    hipLaunchKernelGGL(prefill_w2_kernel<4>, g2, dim3(256), 0, stream, w.items, w.num_items, a.bank, a.expert_bytes,
                       a.w2_off, a.w2_meta_off, a.H, a.I, w.act, w.y);
  } else {
    hipLaunchKernelGGL(prefill_w2_kernel<3>, g2, dim3(256), 0, stream, w.items, w.num_items, a.bank, a.expert_bytes,
                       a.w2_off, a.w2_meta_off, a.H, a.I, w.act, w.y);
  }
  if ((err = hipGetLastError()) != hipSuccess) return err;
  hipLaunchKernelGGL(prefill_reduce_kernel, dim3((a.H + 511) / 512, a.M), dim3(64), 0, stream, a.topk_ids, topk_w,
                     w.slot_row, w.y, a.H, a.topk, a.E, out);
  return hipGetLastError();
}

}  // namespace awq_moe
