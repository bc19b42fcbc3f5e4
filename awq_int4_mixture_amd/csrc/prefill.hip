// gfx950 kernels of the indexed prefill stage: the same expert computation
// as the decode stage for M >= 9 tokens (PR #520 "[Perf][SM70] Narrow
// Qwen3.8 AWQ active grouped decode", Tests: indexed prefill is admitted
// from 9 tokens, disjoint from the grouped decode's 1..8).
//
// Calls of up to 64 tokens and 1,024 slots run the decode kernels on all of
// their tokens (launch_prefill). With more, an expert serves several rows,
// so the work is expert-major and the products run on the matrix cores:
//
//  * route (one workgroup up to 16,384 slots, else two launches over slices
//    of the slots): counts per expert, the experts' rows laid out in
//    ascending expert order, each expert's rows cut into work items of at
//    most 32 rows and wide items of at most 64;
//  * up to 64 tokens, W13 + SwiGLU per (work item, 16-column tile) and W2
//    per (work item, 8 column tiles); from 65 tokens the wide kernels: both
//    products of a wide item in one workgroup at inter <= 160, else W13 per
//    (wide item, 20 column tiles) and W2 per (work item or wide item, 16 or
//    20 column tiles). Each group of 32 K
//    values is one v_mfma_f32_16x16x32_f16 whose B operand is the exact
//    integer (q - z) in fp16 (|q - z| <= 255), so the dequantised weight is
//    never rounded; the group's fp32 result is scaled by s and accumulated
//    in fp32. W2 writes fp32 row results;
//  * reduce: per token, the router-weighted fp32 sum of its rows in
//    ascending (expert id, slot) order, rounded once to fp16, as the decode
//    stage does.
//
// A row's result depends only on its token and expert, not on the other
// rows of its tile, so the order in which rows are placed inside an
// expert's segment (LDS atomics) does not change any output.

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

#include "device_util.h"
#include "kernels.h"

namespace awq_moe {

typedef float f4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

// 16 bytes of the bank; NT marks the load non-temporal (data that no other
// workgroup of the launch will read soon, so the caches need not keep it).
template <bool NT>
__device__ __forceinline__ u32x4_t load16(const uint8_t* p) {
  if constexpr (NT)
    return __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(p));
  else
    return *reinterpret_cast<const u32x4_t*>(p);
}

constexpr int kItemRows = 32;
constexpr int kWideRows = 64;  // rows of a wide work item (the many-rows W13 kernel), a multiple of 16
constexpr int kRouteBatch = 16;           // slot ids per thread in flight in the routing kernels
constexpr int kRouteSlotsPerBlock = 2048;  // slots per routing workgroup (when E allows)
constexpr int kRouteCountCap = 65536;      // workgroups x experts of the per-workgroup counts

// ---------------------------------------------------------------------------
// routing. Up to kRouteBatch * 1024 slots, one workgroup does all of it in
// one launch (place with SINGLE). Beyond, two launches over B workgroups
// that each own a contiguous slice of the slots (B from prefill_route_blocks):
//  * count: the slice's slots per expert (LDS atomics), written to
//    cnt[b][E], and whether the slice holds an id outside [0, E);
//  * place: every workgroup sums cnt over the workgroups for each expert
//    (the total, and the part of the workgroups before it), scans the totals
//    over experts (rows, 32-row items, wide items; thread t owns experts
//    [4t, 4t + 4), E <= 4096), and gives each of its slots the next row of its
//    expert's range after the rows of the lower experts and of the earlier
//    workgroups (LDS atomics: the order inside a workgroup's share of an
//    expert is unspecified). Workgroup 0 writes the items, their numbers and
//    the status word.
// ---------------------------------------------------------------------------
int prefill_route_blocks(int n, int E) {
  int b = (n + kRouteSlotsPerBlock - 1) / kRouteSlotsPerBlock;
  b = min(b, kRouteCountCap / E);
  return max(b, 1);
}

// The slots [s0, s1) of this workgroup, kRouteBatch per thread in flight:
// f(slot, id) for each.
template <class F>
__device__ __forceinline__ void for_slots(const int32_t* __restrict__ ids, int s0, int s1, F&& f) {
  for (int sb = s0 + (int)threadIdx.x; sb < s1; sb += kRouteBatch * 1024) {
    int ev[kRouteBatch];
#pragma unroll
    for (int b = 0; b < kRouteBatch; ++b) {
      const int s = sb + 1024 * b;
      ev[b] = s < s1 ? ids[s] : 0;
    }
#pragma unroll
    for (int b = 0; b < kRouteBatch; ++b) {
      const int s = sb + 1024 * b;
      if (s >= s1) break;
      f(s, ev[b]);
    }
  }
}

__global__ __launch_bounds__(1024) void prefill_count_kernel(const int32_t* __restrict__ ids, int n, int E, int per,
                                                             int32_t* __restrict__ cnt, int32_t* __restrict__ bad) {
  __shared__ int c[AWQ_MOE_KMAX_ROUTER_E];
  __shared__ int any_bad;
  const int t = threadIdx.x, b = blockIdx.x;
  for (int e = t; e < E; e += 1024) c[e] = 0;
  if (t == 0) any_bad = 0;
  __syncthreads();
  const int s0 = b * per, s1 = min(n, s0 + per);
  for_slots(ids, s0, s1, [&](int, int e) {
    if (e >= 0 && e < E)
      atomicAdd(&c[e], 1);
    else
      any_bad = 1;
  });
  __syncthreads();
  for (int e = t; e < E; e += 1024) cnt[(uint64_t)b * E + e] = c[e];
  if (t == 0) bad[b] = any_bad;
}

// SINGLE (n <= kRouteBatch * 1024 slots, one workgroup): the count is taken
// here from the ids held in registers, which then also serve the placement
// (one launch, one read of the ids).
template <bool SINGLE>
__global__ __launch_bounds__(1024) void prefill_place_kernel(const int32_t* __restrict__ ids, int n, int E, int per,
                                                             int nb, const int32_t* __restrict__ cnt,
                                                             const int32_t* __restrict__ bad,
                                                             int32_t* __restrict__ slot_row,
                                                             int32_t* __restrict__ row_slot,
                                                             int32_t* __restrict__ items,
                                                             int32_t* __restrict__ num_items,
                                                             int32_t* __restrict__ witems,
                                                             int32_t* __restrict__ num_witems,
                                                             uint32_t* __restrict__ status) {
  // SINGLE: once the counts are in registers, their LDS takes the slot of
  // each row (u16: n <= 16384), so that row_slot is written in row order
  // (one workgroup's scattered 4-byte stores of it measured 5 us of the
  // 10 us routing at 10,240 slots)
  static_assert(kRouteBatch * 1024 <= 65536 && kRouteBatch * 1024 * 2 >= AWQ_MOE_KMAX_ROUTER_E * 4,
                "slots fit u16 and the row slots fit the counts' LDS");
  __shared__ union {
    int tot[AWQ_MOE_KMAX_ROUTER_E];
    uint16_t slot_of[kRouteBatch * 1024];
  } lds;
  int* tot = lds.tot;
  __shared__ int cur[AWQ_MOE_KMAX_ROUTER_E];
  __shared__ int wsum[16][3];
  __shared__ int any_bad, nrows_s;
  const int t = threadIdx.x, lane = t & 63, wave = t >> 6, b = blockIdx.x;
  int ev[kRouteBatch];  // SINGLE: the ids of slots t + 1024 q
  if constexpr (SINGLE) {
#pragma unroll
    for (int q = 0; q < kRouteBatch; ++q) ev[q] = t + 1024 * q < n ? ids[t + 1024 * q] : 0;  // all in flight
    for (int e = t; e < E; e += 1024) tot[e] = cur[e] = 0;
    if (t == 0) any_bad = 0;
    __syncthreads();
#pragma unroll
    for (int q = 0; q < kRouteBatch; ++q) {
      if (t + 1024 * q >= n) break;
      if (ev[q] >= 0 && ev[q] < E)
        atomicAdd(&tot[ev[q]], 1);
      else
        any_bad = 1;
    }
    __syncthreads();
  }
  // totals per expert and the share of the workgroups before this one
  for (int e = t; !SINGLE && e < E; e += 1024) {
    int all = 0, before = 0;
    for (int w0 = 0; w0 < nb; w0 += 8) {
      int v[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) v[u] = w0 + u < nb ? cnt[(uint64_t)(w0 + u) * E + e] : 0;  // 8 requests in flight
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        all += v[u];
        before += w0 + u < b ? v[u] : 0;
      }
    }
    tot[e] = all;
    cur[e] = before;
  }
  __syncthreads();
  int c4[4], r4[4], i4[4], w4[4], rs = 0, is = 0, ws = 0;
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const int e = 4 * t + q;
    c4[q] = e < E ? tot[e] : 0;
    r4[q] = rs;
    i4[q] = is;
    w4[q] = ws;
    rs += c4[q];
    is += (c4[q] + kItemRows - 1) / kItemRows;
    ws += (c4[q] + kWideRows - 1) / kWideRows;
  }
  int ri = rs, ii = is, wi = ws;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const int a = __shfl_up(ri, off), bb = __shfl_up(ii, off), d = __shfl_up(wi, off);
    if (lane >= off) {
      ri += a;
      ii += bb;
      wi += d;
    }
  }
  if (lane == 63) {
    wsum[wave][0] = ri;
    wsum[wave][1] = ii;
    wsum[wave][2] = wi;
  }
  __syncthreads();
  int rb = ri - rs, ib = ii - is, wb = wi - ws;  // exclusive bases of this thread
  for (int w = 0; w < wave; ++w) {
    rb += wsum[w][0];
    ib += wsum[w][1];
    wb += wsum[w][2];
  }
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const int e = 4 * t + q;
    if (e >= E) break;
    const int row0 = rb + r4[q], it0 = ib + i4[q], wt0 = wb + w4[q];
    cur[e] += row0;  // this workgroup's first row of expert e
    if (b != 0) continue;
    for (int p = 0; p * kItemRows < c4[q]; ++p) {
      items[2 * (it0 + p)] = e;
      items[2 * (it0 + p) + 1] = (row0 + kItemRows * p) | (min(kItemRows, c4[q] - kItemRows * p) << 24);
    }
    // wide items: ceil(c / 64) of them, the rows shared out in multiples of 16
    const int nw = (c4[q] + kWideRows - 1) / kWideRows;
    const int pw = nw ? ((c4[q] + nw - 1) / nw + 15) / 16 * 16 : 0;
    for (int p = 0; p < nw; ++p) {
      witems[2 * (wt0 + p)] = e;
      witems[2 * (wt0 + p) + 1] = (row0 + pw * p) | (min(pw, c4[q] - pw * p) << 24);
    }
  }
  if (b == 0 && t == 1023) {
    *num_items = ib + is;
    *num_witems = wb + ws;
  }
  if (t == 1023) nrows_s = rb + rs;  // rows of all experts (the valid slots)
  if (b == 0 && t == 0) {
    int any = SINGLE ? any_bad : 0;
    for (int w = 0; !SINGLE && w < nb; ++w) any |= bad[w];
    *status = any ? AWQ_MOE_STATUS_BAD_ID_BIT : 0u;
  }
  __syncthreads();  // the counts' LDS is free from here
  if constexpr (SINGLE) {
#pragma unroll
    for (int q = 0; q < kRouteBatch; ++q) {
      const int s = t + 1024 * q;
      if (s >= n) break;
      const int e = ev[q];
      if (e >= 0 && e < E) {
        const int r = atomicAdd(&cur[e], 1);
        slot_row[s] = r;
        lds.slot_of[r] = (uint16_t)s;
      } else {
        slot_row[s] = -1;
      }
    }
    __syncthreads();
    for (int r = t; r < nrows_s; r += 1024) row_slot[r] = lds.slot_of[r];
    return;
  }
  const int s0 = b * per, s1 = min(n, s0 + per);
  for_slots(ids, s0, s1, [&](int s, int e) {
    if (e >= 0 && e < E) {
      const int r = atomicAdd(&cur[e], 1);
      slot_row[s] = r;
      row_slot[r] = s;
    } else {
      slot_row[s] = -1;
    }
  });
}

// ---------------------------------------------------------------------------
// MFMA operands. Lane l of a wave covers column c = l % 16 of a 16-column
// tile and K block kb = l / 16 (K values 8kb .. 8kb + 7 of a 32-value
// group) for B, and row l % 16 with the same K block for A; the result
// holds rows 4kb .. 4kb + 3 of column c.
// ---------------------------------------------------------------------------
// Eight (q - z) values in fp16 from one dword of a unit (value p of the dword
// at bits 4*(p/2) + 16*(p%2)) and the record's zero point. Each pair of
// nibbles is shifted to bits 0..3 and 16..19 and OR-ed into the mantissas of
// a packed 1024.0 (exponent pattern m1024, kept in a VGPR so the mask and
// the OR are one v_and_or_b32), giving 1024 + q exactly; adding the packed
// fp16 -(1024 + z), whose bit pattern is 0xE400 + z for z <= 255, leaves
// q - z exactly (an integer of magnitude <= 255).
__device__ __forceinline__ uint32_t magic1024() {
  uint32_t m;
  asm volatile("v_mov_b32 %0, 0x64006400" : "=v"(m));
  return m;
}

__device__ __forceinline__ h8_t qz_operand(uint32_t w, uint32_t z, uint32_t m1024) {
  const h2_t cz = as_h2(0xE400E400u + z * 0x10001u);
  const h2_t p0 = as_h2((w & 0x000F000Fu) | m1024) + cz;
  const h2_t p1 = as_h2(((w >> 4) & 0x000F000Fu) | m1024) + cz;
  const h2_t p2 = as_h2(((w >> 8) & 0x000F000Fu) | m1024) + cz;
  const h2_t p3 = as_h2(((w >> 12) & 0x000F000Fu) | m1024) + cz;
  return __builtin_bit_cast(h8_t, make_uint4(__builtin_bit_cast(uint32_t, p0), __builtin_bit_cast(uint32_t, p1),
                                             __builtin_bit_cast(uint32_t, p2), __builtin_bit_cast(uint32_t, p3)));
}

__device__ __forceinline__ f4_t mfma16(const h8_t& a, const h8_t& b) {
  const f4_t zero = {0.f, 0.f, 0.f, 0.f};
  return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, zero, 0, 0, 0);
}

__device__ __forceinline__ void scale_add(f4_t& acc, float s, const f4_t& d) {
#pragma unroll
  for (int i = 0; i < 4; ++i) acc[i] = fmaf(s, d[i], acc[i]);
}

// Linear workgroup ids are dealt to the 8 XCDs round robin. With a grid of
// (NT tiles, items rounded up to a multiple of 8 << run_log2) this maps
// linear id L so that an item's NT tiles are consecutive ids of one XCD,
// which then reads the item's activation rows into its L2 once, and runs of
// 2^run_log2 consecutive items (an expert's items are consecutive) go to one
// XCD together, where the expert's weights are read into its L2 once for
// all of them. XCD x = L % 8 takes its q-th item, q = (L / 8) / NT, from
// run q >> run_log2 of the runs dealt to it:
// item = ((q >> run_log2) << (run_log2 + 3)) + (x << run_log2) + q % 2^run_log2,
// tile = (L / 8) % NT (a bijection on the grid). With run_log2 = 0 items are
// dealt one at a time. Runs pay where experts have several items; where
// they have one, a run's granularity only unbalances the XCDs (M = 128:
// 120 against 116 us per call).
__device__ __forceinline__ void xcd_item_tile(int run_log2, int& item, int& tile) {
  const int NT = gridDim.x;
  const int L = blockIdx.y * NT + blockIdx.x;
  const int x = L & 7, p = L >> 3, q = p / NT;
  item = ((q >> run_log2) << (run_log2 + 3)) + (x << run_log2) + (q & ((1 << run_log2) - 1));
  tile = p - q * NT;
}

__device__ __forceinline__ void item_of(const int32_t* __restrict__ items, int it, int& e, int& row0, int& rows) {
  e = items[2 * it];
  const int rp = items[2 * it + 1];
  row0 = rp & 0xFFFFFF;
  rows = rp >> 24;
}

// ---------------------------------------------------------------------------
// Weight staging. A chunk of kc groups of T adjacent column tiles is copied
// from the bank straight into LDS (global_load_lds_dwordx4: 16 bytes per
// lane, lane i at the wave's LDS base + 16 i), the records through registers
// as dwords. In the bank a tile holds, for each j = column % 4, a run of 4G
// units ordered (group, quad); the chunk is the units of groups
// [g0, g0 + kc) of each run and the records of those groups, which are
// contiguous. In LDS the runs are padded to a stride of 16 (mod 64) dwords,
// so the 64 lanes of an operand read (column c = 4 quad + j, dword kb) hit
// 64 different banks.
// ---------------------------------------------------------------------------
constexpr int run_stride(int kc) { return 16 * kc + ((16 - 16 * kc) % 64 + 64) % 64; }

// A record piece of a chunk: bank offset src and LDS offset dst. Pieces are
// numbered against the full chunk size KC (compile-time divisors); a shorter
// last chunk leaves the pieces past kc groups off.
struct Piece {
  bool on;
  uint64_t src;
  int dst;
};

// Record piece p: 4 consecutive records (12 or 16 bytes, 4-byte aligned) of
// tile tt, stored in LDS as 4 dwords (a 3-byte record becomes its 4-byte
// form), so that an operand read takes one aligned dword.
template <int RB, int KC>
__device__ __forceinline__ Piece record_piece(int p, int T, int G, int g0, int kc, int tile_rb) {
  constexpr int kPerTile = 4 * KC;  // record quads of a full chunk
  const int tt = p / kPerTile, rem = p - tt * kPerTile;
  Piece r;
  r.on = tt < T && rem < 4 * kc;
  r.src = (uint64_t)tt * 16 * G * RB + (16 * g0 + 4 * rem) * RB;
  r.dst = tt * tile_rb + 16 * rem;
  return r;
}

template <int RB>
__device__ __forceinline__ uint4 load_records4(const uint8_t* __restrict__ base, const Piece& pc) {
  if (!pc.on) return make_uint4(0, 0, 0, 0);
  if constexpr (RB == 4) {
    return *reinterpret_cast<const uint4*>(base + pc.src);
  } else {
    typedef uint32_t u32x3 __attribute__((ext_vector_type(3), aligned(4)));
    const u32x3 d = *reinterpret_cast<const u32x3*>(base + pc.src);
    return make_uint4(d.x & 0xFFFFFFu, (d.x >> 24) | ((d.y & 0xFFFFu) << 8), (d.y >> 16) | ((d.z & 0xFFu) << 16),
                      d.z >> 8);
  }
}

// Operand of lane (column c = 4 quad + j, block kb) for chunk-local group gl.
template <int RB>
__device__ __forceinline__ void lds_operand(const uint32_t* __restrict__ wl, const uint8_t* __restrict__ rl, int rs,
                                            int gl, int quad, int j, int kb, uint32_t m1024, h8_t& b, float& s) {
  const uint32_t w = wl[j * rs + (4 * gl + quad) * 4 + kb];
  const uint32_t r = reinterpret_cast<const uint32_t*>(rl)[16 * gl + 4 * quad + j];
  s = (float)__builtin_bit_cast(_Float16, (uint16_t)(r & 0xFFFFu));
  b = qz_operand(w, (r >> 16) & 0xFFu, m1024);
}

// ---------------------------------------------------------------------------
// W13 + SwiGLU: grid (2I/16 column tiles, work items), 4 waves. The tile is
// staged in chunks of up to 80 groups (all of K at hidden 2560): the weight
// runs go straight from the bank into LDS (global_load_lds_dwordx4, lane i
// of a load at LDS base + 16 i; wave j copies run j), the records through
// registers as dwords, and the workgroup waits once per chunk. Within a
// chunk wave w takes the groups gl = w, w + 4, ... in batches (5 groups for
// items of up to 16 rows, 2 for two-tile items):
// a batch's activation loads are issued together (unconditionally, from
// clamped groups) and then consumed, so a wave waits once per batch while
// few registers stay live. Groups past the chunk get a zero scale. At the
// end the waves' partial tiles are summed in LDS in wave order. Gate and up
// of intermediate i are columns 2i and 2i + 1, i.e. neighbouring lanes.
// ---------------------------------------------------------------------------
constexpr int kW13Chunk = 80;
constexpr int kW13PerWave = kW13Chunk / 4;
// Groups per batch of activation loads (one memory round trip per batch);
// a single-tile item needs half the registers per group. The LDS of a
// workgroup already limits a SIMD to 6 waves, so up to ~85 VGPRs are free
// (5 and 2: 78 VGPRs; 5 and 4 measured no better, 10 and 5 take 125).
constexpr int w13_batch(int nrt) { return nrt == 2 ? 2 : 5; }
constexpr int kW13WlDw = 4 * run_stride(kW13Chunk);
constexpr int kW13RecPieces = (4 * kW13Chunk + 255) / 256;  // record quads per thread
static_assert(kW13PerWave % w13_batch(1) == 0 && kW13PerWave % w13_batch(2) == 0, "batches tile the wave's groups");
static_assert(kW13RecPieces <= 2, "record staging capacity");
static_assert(kW13WlDw >= 4 * 2 * 64 * 4, "the partial tiles reuse the weight buffer");

typedef __attribute__((address_space(3))) void lds_void_t;
typedef __attribute__((address_space(1))) const void glb_void_t;

// 16 bytes per lane from global memory straight into LDS, lane i at
// lds_base + 16 i (lds_base is the same for the whole wave).
__device__ __forceinline__ void lds_direct16(const uint8_t* src, uint32_t* lds_base) {
  __builtin_amdgcn_global_load_lds((glb_void_t*)src, (lds_void_t*)lds_base, 16, 0, 0);
}

template <int RB, int NRT>
__device__ __forceinline__ void w13_chunk(const uint32_t* wl, const uint8_t* rl, const uint16_t* __restrict__ xr0,
                                          const uint16_t* __restrict__ xr1, int g0, int kc, int wave, int quad,
                                          int j, int kb, uint32_t m1024, f4_t& acc0, f4_t& acc1) {
  constexpr int rs = run_stride(kW13Chunk);
  constexpr int kB = w13_batch(NRT);
#pragma unroll 1
  for (int i0 = 0; i0 < kW13PerWave; i0 += kB) {
    h8_t a0[kB], a1[kB];
#pragma unroll
    for (int u = 0; u < kB; ++u) {
      const int g = g0 + min(wave + 4 * (i0 + u), kc - 1);
      a0[u] = *reinterpret_cast<const h8_t*>(xr0 + 32 * g + 8 * kb);
      if constexpr (NRT == 2) a1[u] = *reinterpret_cast<const h8_t*>(xr1 + 32 * g + 8 * kb);
    }
#pragma unroll
    for (int u = 0; u < kB; ++u) {
      const int gl = wave + 4 * (i0 + u);
      h8_t b;
      float sc;
      lds_operand<RB>(wl, rl, rs, min(gl, kW13Chunk - 1), quad, j, kb, m1024, b, sc);
      sc = gl < kc ? sc : 0.f;  // past the chunk: stale LDS, finite operand, zero weight
      scale_add(acc0, sc, mfma16(a0[u], b));
      if constexpr (NRT == 2) scale_add(acc1, sc, mfma16(a1[u], b));
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
                                                          int topk, uint16_t* __restrict__ act, int run_log2) {
  // staged weights, then (after the last chunk) the waves' partial tiles
  __shared__ __attribute__((aligned(16))) uint32_t wl[kW13WlDw];
  __shared__ __attribute__((aligned(16))) uint8_t rl[16 * kW13Chunk * 4];  // records as dwords
  int it, nt;
  xcd_item_tile(run_log2, it, nt);
  if (it >= *num_items) return;
  int e, row0, rows;
  item_of(items, it, e, row0, rows);
  const int G = H >> 5;
  const uint32_t m1024 = magic1024();
  const int lane = threadIdx.x & 63, wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int c = lane & 15, kb = lane >> 4, quad = c >> 2, j = c & 3;
  const uint8_t* blk = bank + (uint64_t)e * expert_bytes;
  const uint8_t* units = blk + units_off + (uint64_t)nt * 256 * G;
  const uint8_t* recs = blk + meta_off + (uint64_t)nt * 16 * G * RB;
  const int nrt = rows > 16 ? 2 : 1;
  const uint16_t* xr0 = x + (uint64_t)(row_slot[row0 + min(c, rows - 1)] / topk) * H;
  const uint16_t* xr1 = x + (uint64_t)(row_slot[row0 + min(16 + c, rows - 1)] / topk) * H;
  f4_t acc0 = {0.f, 0.f, 0.f, 0.f}, acc1 = {0.f, 0.f, 0.f, 0.f};
  constexpr int rs = run_stride(kW13Chunk);
  for (int g0 = 0; g0 < G; g0 += kW13Chunk) {
    const int kc = min(kW13Chunk, G - g0);
    if (g0 > 0) __syncthreads();  // the previous chunk's LDS reads are done
    {
      // run j = wave: 4 kc units of 16 bytes, 64 per load
      const uint8_t* src = units + (uint64_t)wave * 64 * G + 64 * g0;
      uint32_t* dst = wl + wave * rs;
      for (int i = 0; 64 * i < 4 * kc; ++i) {
        const int u = 64 * i + lane;
        if (u < 4 * kc) lds_direct16(src + 16 * u, dst + 256 * i);
      }
    }
    // records: every load is issued (a piece past the chunk rereads the run's
    // first quad) before any is converted to dwords
    typedef uint32_t u32x3 __attribute__((ext_vector_type(3), aligned(4)));
    u32x3 rv[kW13RecPieces];
    int rd[kW13RecPieces];
#pragma unroll
    for (int q = 0; q < kW13RecPieces; ++q) {
      const Piece pc = record_piece<RB, kW13Chunk>((int)threadIdx.x + 256 * q, 1, G, g0, kc, 0);
      rv[q] = *reinterpret_cast<const u32x3*>(recs + (pc.on ? pc.src : 0));
      rd[q] = pc.on ? pc.dst : -1;
    }
    uint32_t rw[kW13RecPieces];  // the fourth dword of a 4-byte record quad
    if constexpr (RB == 4) {
#pragma unroll
      for (int q = 0; q < kW13RecPieces; ++q) {
        const Piece pc = record_piece<RB, kW13Chunk>((int)threadIdx.x + 256 * q, 1, G, g0, kc, 0);
        rw[q] = *reinterpret_cast<const uint32_t*>(recs + (pc.on ? pc.src : 0) + 12);
      }
    }
#pragma unroll
    for (int q = 0; q < kW13RecPieces; ++q) {
      if (rd[q] < 0) continue;
      const u32x3 d = rv[q];
      uint4 v;
      if constexpr (RB == 4) {
        v = make_uint4(d.x, d.y, d.z, rw[q]);
      } else {
        v = make_uint4(d.x & 0xFFFFFFu, (d.x >> 24) | ((d.y & 0xFFFFu) << 8), (d.y >> 16) | ((d.z & 0xFFu) << 16),
                       d.z >> 8);
      }
      *reinterpret_cast<uint4*>(rl + rd[q]) = v;
    }
    // the barrier waits for every load of the workgroup, the LDS-direct ones included
    __syncthreads();
    if (nrt == 2)
      w13_chunk<RB, 2>(wl, rl, xr0, xr1, g0, kc, wave, quad, j, kb, m1024, acc0, acc1);
    else
      w13_chunk<RB, 1>(wl, rl, xr0, xr1, g0, kc, wave, quad, j, kb, m1024, acc0, acc1);
  }
  f4_t* red = reinterpret_cast<f4_t*>(wl);  // [wave][rt][lane]
  __syncthreads();                          // every wave is done with the staged weights
  red[(2 * wave + 0) * 64 + lane] = acc0;
  red[(2 * wave + 1) * 64 + lane] = acc1;
  __syncthreads();
  if (wave != 0) return;
  for (int rt = 0; rt < nrt; ++rt) {
    const f4_t d = red[rt * 64 + lane] + red[(2 + rt) * 64 + lane] + red[(4 + rt) * 64 + lane] +
                   red[(6 + rt) * 64 + lane];
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

// Calls of up to kDecodeFormMaxTokens tokens and kDecodeFormMaxSlots slots
// run the decode kernels (per slot and tile, per token and tile: no routing,
// no row results; M = 9: 39.4 -> 19.2 us per call, 16: 45.5 -> 24.4, 32: 60.4
// -> 38.9, 48: 73.0 -> 51.8, 64: 82.4 -> 66.3 against the per-tile kernels).
// From kWideMinTokens the wide kernels (items of up to 64 rows, 20 column
// tiles per workgroup; both products in one launch at inter <= 160: M = 96
// 89.6 against 95.7 per-tile and 96.0 in the decode form; M = 128 90.2
// against 108.1 per-tile). Between (more slots), the per-tile kernels above.
constexpr int kDecodeFormMaxTokens = 64, kDecodeFormMaxSlots = 1024;
constexpr int kWideMinTokens = kDecodeFormMaxTokens + 1;
// Slots from which W2 takes the wide items (below: the 32-row items, where
// experts have few rows: M = 1024, 154.8 against 160.1 us per call; M =
// 4096, 404.8 against 399.0).
constexpr int kW2WideItemsFrom = 16384;

// ---------------------------------------------------------------------------
// Both products for calls with many rows per expert ("wide" kernels): work
// items of up to 64 rows of one expert (wide items), grid (ceil(NT / (4 CT))
// blocks of 4 CT column tiles, wide items), 4 waves. Wave w owns the CT
// consecutive tiles CT w .. CT w + CT - 1 of its block over all of K and all
// RT 16-row tiles of the item, so one (q - z) operand feeds RT matrix-core
// products and the item's rows, staged in LDS, serve all 4 CT tiles.
//   W13: A = the item's token rows of x (gathered), K = hidden, N = 2 inter,
//        SwiGLU into act (fp16, by row), chunks of 4 groups, CT = 5;
//   W2:  A = the item's rows of act, K = inter, N = hidden, fp32 row
//        results y (by row), chunks of 5 groups (all of K at inter 160),
//        CT = 5.
//
// Data flow per chunk of CG groups: the item's A units (16 bytes each,
// [group][k block][row] in LDS so that an operand read is 1 KB contiguous;
// the row is XOR-swizzled inside its 16-row tile with (4 group + k block) so
// that the staging writes spread over the banks) and the block's records are
// requested one chunk ahead into registers and written to LDS at the chunk
// boundary, the records decoded once there into {fp32 scale (zero for a
// group past K), the two packed fp16 offsets the operand subtracts}. The
// weights take one of two ways (wx_ring):
//   * LDS (W2): the block's weights of the chunk go the same way as A, 16
//     bytes per lane, so a load covers contiguous runs of 64 CG bytes; each
//     lane then reads its operand dword (dword kb of column c's unit) from
//     LDS;
//   * register ring (W13): each lane requests its operand dwords of its
//     wave's tiles straight into registers CG groups ahead of their use.
// Loads are unconditional, their addresses clamped into K, into the block's
// tiles and into the item's rows; a group past K meets a zero scale.
// Addresses are a uniform base (scalar registers) plus a 32-bit lane offset,
// so the loads take the scalar-base form.
// ---------------------------------------------------------------------------
constexpr int kWxRows = 64;                 // A rows of an LDS chunk (room for 4 row tiles)
constexpr int kWxRT = kWideRows / 16;       // 16-row tiles of the largest wide item
// column tiles per wave: W13 5; W2 5 over wide items, 4 over 32-row items
// (a register budget for three workgroups per CU)
constexpr int kWxCT13 = 5, kWxCT2 = 5, kWxCT2Narrow = 4;
constexpr int wx_ct(int stage, int rtmax) { return stage == 0 ? kWxCT13 : rtmax <= 2 ? kWxCT2Narrow : kWxCT2; }
constexpr int kWxCG13 = 4, kWxCG2 = 5;      // groups per chunk of the two stages
// LDS dwords of a stage's A chunk, decoded records of a chunk and weights of a chunk
constexpr int wx_a_dw(int cg) { return cg * 4 * kWxRows * 4; }
constexpr int wx_r_dw(int ct, int cg) { return 4 * ct * cg * 16 * 2; }
// weight runs in LDS: a run of a chunk is 16 CG dwords, padded to a stride of
// 16 or 48 (mod 64) dwords so that the 64 lanes of an operand read (column
// c = 4 quad + j, dword kb) hit 64 different banks
constexpr int wx_run_stride(int cg) { return 16 * cg + ((16 - 16 * cg) % 64 + 64) % 64; }
constexpr int wx_b_dw(int ct, int cg) { return 4 * ct * 4 * wx_run_stride(cg); }
static_assert(kWideRows % 16 == 0 && kWxRT >= 1 && kWxRT <= 4, "wide items of 1 to 4 row tiles");
enum WideStage { kWideW13 = 0, kWideW2 = 1 };
// Where a stage's weights go: W13 keeps a register ring per wave (each lane's
// operand dwords requested CG groups ahead; measured faster than LDS staging
// at 4096 tokens, equal at 1024), W2 stages them in LDS (its K is short, so
// the whole chunk is requested at once in contiguous runs; measured faster).
constexpr bool wx_ring(int stage) { return stage == 0; }
// The ring's two forms: per group, each lane requests its operand dword (four
// 64-byte pieces per request) as soon as the group before is used; per chunk,
// each lane requests a whole 16-byte unit (256 contiguous bytes per run) and
// a transpose across the wave's lane rows rebuilds the operands. Items of up
// to two row tiles are load-bound and take the second (W13 at M = 256: 59.8
// -> 48.8 us, M = 512: 62.9 -> 56.6 us); with more row tiles the extra moves
// and swaps cost more than the longer runs save (M = 4096: 145 -> 155 us).
constexpr bool wx_ring_units(int stage, int rt) { return wx_ring(stage) && rt <= 2; }

// f(std::integral_constant<int, i>) for i = 0 .. N - 1, each a separate
// instantiation, so that indices derived from i are compile-time constants.
template <int N, int I = 0, class F>
__device__ __forceinline__ void static_for(F&& f) {
  if constexpr (I < N) {
    f(std::integral_constant<int, I>{});
    static_for<N, I + 1>(f);
  }
}

// Keeps the memory requests above where they are: neither the IR passes
// (the empty asm is a compiler memory barrier) nor the machine scheduler
// (sched_barrier) move them past this point towards their first use. The
// pointers of the kernels that rely on it carry no __restrict__: a load
// through a no-alias pointer may legally cross the compiler barrier.
__device__ __forceinline__ void issue_here() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_sched_barrier(0);
}

__device__ __forceinline__ uint32_t magic64() {
  uint32_t m;
  asm volatile("v_mov_b32 %0, 0x54005400" : "=v"(m));
  return m;
}

// Eight (q - z) values in fp16 from one dword of a unit (value p at bits
// 4*(p/2) + 16*(p%2)). The nibbles at bits 0..3 of a half OR-ed into the
// mantissa of 1024.0 give 1024 + q; those at bits 4..7 OR-ed into the
// mantissa of 64.0 (whose last mantissa bit is worth 1/16) give 64 + q, so
// two of the four pairs need no shift. czz holds -(1024 + z) in its low half
// and -(64 + z) in its high half; every sum is an exact integer.
__device__ __forceinline__ h8_t qz_operand64(uint32_t w, uint32_t czz, uint32_t m1024, uint32_t m64) {
  const h2_t c = as_h2(czz);
  const h2_t c1024 = __builtin_shufflevector(c, c, 0, 0), c64 = __builtin_shufflevector(c, c, 1, 1);
  const uint32_t w8 = w >> 8;
  const h2_t p0 = as_h2((w & 0x000F000Fu) | m1024) + c1024;
  const h2_t p1 = as_h2((w & 0x00F000F0u) | m64) + c64;
  const h2_t p2 = as_h2((w8 & 0x000F000Fu) | m1024) + c1024;
  const h2_t p3 = as_h2((w8 & 0x00F000F0u) | m64) + c64;
  return __builtin_bit_cast(h8_t, make_uint4(__builtin_bit_cast(uint32_t, p0), __builtin_bit_cast(uint32_t, p1),
                                             __builtin_bit_cast(uint32_t, p2), __builtin_bit_cast(uint32_t, p3)));
}

// A decoded record: {the scale in fp32 (0 when not live), czz as above}.
__device__ __forceinline__ uint2 decode_record(uint32_t r, bool live) {
  const float s = (float)__builtin_bit_cast(_Float16, (uint16_t)(r & 0xFFFFu));
  const uint32_t z = (r >> 16) & 0xFFu;
  const _Float16 m64z = (_Float16)(-64.0f - (float)z);  // exact: 64 + z <= 319
  return make_uint2(live ? __builtin_bit_cast(uint32_t, s) : 0u,
                    (0xE400u + z) | ((uint32_t)__builtin_bit_cast(uint16_t, m64z) << 16));
}

// 4 x 4 transpose across the four 16-lane rows of a wave: on entry lane row r
// holds m[r][0..3] in v[0..3], on exit m[0..3][r]. The 32-lane swaps exchange
// rows {2, 3} of v[0], v[1] with rows {0, 1} of v[2], v[3]; the 16-lane swaps
// then exchange the odd rows of v[0], v[2] with the even rows of v[1], v[3].
__device__ __forceinline__ void rows_transpose4(uint32_t (&v)[4]) {
  const auto s02 = __builtin_amdgcn_permlane32_swap(v[0], v[2], false, false);
  const auto s13 = __builtin_amdgcn_permlane32_swap(v[1], v[3], false, false);
  const auto s01 = __builtin_amdgcn_permlane16_swap(s02[0], s13[0], false, false);
  const auto s23 = __builtin_amdgcn_permlane16_swap(s02[1], s13[1], false, false);
  v[0] = s01[0], v[1] = s01[1], v[2] = s23[0], v[3] = s23[1];
}

// The LDS dword offset of unit (16-row tile slot row', group g, k block kb)
// of a staged A chunk of kWxRows rows: [group][k block][row], the row
// XOR-swizzled inside its 16-row tile with (4 g + kb).
__device__ __forceinline__ int wx_a_unit(int g, int kb, int row) {
  return ((g * 4 + kb) * 64 + (row & ~15) + ((row & 15) ^ ((4 * g + kb) & 15))) * 4;
}

// One wide item of one column block. K = 32 G; the A rows are K fp16 long.
// TO_LDS (W13 only): act goes to LDS at `out` in the A layout of a W2 chunk
// (every row of the item's row tiles, padding rows included) instead of to
// global memory. NTW: the whole-unit ring's weight loads are non-temporal.
template <int RB, int RT, int CG, int CT, int STAGE, bool TO_LDS = false, bool NTW = false>
__device__ __forceinline__ void wide_item(const uint8_t* units, const uint8_t* recs, const uint16_t* a_src,
                                          const int32_t* row_slot, int row0, int rows, int topk, int G, int NT,
                                          int nb0, void* out, int out_stride, uint32_t* al, uint32_t* rl,
                                          uint32_t* bl) {
  typedef uint32_t u32x3 __attribute__((ext_vector_type(3), aligned(4)));
  constexpr int kNU = (RT * CG + 3) / 4;           // A units per thread and chunk
  constexpr int kUnits = 16 * RT * CG * 4;         // A units of a chunk
  constexpr int kWxTiles = 4 * CT;                 // column tiles of the block
  constexpr int kQuads = kWxTiles * CG * 4;        // record quads of a chunk
  constexpr int kNQ = (kQuads + 255) / 256;        // record quads per thread and chunk
  const int t = threadIdx.x, lane = t & 63, wave = __builtin_amdgcn_readfirstlane(t >> 6);
  const int c = lane & 15, kb = lane >> 4, quad = c >> 2, j = c & 3;
  const uint32_t m1024 = magic1024(), m64 = magic64();
  const int Tb = min(kWxTiles, NT - nb0);  // tiles of this block
  // A units of this thread: u = t + 256 i is k block u & 3 of group
  // (u >> 2) % CG of row (u >> 2) / CG
  const uint8_t* ab = reinterpret_cast<const uint8_t*>(a_src);
  uint32_t ao[kNU];  // byte offset of the unit's k block in its row
  int agl[kNU], adst[kNU];
#pragma unroll
  for (int i = 0; i < kNU; ++i) {
    const int u = t + 256 * i, gl = (u >> 2) % CG, row = (u >> 2) / CG, akb = u & 3;
    const int r = row0 + min(row, rows - 1);
    const uint32_t arow = STAGE == kWideW13 ? (uint32_t)(row_slot[r] / topk) : (uint32_t)r;
    ao[i] = arow * (uint32_t)G * 64u + 16u * akb;
    agl[i] = gl;
    const int h = (4 * gl + akb) & 15;
    adst[i] = u < kUnits ? ((gl * 4 + akb) * kWxRows + (row & ~15) + ((row & 15) ^ h)) * 4 : -1;
  }
  // record quads of this thread: u = t + 256 q is records 4 (u & 3) .. + 3 of
  // group (u >> 2) % CG of the chunk, tile u / (4 CG) of the block
  uint32_t ro[kNQ];
  int rgl[kNQ], rdst[kNQ];
#pragma unroll
  for (int q = 0; q < kNQ; ++q) {
    const int u = min(t + 256 * q, kQuads - 1);
    ro[q] = (uint32_t)min(u / (4 * CG), Tb - 1) * 16u * G * RB + 4u * (u & 3) * RB;
    rgl[q] = (u >> 2) % CG;
    rdst[q] = t + 256 * q < kQuads ? 8 * u : -1;  // dword offset of its 4 decoded records
  }
  // weight units of this thread: u = t + 256 i is unit u % (4 CG) (group
  // (u % (4 CG)) / 4, quad u % 4) of run (u / (4 CG)) % 4 of tile u / (16 CG)
  constexpr bool RING = wx_ring(STAGE);
  constexpr int kRS = wx_run_stride(CG);
  constexpr int kBU = RING ? 0 : kWxTiles * 4 * 4 * CG;  // weight units of a chunk staged in LDS
  constexpr int kNB = kBU ? (kBU + 255) / 256 : 1;       // weight units per thread and chunk (1 unused with RING)
  uint32_t bo[kNB];
  int bgl[kNB], bdst[kNB];
#pragma unroll
  for (int i = 0; i < kNB; ++i) {
    const int u = min(t + 256 * i, kBU - 1), ur = u % (4 * CG), run = u / (4 * CG);
    const int tt = run >> 2, jr = run & 3;
    bo[i] = (uint32_t)min(tt, Tb - 1) * 256u * G + (uint32_t)jr * 64u * G + 16u * (ur & 3);
    bgl[i] = ur >> 2;
    bdst[i] = t + 256 * i < kBU ? run * kRS + 4 * ur : -1;
  }
  // plain loads: an expert's second item finds its weights in the caches
  // (non-temporal loads measured slower here, while they speed up the
  // reduce's read-once rows)
  auto ld_b = [&](int i, int g0) {
    return *reinterpret_cast<const u32x4_t*>(units + 64 * min(g0 + bgl[i], G - 1) + bo[i]);
  };
  // the register ring (RING), tile CT wave + ct clamped into the block:
  //  * per group (!RU): this lane's operand dword of group g;
  //  * per chunk (RU): lane (c, kb) requests the whole unit of column c,
  //    group g0 + kb (clamped into K), so the 16 lanes of a run j read the
  //    run's 256 contiguous bytes of the chunk; rows_transpose4 then hands
  //    lane (c, kb) dword kb of column c's unit of each of the chunk's groups.
  constexpr bool RU = wx_ring_units(STAGE, RT);
  static_assert(!RU || CG == 4, "the ring's transpose takes chunks of 4 groups");
  const uint32_t bor = (uint32_t)j * 64u * G + 16u * quad + (RU ? 0u : 4u * kb);
  const uint8_t* tbase[CT];
#pragma unroll
  for (int ct = 0; ct < CT; ++ct) tbase[ct] = units + (uint64_t)min(CT * wave + ct, Tb - 1) * 256 * G;
  auto ld_r = [&](int ct, int g) { return *reinterpret_cast<const uint32_t*>(tbase[ct] + 64 * min(g, G - 1) + bor); };
  auto ld_ru = [&](int ct, int g0) {  // group min(g0 + kb, G - 1) as a uniform part plus a lane part
    const int gu = min(g0, G - 1);
    const uint32_t lo = 64u * (uint32_t)min(kb, G - 1 - gu) + bor;
    return load16<NTW>(tbase[ct] + 64 * gu + lo);
  };
  auto ld_a = [&](int i, int g0) { return *reinterpret_cast<const u32x4_t*>(ab + 64 * min(g0 + agl[i], G - 1) + ao[i]); };
  auto rsrc = [&](int q, int g0) { return recs + 16 * RB * min(g0 + rgl[q], G - 1) + ro[q]; };
  u32x4_t av[kNU], bv[kNB];
  u32x3 rv[kNQ];
  uint32_t rw[kNQ];  // the fourth record of a 4-byte quad
  auto load_chunk = [&](int g0) {
#pragma unroll
    for (int i = 0; i < kNB; ++i)
      if constexpr (!RING) bv[i] = ld_b(i, g0);
#pragma unroll
    for (int i = 0; i < kNU; ++i) av[i] = ld_a(i, g0);
#pragma unroll
    for (int q = 0; q < kNQ; ++q) {
      const uint8_t* src = rsrc(q, g0);
      rv[q] = *reinterpret_cast<const u32x3*>(src);
      if constexpr (RB == 4) rw[q] = *reinterpret_cast<const uint32_t*>(src + 12);
    }
  };
  load_chunk(0);
  // chunk requests before ring requests, in the same order as in the loop,
  // so that the wait for the chunk's A and records leaves the ring in flight
  uint32_t bq[RING && !RU ? CG : 1][CT];  // per group: [group of the chunk][tile]
  u32x4_t braw[RU ? CT : 1];              // per chunk: the next chunk's units
  if constexpr (RING && !RU) {
    issue_here();
#pragma unroll
    for (int g = 0; g < CG; ++g) {
#pragma unroll
      for (int ct = 0; ct < CT; ++ct) bq[g][ct] = ld_r(ct, g);
      issue_here();
    }
  }
  if constexpr (RU) {
    issue_here();
#pragma unroll
    for (int ct = 0; ct < CT; ++ct) braw[ct] = ld_ru(ct, 0);
    issue_here();
  }
  f4_t acc[CT][RT];
#pragma unroll
  for (int ct = 0; ct < CT; ++ct)
#pragma unroll
    for (int rt = 0; rt < RT; ++rt) acc[ct][rt] = f4_t{0.f, 0.f, 0.f, 0.f};
  for (int g0 = 0; g0 < G; g0 += CG) {
    if (g0 > 0) __syncthreads();  // every wave is done with the previous chunk's LDS
#pragma unroll
    for (int i = 0; i < kNB; ++i)
      if (!RING && bdst[i] >= 0) *reinterpret_cast<u32x4_t*>(bl + bdst[i]) = bv[i];
#pragma unroll
    for (int i = 0; i < kNU; ++i)
      if (adst[i] >= 0) *reinterpret_cast<u32x4_t*>(al + adst[i]) = av[i];
#pragma unroll
    for (int q = 0; q < kNQ; ++q) {
      if (rdst[q] < 0) continue;
      const u32x3 d = rv[q];
      uint32_t r4[4];
      if constexpr (RB == 4) {
        r4[0] = d.x, r4[1] = d.y, r4[2] = d.z, r4[3] = rw[q];
      } else {
        r4[0] = d.x, r4[1] = (d.x >> 24) | (d.y << 8), r4[2] = (d.y >> 16) | (d.z << 16), r4[3] = d.z >> 8;
      }
      const bool live = g0 + rgl[q] < G;
      const uint2 d0 = decode_record(r4[0], live), d1 = decode_record(r4[1], live);
      const uint2 d2 = decode_record(r4[2], live), d3 = decode_record(r4[3], live);
      const u32x4_t lo = {d0.x, d0.y, d1.x, d1.y}, hi = {d2.x, d2.y, d3.x, d3.y};
      *reinterpret_cast<u32x4_t*>(rl + rdst[q]) = lo;
      *reinterpret_cast<u32x4_t*>(rl + rdst[q] + 4) = hi;
    }
    __syncthreads();
    // RU: this chunk's units, transposed into bt[tile][group of the chunk]
    // where a tile is first used, so that each waits only for its own load
    u32x4_t bcur[RU ? CT : 1];
    uint32_t bt[RU ? CT : 1][4];
    if constexpr (RU) {
#pragma unroll
      for (int ct = 0; ct < CT; ++ct) bcur[ct] = braw[ct];
    }
    load_chunk(g0 + CG);  // the next chunk (clamped past K: loaded, never used)
    if constexpr (RU) {
#pragma unroll
      for (int ct = 0; ct < CT; ++ct) braw[ct] = ld_ru(ct, g0 + CG);
    }
    issue_here();
#pragma unroll
    for (int gl = 0; gl < CG; ++gl) {
      const int cs = c ^ ((4 * gl + kb) & 15);  // the swizzled row of lane c in its tile
      h8_t a[RT];
#pragma unroll
      for (int rt = 0; rt < RT; ++rt)
        a[rt] = *reinterpret_cast<const h8_t*>(al + ((gl * 4 + kb) * kWxRows + 16 * rt + cs) * 4);
#pragma unroll
      for (int ct = 0; ct < CT; ++ct) {
        if constexpr (RU) {
          if (gl == 0) {
            bt[ct][0] = bcur[ct].x, bt[ct][1] = bcur[ct].y, bt[ct][2] = bcur[ct].z, bt[ct][3] = bcur[ct].w;
            rows_transpose4(bt[ct]);
          }
        }
        const int tb = min(CT * wave + ct, Tb - 1);
        const uint2 sc = *reinterpret_cast<const uint2*>(rl + ((tb * CG + gl) * 16 + c) * 2);
        const uint32_t wq = RU     ? bt[RU ? ct : 0][gl]
                            : RING ? bq[RING ? gl : 0][ct]
                                   : bl[(tb * 4 + j) * kRS + (4 * gl + quad) * 4 + kb];
        const h8_t b = qz_operand64(wq, sc.y, m1024, m64);
        const float s = __builtin_bit_cast(float, sc.x);
#pragma unroll
        for (int rt = 0; rt < RT; ++rt) scale_add(acc[ct][rt], s, mfma16(a[rt], b));
      }
      if constexpr (RING && !RU) {
#pragma unroll
        for (int ct = 0; ct < CT; ++ct) bq[gl][ct] = ld_r(ct, g0 + gl + CG);
        issue_here();  // the same for the weight ring
      }
    }
  }
#pragma unroll
  for (int ct = 0; ct < CT; ++ct) {
    const int tb = CT * wave + ct;
    if (tb >= Tb) break;
    const int nt = nb0 + tb;
#pragma unroll
    for (int rt = 0; rt < RT; ++rt) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float d = acc[ct][rt][i];
        const int row = 16 * rt + 4 * kb + i;
        if constexpr (STAGE == kWideW13 && TO_LDS) {
          const float up = dpp<kQuadSwap1>(d);  // column c ^ 1
          if (!(c & 1)) {
            const float a = d / (1.0f + __expf(-d)) * up;
            const int ac = nt * 8 + (c >> 1);  // act column: group ac / 32, k block (ac / 8) % 4
            static_cast<uint16_t*>(out)[2 * wx_a_unit(ac >> 5, (ac >> 3) & 3, row) + (ac & 7)] =
                __builtin_bit_cast(uint16_t, (_Float16)a);
          }
        } else if constexpr (STAGE == kWideW13) {
          const float up = dpp<kQuadSwap1>(d);  // column c ^ 1
          if (!(c & 1) && row < rows) {
            const float a = d / (1.0f + __expf(-d)) * up;
            static_cast<uint16_t*>(out)[(uint64_t)(row0 + row) * out_stride + nt * 8 + (c >> 1)] =
                __builtin_bit_cast(uint16_t, (_Float16)a);
          }
        } else {
          if (row < rows) static_cast<float*>(out)[(uint64_t)(row0 + row) * out_stride + nt * 16 + c] = d;
        }
      }
    }
  }
}

// STAGE kWideW13: a = x, out = act (stride inter); kWideW2: a = act, out = y
// (stride hidden).
template <int RB, int STAGE, int RTMAX>
__global__ __launch_bounds__(256, RTMAX <= 2 ? 3 : 2) void prefill_wide_kernel(const int32_t* items, const int32_t* num_items,
                                                              const int32_t* row_slot, const uint8_t* bank,
                                                              const uint16_t* a, uint64_t expert_bytes,
                                                              uint64_t units_off, uint64_t meta_off, int H, int I,
                                                              int topk, void* out, int run_log2) {
  constexpr int CG = STAGE == kWideW13 ? kWxCG13 : kWxCG2;
  constexpr int CT = wx_ct(STAGE, RTMAX);
  __shared__ __attribute__((aligned(16))) uint32_t al[wx_a_dw(CG)];
  __shared__ __attribute__((aligned(16))) uint32_t rl[wx_r_dw(CT, CG)];
  __shared__ __attribute__((aligned(16))) uint32_t bl[wx_ring(STAGE) ? 4 : wx_b_dw(CT, CG)];
  constexpr int kWxTiles = 4 * CT;
  int it, bx;
  xcd_item_tile(run_log2, it, bx);
  if (it >= *num_items) return;
  int e, row0, rows;
  item_of(items, it, e, row0, rows);
  const int G = (STAGE == kWideW13 ? H : I) >> 5, NT = (STAGE == kWideW13 ? 2 * I : H) >> 4;
  const int nb0 = kWxTiles * bx, out_stride = STAGE == kWideW13 ? I : H;
  const uint8_t* blk = bank + (uint64_t)e * expert_bytes;
  const uint8_t* units = blk + units_off + (uint64_t)nb0 * 256 * G;
  const uint8_t* recs = blk + meta_off + (uint64_t)nb0 * 16 * G * RB;
  const int rt = (rows + 15) >> 4;  // 1 .. RTMAX
  static_for<RTMAX>([&](auto i_c) {
    constexpr int RT = decltype(i_c)::value + 1;
    if (rt == RT)
      wide_item<RB, RT, CG, CT, STAGE>(units, recs, a, row_slot, row0, rows, topk, G, NT, nb0, out, out_stride, al,
                                       rl, bl);
  });
}

// ---------------------------------------------------------------------------
// Both products of one wide item in one workgroup (inter <= 160, so that the
// item's act rows, all of W2's K, fit one LDS chunk and W13's 2 inter / 16
// column tiles one block of 20): W13 + SwiGLU as in prefill_wide_kernel with
// act written to LDS in the A layout of a W2 chunk, then W2 over every block
// of 20 column tiles with that A resident. The next block's weights and
// records are requested before the current block computes. One launch less
// than the two wide kernels, and no act round trip through global memory;
// the arithmetic and its order are the same, so the results are too.
// ---------------------------------------------------------------------------
constexpr int kFusedMaxInter = 32 * kWxCG2;  // 160

template <int RB, int RT, int CT, bool NTW>
__device__ __forceinline__ void w2_resident(const uint8_t* units, const uint8_t* recs, const uint32_t* al, int G,
                                            int NT, int row0, int rows, float* y, int H, uint32_t* rl,
                                            uint32_t* bl) {
  typedef uint32_t u32x3 __attribute__((ext_vector_type(3), aligned(4)));
  constexpr int CG = kWxCG2;                       // all of K (G <= CG) in the one chunk
  constexpr int kWxTiles = 4 * CT;                 // column tiles of a block
  constexpr int kQuads = kWxTiles * CG * 4;        // record quads of a block
  constexpr int kNQ = (kQuads + 255) / 256;
  constexpr int kRS = wx_run_stride(CG);
  constexpr int kBU = kWxTiles * 4 * 4 * CG;       // weight units of a block
  constexpr int kNB = (kBU + 255) / 256;
  // an opaque copy of the thread index, so that this phase's per-thread
  // offsets are computed here and do not stay live through the phase before
  int t;
  asm volatile("v_mov_b32 %0, %1" : "=v"(t) : "v"((int)threadIdx.x));
  const int lane = t & 63, wave = __builtin_amdgcn_readfirstlane(t >> 6);
  const int c = lane & 15, kb = lane >> 4, quad = c >> 2, j = c & 3;
  const uint32_t m1024 = magic1024(), m64 = magic64();
  const int nblk = (NT + kWxTiles - 1) / kWxTiles;
  // this thread's weight units and record quads of a block, as in wide_item:
  // the tile within the block and the offset inside the tile (group clamped
  // into K); a block's requests are its uniform base plus 32-bit lane offsets
  uint32_t bo[kNB];
  int btl[kNB], bdst[kNB];
#pragma unroll
  for (int i = 0; i < kNB; ++i) {
    const int u = min(t + 256 * i, kBU - 1), ur = u % (4 * CG), run = u / (4 * CG);
    btl[i] = run >> 2;
    bo[i] = (uint32_t)(run & 3) * 64u * G + 16u * (ur & 3) + 64u * (uint32_t)min(ur >> 2, G - 1);
    bdst[i] = t + 256 * i < kBU ? run * kRS + 4 * ur : -1;
  }
  uint32_t ro[kNQ];
  int rtl[kNQ], rgl[kNQ], rdst[kNQ];
#pragma unroll
  for (int q = 0; q < kNQ; ++q) {
    const int u = min(t + 256 * q, kQuads - 1);
    rtl[q] = u / (4 * CG);
    rgl[q] = (u >> 2) % CG;
    ro[q] = 4u * (u & 3) * RB + 16u * RB * (uint32_t)min(rgl[q], G - 1);
    rdst[q] = t + 256 * q < kQuads ? 8 * u : -1;
  }
  u32x4_t bv[kNB];
  u32x3 rv[kNQ];
  uint32_t rw[kNQ];
  const uint32_t tile_b = 256u * G, tile_r = 16u * G * RB;  // bytes of a tile's weights and records
  auto load_block = [&](int b) {  // clamped into the blocks, the block's tiles and K
    const int nb0 = kWxTiles * min(b, nblk - 1), Tb = min(kWxTiles, NT - nb0);
    const uint8_t* ub = units + (uint64_t)nb0 * tile_b;
    const uint8_t* rb = recs + (uint64_t)nb0 * tile_r;
#pragma unroll
    for (int i = 0; i < kNB; ++i)
      bv[i] = load16<NTW>(ub + ((uint32_t)min(btl[i], Tb - 1) * tile_b + bo[i]));
#pragma unroll
    for (int q = 0; q < kNQ; ++q) {
      const uint8_t* src = rb + ((uint32_t)min(rtl[q], Tb - 1) * tile_r + ro[q]);
      rv[q] = *reinterpret_cast<const u32x3*>(src);
      if constexpr (RB == 4) rw[q] = *reinterpret_cast<const uint32_t*>(src + 12);
    }
  };
  load_block(0);
#pragma unroll 1
  for (int b = 0; b < nblk; ++b) {
    const int nb0 = kWxTiles * b, Tb = min(kWxTiles, NT - nb0);
    if (b > 0) __syncthreads();  // every wave is done with the previous block's LDS
#pragma unroll
    for (int i = 0; i < kNB; ++i)
      if (bdst[i] >= 0) *reinterpret_cast<u32x4_t*>(bl + bdst[i]) = bv[i];
#pragma unroll
    for (int q = 0; q < kNQ; ++q) {
      if (rdst[q] < 0) continue;
      const u32x3 dr = rv[q];
      uint32_t r4[4];
      if constexpr (RB == 4) {
        r4[0] = dr.x, r4[1] = dr.y, r4[2] = dr.z, r4[3] = rw[q];
      } else {
        r4[0] = dr.x, r4[1] = (dr.x >> 24) | (dr.y << 8), r4[2] = (dr.y >> 16) | (dr.z << 16), r4[3] = dr.z >> 8;
      }
      const bool live = rgl[q] < G;
      const uint2 d0 = decode_record(r4[0], live), d1 = decode_record(r4[1], live);
      const uint2 d2 = decode_record(r4[2], live), d3 = decode_record(r4[3], live);
      const u32x4_t lo = {d0.x, d0.y, d1.x, d1.y}, hi = {d2.x, d2.y, d3.x, d3.y};
      *reinterpret_cast<u32x4_t*>(rl + rdst[q]) = lo;
      *reinterpret_cast<u32x4_t*>(rl + rdst[q] + 4) = hi;
    }
    __syncthreads();
    load_block(b + 1);  // the next block (past the last: the last again, never used)
    issue_here();
    f4_t acc[CT][RT];
#pragma unroll
    for (int ct = 0; ct < CT; ++ct)
#pragma unroll
      for (int rt = 0; rt < RT; ++rt) acc[ct][rt] = f4_t{0.f, 0.f, 0.f, 0.f};
    // Compile-time LDS offsets throughout: the act groups past K hold zeros,
    // and the staged tile slots past the block's last hold copies of it.
#pragma unroll
    for (int gl = 0; gl < CG; ++gl) {
      h8_t a[RT];  // the item's act rows (resident)
#pragma unroll
      for (int rt = 0; rt < RT; ++rt)
        a[rt] = *reinterpret_cast<const h8_t*>(al + wx_a_unit(gl, kb, 16 * rt + c));
#pragma unroll
      for (int ct = 0; ct < CT; ++ct) {
        const int tb = CT * wave + ct;
        const uint2 sc = *reinterpret_cast<const uint2*>(rl + ((tb * CG + gl) * 16 + c) * 2);
        const h8_t bq = qz_operand64(bl[(tb * 4 + j) * kRS + (4 * gl + quad) * 4 + kb], sc.y, m1024, m64);
        const float sf = __builtin_bit_cast(float, sc.x);
#pragma unroll
        for (int rt = 0; rt < RT; ++rt) {
          scale_add(acc[ct][rt], sf, mfma16(a[rt], bq));
          // the sum is formed here: left alone, the compiler sinks every
          // scale-add to the stores and keeps all the groups' products live
          asm volatile("" : "+v"(acc[ct][rt]));
        }
      }
    }
    // A wave's tiles past the block's last are clamped to it, as in the
    // products: those waves store the same values to the same place again,
    // which keeps the stores out of branches (and the registers unspilled).
    // Each store: a uniform base (row 16 rt + i of the item, the wave's tile)
    // plus the lane's fixed offset (its rows 4 kb on, column c).
    const uint32_t lane_off = (uint32_t)(4 * kb * H + c);
#pragma unroll
    for (int ct = 0; ct < CT; ++ct) {
      const int tb = min(CT * wave + ct, Tb - 1);
#pragma unroll
      for (int rt = 0; rt < RT; ++rt)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          float* yb = y + ((uint64_t)(row0 + 16 * rt + i) * H + (nb0 + tb) * 16);
          if (16 * rt + 4 * kb + i < rows) yb[lane_off] = acc[ct][rt][i];
        }
    }
  }
}

// NT13 / NT2: non-temporal weight loads in the W13 ring (items of one or two
// row tiles) and in W2.
template <int RB, int RTMAX, bool NT13, bool NT2>
__global__ __launch_bounds__(256, 2) void prefill_fused_kernel(const int32_t* items, const int32_t* num_items,
                                                               const int32_t* row_slot, const uint8_t* bank,
                                                               const uint16_t* x, uint64_t expert_bytes,
                                                               uint64_t w13_off, uint64_t w13_meta_off,
                                                               uint64_t w2_off, uint64_t w2_meta_off, int H, int I,
                                                               int topk, float* y, int run_log2) {
  constexpr int CT = kWxCT13;
  static_assert(kWxCT2 == CT, "one block width for both products");
  // act (the W2 A chunk) stays for the whole item; W13's staging and W2's
  // weights and records share the rest
  constexpr int kW13Dw = wx_a_dw(kWxCG13) + wx_r_dw(CT, kWxCG13);
  constexpr int kW2Dw = wx_r_dw(CT, kWxCG2) + wx_b_dw(CT, kWxCG2);
  __shared__ __attribute__((aligned(16))) uint32_t act[wx_a_dw(kWxCG2)];
  __shared__ __attribute__((aligned(16))) uint32_t lds[kW13Dw > kW2Dw ? kW13Dw : kW2Dw];
  __shared__ __attribute__((aligned(16))) uint32_t ring[4];  // unused (W13 keeps its weights in registers)
  int it, bx;
  xcd_item_tile(run_log2, it, bx);
  if (it >= *num_items) return;
  int e, row0, rows;
  item_of(items, it, e, row0, rows);
  const uint8_t* blk = bank + (uint64_t)e * expert_bytes;
  const int G13 = H >> 5, NT13c = (2 * I) >> 4, G2 = I >> 5, NT2c = H >> 4;  // groups and column tiles
  const int rt = (rows + 15) >> 4;  // 1 .. RTMAX
  // the act groups past K (inter < 160) are zeros for the W2 products
  for (int d = G2 * 1024 + (int)threadIdx.x; d < kWxCG2 * 1024; d += 256) act[d] = 0u;
  static_for<RTMAX>([&](auto i_c) {
    constexpr int RT = decltype(i_c)::value + 1;
    if (rt == RT) {
      wide_item<RB, RT, kWxCG13, CT, kWideW13, true, NT13>(blk + w13_off, blk + w13_meta_off, x, row_slot, row0,
                                                           rows, topk, G13, NT13c, 0, act, 0, lds,
                                                           lds + wx_a_dw(kWxCG13), ring);
      __syncthreads();  // act complete; W13's LDS free
      w2_resident<RB, RT, CT, NT2>(blk + w2_off, blk + w2_meta_off, act, G2, NT2c, row0, rows, y, H, lds,
                                   lds + wx_r_dw(CT, kWxCG2));
    }
  });
}

// ---------------------------------------------------------------------------
// W2: grid (ceil(H/16 / 8) column blocks, work items), 4 waves. The 8 tiles
// of the block are staged in chunks of up to 5 groups (all of K at inter
// 160) with LDS-direct loads, the activations of the chunk are requested
// with them, and wave w takes tiles w and w + 4 over the chunk's groups,
// writing fp32 row results.
// ---------------------------------------------------------------------------
constexpr int kW2Chunk = 5;
constexpr int kW2TileDw = 4 * run_stride(kW2Chunk);
constexpr int kW2TileUnits = 16 * kW2Chunk;                // 16-byte units of a staged tile
constexpr int kW2Loads = (8 * kW2TileUnits + 63) / 64;     // 64-unit LDS-direct loads per block
static_assert(run_stride(kW2Chunk) == 4 * 4 * kW2Chunk, "W2 runs are unpadded, so a block is one contiguous LDS run");

template <int RB, int NRT>
__device__ __forceinline__ void w2_block(const uint8_t* __restrict__ units, const uint8_t* __restrict__ recs,
                                         const uint16_t* __restrict__ ar0, const uint16_t* __restrict__ ar1, int G,
                                         int T, uint32_t* wl, uint8_t* rl, f4_t (&acc)[2][2]) {
  const uint32_t m1024 = magic1024();
  const int lane = threadIdx.x & 63, wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int c = lane & 15, kb = lane >> 4, quad = c >> 2, j = c & 3;
  constexpr int rs = run_stride(kW2Chunk);
  for (int g0 = 0; g0 < G; g0 += kW2Chunk) {
    const int kc = min(kW2Chunk, G - g0);
    if (g0 > 0) __syncthreads();  // the previous chunk's LDS reads are done
    // weights: the chunk's 8 tiles x 4 runs x 4 kc units lie contiguously in
    // LDS (the runs need no padding), 64 units per LDS-direct load, each lane
    // with its own bank address
#pragma unroll
    for (int i = wave; i < kW2Loads; i += 4) {
      const int up = 64 * i + lane;
      const int tt = up / kW2TileUnits, rem = up - tt * kW2TileUnits;
      const int jr = rem / (4 * kW2Chunk), u = rem - jr * (4 * kW2Chunk);
      if (tt < T && u < 4 * kc)
        lds_direct16(units + (uint64_t)tt * 256 * G + (uint64_t)jr * 64 * G + 64 * g0 + 16 * u, wl + 256 * i);
    }
    const Piece prc = record_piece<RB, kW2Chunk>((int)threadIdx.x, T, G, g0, kc, 16 * kW2Chunk * 4);
    const uint4 vr = load_records4<RB>(recs, prc);
    h8_t a0[kW2Chunk], a1[kW2Chunk];
#pragma unroll
    for (int i = 0; i < kW2Chunk; ++i) {
      const int g = g0 + min(i, kc - 1);
      a0[i] = *reinterpret_cast<const h8_t*>(ar0 + 32 * g + 8 * kb);
      if constexpr (NRT == 2) a1[i] = *reinterpret_cast<const h8_t*>(ar1 + 32 * g + 8 * kb);
    }
    if (prc.on) *reinterpret_cast<uint4*>(rl + prc.dst) = vr;
    // the barrier waits for every load of the workgroup, the LDS-direct ones included
    __syncthreads();
#pragma unroll
    for (int i = 0; i < kW2Chunk; ++i) {
#pragma unroll
      for (int q = 0; q < 2; ++q) {
        const int tt = wave + 4 * q;
        if (tt < T) {
          h8_t b;
          float sc;
          lds_operand<RB>(wl + tt * kW2TileDw, rl + tt * 16 * kW2Chunk * 4, rs, i, quad, j, kb, m1024, b, sc);
          sc = i < kc ? sc : 0.f;
          scale_add(acc[q][0], sc, mfma16(a0[i], b));
          if constexpr (NRT == 2) scale_add(acc[q][1], sc, mfma16(a1[i], b));
        }
      }
    }
  }
}

template <int RB>
__global__ __launch_bounds__(256) void prefill_w2_kernel(const int32_t* __restrict__ items,
                                                         const int32_t* __restrict__ num_items,
                                                         const uint8_t* __restrict__ bank, uint64_t expert_bytes,
                                                         uint64_t units_off, uint64_t meta_off, int H, int I,
                                                         const uint16_t* __restrict__ act, float* __restrict__ y,
                                                         int run_log2) {
  __shared__ __attribute__((aligned(16))) uint32_t wl[8 * kW2TileDw];
  __shared__ __attribute__((aligned(16))) uint8_t rl[8 * 16 * kW2Chunk * 4];
  int it, nb;
  xcd_item_tile(run_log2, it, nb);
  if (it >= *num_items) return;
  int e, row0, rows;
  item_of(items, it, e, row0, rows);
  const int G = I >> 5, NT = H >> 4;
  const int lane = threadIdx.x & 63, wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int c = lane & 15, kb = lane >> 4;
  const int nt0 = nb * 8;
  const int T = min(8, NT - nt0);  // 8, or the last block's 2, 4 or 6 tiles
  const uint8_t* blk = bank + (uint64_t)e * expert_bytes;
  const uint8_t* units = blk + units_off + (uint64_t)nt0 * 256 * G;
  const uint8_t* recs = blk + meta_off + (uint64_t)nt0 * 16 * G * RB;
  const uint16_t* ar0 = act + (uint64_t)(row0 + min(c, rows - 1)) * I;
  const uint16_t* ar1 = act + (uint64_t)(row0 + min(16 + c, rows - 1)) * I;
  f4_t acc[2][2] = {};
  if (rows > 16)
    w2_block<RB, 2>(units, recs, ar0, ar1, G, T, wl, rl, acc);
  else
    w2_block<RB, 1>(units, recs, ar0, ar1, G, T, wl, rl, acc);
  const int nrt = rows > 16 ? 2 : 1;
#pragma unroll
  for (int q = 0; q < 2; ++q) {
    const int tt = wave + 4 * q;
    if (tt >= T) break;
    const int nt = nt0 + tt;
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
// reduce: grid (ceil(H/512), ceil(M/4)), four waves, wave w taking token
// 4 blockIdx.y + w (four-wave workgroups: one-wave workgroups left CUs short
// of waves); lane l sums columns 4l .. 4l + 3 and 256 + 4l .. 256 + 4l + 3 of
// a 512-column block (each of the two loads of a row covers 1 KB). The
// token's valid slots are ranked by (expert id, slot) with lane reads, then
// summed in that order: acc = fma(w, y, acc) from +0, rounded once to fp16.
// The rows are requested kRedBatch at a time before any is summed (one
// memory round trip per batch), with non-temporal loads (each row is read
// once).
// ---------------------------------------------------------------------------
constexpr int kRedBatch = 8;

__global__ __launch_bounds__(256) void prefill_reduce_kernel(const int32_t* __restrict__ ids,
                                                             const float* __restrict__ topk_w,
                                                             const int32_t* __restrict__ slot_row,
                                                             const float* __restrict__ y, int M, int H, int topk,
                                                             int E, uint16_t* __restrict__ out) {
  __shared__ int order_row[4][AWQ_MOE_KMAX_TOPK];
  __shared__ float order_w[4][AWQ_MOE_KMAX_TOPK];
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int tok = blockIdx.y * 4 + wave;
  const bool live_tok = tok < M;
  const int s = (live_tok ? tok : 0) * topk + lane;
  const int id = lane < topk ? ids[s] : -1;
  const bool valid = live_tok && lane < topk && id >= 0 && id < E;
  const int key = valid ? id * 32 + lane : 0x7FFFFFFF;
  int rank = 0;
  for (int jj = 0; jj < topk; ++jj) rank += __builtin_amdgcn_readlane(key, jj) < key;
  if (valid) {
    order_row[wave][rank] = slot_row[s];
    order_w[wave][rank] = topk_w[s];
  }
  const int nvalid = __popcll(__ballot(valid));
  __syncthreads();
  const int col = blockIdx.x * 512 + 4 * lane;  // and col + 256
  if (!live_tok || col >= H) return;
  const bool hi_half = col + 256 < H;
  float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  for (int r0 = 0; r0 < nvalid; r0 += kRedBatch) {
    f4_t v[kRedBatch][2];
#pragma unroll
    for (int b = 0; b < kRedBatch; ++b) {
      // rows past the token's last are requested again from its first (never summed)
      const float* yr = y + (uint64_t)order_row[wave][r0 + b < nvalid ? r0 + b : 0] * H + col;
      v[b][0] = __builtin_nontemporal_load(reinterpret_cast<const f4_t*>(yr));
      v[b][1] = __builtin_nontemporal_load(reinterpret_cast<const f4_t*>(yr + (hi_half ? 256 : 0)));
    }
#pragma unroll
    for (int b = 0; b < kRedBatch; ++b) {
      if (r0 + b >= nvalid) break;
      const float w = order_w[wave][r0 + b];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        acc[i] = fmaf(w, v[b][0][i], acc[i]);
        acc[4 + i] = fmaf(w, v[b][1][i], acc[4 + i]);
      }
    }
  }
  typedef _Float16 h4_t __attribute__((ext_vector_type(4)));
  h4_t o0, o1;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    o0[i] = (_Float16)acc[i];
    o1[i] = (_Float16)acc[4 + i];
  }
  *reinterpret_cast<h4_t*>(out + (uint64_t)tok * H + col) = o0;
  if (hi_half) *reinterpret_cast<h4_t*>(out + (uint64_t)tok * H + col + 256) = o1;
}

// ---------------------------------------------------------------------------
// launchers
// ---------------------------------------------------------------------------
int prefill_max_items(int n, int E) { return (n + kItemRows - 1) / kItemRows + (E < n ? E : n); }
int prefill_max_wide_items(int n, int E) { return (n + kWideRows - 1) / kWideRows + (E < n ? E : n); }

template <int RB, bool NT13, bool NT2>
static void launch_fused(const StageArgs& a, const uint16_t* x, const PrefillWs& w, int witems8, int wrun_log2,
                         hipStream_t stream) {
  hipLaunchKernelGGL((prefill_fused_kernel<RB, kWxRT, NT13, NT2>), dim3(1, witems8), dim3(256), 0, stream, w.witems,
                     w.num_witems, w.row_slot, a.bank, x, a.expert_bytes, a.w13_off, a.w13_meta_off, a.w2_off,
                     a.w2_meta_off, a.H, a.I, a.topk, w.y, wrun_log2);
}

// Non-temporal weight loads in the one-launch kernel, by the mean rows per
// expert r = n / E (n slots): W13's whole-unit ring when r <= 32 (an
// expert then mostly has one item, and no other workgroup reads its
// weights), W2 when r >= 16. Per call at the rank layer (µs, one run of
// each under the kernel trace; plain / W13 / W2 / both): 128 tokens
// (r = 2.5) 91.9 / 89.4 / 93.1 / 92.2, 1024 (r = 20) 142.1 / 139.8 / 140.4 /
// 137.7, 4096 (r = 80) 359.7 / 362.3 / 354.1 / 355.2.
template <int RB>
static void launch_fused_rb(const StageArgs& a, const uint16_t* x, const PrefillWs& w, int witems8, int wrun_log2,
                            hipStream_t stream) {
  const uint64_t n = (uint64_t)a.M * a.topk;
  const bool nt13 = n <= 32ull * a.E, nt2 = n >= 16ull * a.E;
  if (nt13 && nt2)
    launch_fused<RB, true, true>(a, x, w, witems8, wrun_log2, stream);
  else if (nt13)
    launch_fused<RB, true, false>(a, x, w, witems8, wrun_log2, stream);
  else
    launch_fused<RB, false, true>(a, x, w, witems8, wrun_log2, stream);
}

hipError_t launch_prefill(const StageArgs& a, const uint16_t* x, const float* topk_w, uint16_t* out,
                          const PrefillWs& w, hipStream_t stream) {
  const int n = a.M * a.topk;
  if (a.M <= kDecodeFormMaxTokens && n <= kDecodeFormMaxSlots) {
    // few tokens: the decode kernels (W13 per slot and tile, W2 per token
    // and tile, the token's slots summed in ascending (expert, slot) order),
    // on the workspace's first bytes in the decode layout (status word at 0,
    // act at 256); no routing and no row results
    uint8_t* ws0 = reinterpret_cast<uint8_t*>(w.status);
    hipError_t e = launch_w13_swiglu(a, x, ws0, false, 0.f, kW13Table, stream);
    if (e != hipSuccess) return e;
    return launch_w2_reduce(a, reinterpret_cast<const uint16_t*>(ws0 + AWQ_MOE_KWS_ACT_OFFSET), topk_w, out,
                            nullptr, kW2Table, stream);
  }
  const int max_items = prefill_max_items(n, a.E);
  hipError_t err;
  if (n <= kRouteBatch * 1024) {
    hipLaunchKernelGGL(prefill_place_kernel<true>, dim3(1), dim3(1024), 0, stream, a.topk_ids, n, a.E, n, 1,
                       w.route_cnt, w.route_bad, w.slot_row, w.row_slot, w.items, w.num_items, w.witems, w.num_witems,
                       w.status);
  } else {
    const int nb = prefill_route_blocks(n, a.E), per = (n + nb - 1) / nb;
    hipLaunchKernelGGL(prefill_count_kernel, dim3(nb), dim3(1024), 0, stream, a.topk_ids, n, a.E, per, w.route_cnt,
                       w.route_bad);
    if ((err = hipGetLastError()) != hipSuccess) return err;
    hipLaunchKernelGGL(prefill_place_kernel<false>, dim3(nb), dim3(1024), 0, stream, a.topk_ids, n, a.E, per, nb,
                       w.route_cnt, w.route_bad, w.slot_row, w.row_slot, w.items, w.num_items, w.witems, w.num_witems,
                       w.status);
  }
  if ((err = hipGetLastError()) != hipSuccess) return err;
  // runs of 8 items per XCD from 64 rows per expert on average (2 items or more each)
  const int run_log2 = n >= 64 * a.E ? 3 : 0;
  const int round = 8 << run_log2;
  const int items8 = (max_items + round - 1) / round * round;  // whole XCD rounds (see xcd_item_tile)
  const dim3 g13((2 * a.I) / 16, items8), g2(((a.H / 16) + 7) / 8, items8);
  const bool wide = a.M >= kWideMinTokens;
  const int wrun_log2 = n >= 64 * a.E ? 1 : 0;
  const int wround = 8 << wrun_log2;
  const int witems8 = (prefill_max_wide_items(n, a.E) + wround - 1) / wround * wround;
  if (wide && a.I <= kFusedMaxInter) {
    // both products per wide item in one launch
    if (a.RB == 4)
      launch_fused_rb<4>(a, x, w, witems8, wrun_log2, stream);
    else
      launch_fused_rb<3>(a, x, w, witems8, wrun_log2, stream);
  } else if (wide) {
    // many rows per expert: wide items, 20 column tiles per workgroup
    const dim3 g13w(((2 * a.I) / 16 + 4 * kWxCT13 - 1) / (4 * kWxCT13), witems8);
    if (a.RB == 4)
      hipLaunchKernelGGL((prefill_wide_kernel<4, kWideW13, kWxRT>), g13w, dim3(256), 0, stream, w.witems, w.num_witems,
                         w.row_slot, a.bank, x, a.expert_bytes, a.w13_off, a.w13_meta_off, a.H, a.I, a.topk,
                         (void*)w.act, wrun_log2);
    else
      hipLaunchKernelGGL((prefill_wide_kernel<3, kWideW13, kWxRT>), g13w, dim3(256), 0, stream, w.witems, w.num_witems,
                         w.row_slot, a.bank, x, a.expert_bytes, a.w13_off, a.w13_meta_off, a.H, a.I, a.topk,
                         (void*)w.act, wrun_log2);
  } else if (a.RB == 4) {
    hipLaunchKernelGGL(prefill_w13_kernel<4>, g13, dim3(256), 0, stream, w.items, w.num_items, w.row_slot, a.bank, x,
                       a.expert_bytes, a.w13_off, a.w13_meta_off, a.H, a.I, a.topk, w.act, run_log2);
  } else {
    hipLaunchKernelGGL(prefill_w13_kernel<3>, g13, dim3(256), 0, stream, w.items, w.num_items, w.row_slot, a.bank, x,
                       a.expert_bytes, a.w13_off, a.w13_meta_off, a.H, a.I, a.topk, w.act, run_log2);
  }
  if ((err = hipGetLastError()) != hipSuccess) return err;
  if (wide && a.I <= kFusedMaxInter) {
    // W2 ran in the fused launch
  } else if (wide && n < kW2WideItemsFrom) {
    // W2 over the 32-row work items (two row tiles at most): a smaller
    // register budget, three workgroups per CU
    const dim3 g2n(((a.H / 16) + 4 * kWxCT2Narrow - 1) / (4 * kWxCT2Narrow), items8);
    if (a.RB == 4)
      hipLaunchKernelGGL((prefill_wide_kernel<4, kWideW2, 2>), g2n, dim3(256), 0, stream, w.items, w.num_items,
                         w.row_slot, a.bank, w.act, a.expert_bytes, a.w2_off, a.w2_meta_off, a.H, a.I, a.topk,
                         (void*)w.y, run_log2);
    else
      hipLaunchKernelGGL((prefill_wide_kernel<3, kWideW2, 2>), g2n, dim3(256), 0, stream, w.items, w.num_items,
                         w.row_slot, a.bank, w.act, a.expert_bytes, a.w2_off, a.w2_meta_off, a.H, a.I, a.topk,
                         (void*)w.y, run_log2);
  } else if (wide) {
    const dim3 g2w(((a.H / 16) + 4 * kWxCT2 - 1) / (4 * kWxCT2), witems8);
    if (a.RB == 4)
      hipLaunchKernelGGL((prefill_wide_kernel<4, kWideW2, kWxRT>), g2w, dim3(256), 0, stream, w.witems, w.num_witems,
                         w.row_slot, a.bank, w.act, a.expert_bytes, a.w2_off, a.w2_meta_off, a.H, a.I, a.topk,
                         (void*)w.y, wrun_log2);
    else
      hipLaunchKernelGGL((prefill_wide_kernel<3, kWideW2, kWxRT>), g2w, dim3(256), 0, stream, w.witems, w.num_witems,
                         w.row_slot, a.bank, w.act, a.expert_bytes, a.w2_off, a.w2_meta_off, a.H, a.I, a.topk,
                         (void*)w.y, wrun_log2);
  } else if (a.RB == 4) {
    hipLaunchKernelGGL(prefill_w2_kernel<4>, g2, dim3(256), 0, stream, w.items, w.num_items, a.bank, a.expert_bytes,
                       a.w2_off, a.w2_meta_off, a.H, a.I, w.act, w.y, run_log2);
  } else {
    hipLaunchKernelGGL(prefill_w2_kernel<3>, g2, dim3(256), 0, stream, w.items, w.num_items, a.bank, a.expert_bytes,
                       a.w2_off, a.w2_meta_off, a.H, a.I, w.act, w.y, run_log2);
  }
  if ((err = hipGetLastError()) != hipSuccess) return err;
  hipLaunchKernelGGL(prefill_reduce_kernel, dim3((a.H + 511) / 512, (a.M + 3) / 4), dim3(256), 0, stream, a.topk_ids,
                     topk_w, w.slot_row, w.y, a.M, a.H, a.topk, a.E, out);
  return hipGetLastError();
}

}  // namespace awq_moe
