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
constexpr int kRouteBatch = 16;  // slot ids per thread in flight in the routing kernel

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
  // The slots are read kRouteBatch per thread at a time, every load issued
  // before the first is used: one memory round trip per batch, not per slot.
  for (int s0 = t; s0 < n; s0 += kRouteBatch * 1024) {
    int ev[kRouteBatch];
#pragma unroll
    for (int b = 0; b < kRouteBatch; ++b) {
      const int s = s0 + 1024 * b;
      ev[b] = s < n ? ids[s] : 0;
    }
#pragma unroll
    for (int b = 0; b < kRouteBatch; ++b) {
      if (s0 + 1024 * b >= n) break;
      const int e = ev[b];
      if (e >= 0 && e < E)
        atomicAdd(&cnt[e], 1);
      else
        bad = 1;
    }
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
  for (int s0 = t; s0 < n; s0 += kRouteBatch * 1024) {
    int ev[kRouteBatch];
#pragma unroll
    for (int b = 0; b < kRouteBatch; ++b) {
      const int s = s0 + 1024 * b;
      ev[b] = s < n ? ids[s] : 0;
    }
#pragma unroll
    for (int b = 0; b < kRouteBatch; ++b) {
      const int s = s0 + 1024 * b;
      if (s >= n) break;
      const int e = ev[b];
      if (e >= 0 && e < E) {
        const int r = atomicAdd(&cur[e], 1);
        slot_row[s] = r;
        row_slot[r] = s;
      } else {
        slot_row[s] = -1;
      }
    }
  }
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

// ---------------------------------------------------------------------------
// W13 + SwiGLU for calls with many rows per expert: grid (ceil(NT/4) groups
// of 4 column tiles, work items), 4 waves; wave w owns tile 4 q + w over
// all of K, so an activation row staged once serves four tiles. Per chunk
// of kMtChunk groups everything goes straight into LDS with LDS-direct
// loads: the item's activations as [group][k block][row][16 B] (a load of
// 64 lanes is 2 k blocks x 32 rows of one group, and an MFMA operand read
// is 1 KB contiguous), the four tiles' weight runs at a stride of
// kMtRun units (16 or 48 mod 64 dwords, so operand reads hit 64 banks; pad
// units, if any, are lanes that load nothing), the records through
// registers as dwords. Chunks of 8 groups keep the LDS at 27 KB, so five
// workgroups fit on a CU (10 groups, 34 KB: four).
// Each wave keeps its tile's sums in registers to the end (no cross-wave
// reduction), then applies SwiGLU.
// ---------------------------------------------------------------------------
constexpr int kMtChunk = 8;
// Calls from this many tokens take the multi-tile W13 kernel. Single-tile
// against multi-tile, us per call: M = 32: 62.2 / 63.6, M = 64: 88.1 / 91.4,
// M = 128: 113.8 / 112.9 (even); from M = 256 the multi-tile kernel is ahead.
constexpr int kMtMinTokens = 256;
constexpr int kMtRun = 36;  // units per weight run in LDS (4 * kMtChunk = 32 used)
constexpr int kMtAUnits = kMtChunk * 4 * 32;       // 16-byte activation units per chunk
constexpr int kMtBUnits = 16 * kMtRun;             // 4 tiles x 4 runs
constexpr int kMtBLoads = (kMtBUnits + 63) / 64;
constexpr int kMtRecDw = 16 * kMtChunk;            // record dwords per tile and chunk
static_assert(((4 * kMtRun) % 64 == 16 || (4 * kMtRun) % 64 == 48) && kMtRun >= 4 * kMtChunk,
              "weight runs: 64 banks, room for a chunk");
static_assert(4 * 4 * kMtChunk <= 256, "record quads: one per thread");

template <int RB>
__global__ __launch_bounds__(256) void prefill_w13_mt_kernel(const int32_t* __restrict__ items,
                                                             const int32_t* __restrict__ num_items,
                                                             const int32_t* __restrict__ row_slot,
                                                             const uint8_t* __restrict__ bank,
                                                             const uint16_t* __restrict__ x, uint64_t expert_bytes,
                                                             uint64_t units_off, uint64_t meta_off, int H, int I,
                                                             int topk, uint16_t* __restrict__ act, int run_log2) {
  __shared__ __attribute__((aligned(16))) uint32_t al[kMtAUnits * 4];
  __shared__ __attribute__((aligned(16))) uint32_t bl[kMtBUnits * 4];
  __shared__ __attribute__((aligned(16))) uint32_t rl[4 * kMtRecDw];
  int it, tq;
  xcd_item_tile(run_log2, it, tq);
  if (it >= *num_items) return;
  int e, row0, rows;
  item_of(items, it, e, row0, rows);
  const int G = H >> 5, NT = (2 * I) >> 4;
  const uint32_t m1024 = magic1024();
  const int t = threadIdx.x, lane = t & 63, wave = __builtin_amdgcn_readfirstlane(t >> 6);
  const int c = lane & 15, kb = lane >> 4, quad = c >> 2, j = c & 3;
  const int nt0 = 4 * tq, T = min(4, NT - nt0);
  const uint8_t* blk = bank + (uint64_t)e * expert_bytes;
  const uint8_t* units = blk + units_off + (uint64_t)nt0 * 256 * G;
  const uint8_t* recs = blk + meta_off + (uint64_t)nt0 * 16 * G * RB;
  const int nrt = rows > 16 ? 2 : 1;
  // the activation row this lane copies (row = lane & 31; rows past the item repeat its last row)
  const int arow = lane & 31;
  const uint16_t* xrow = x + (uint64_t)(row_slot[row0 + min(arow, rows - 1)] / topk) * H + 8 * (lane >> 5);
  f4_t acc0 = {0.f, 0.f, 0.f, 0.f}, acc1 = {0.f, 0.f, 0.f, 0.f};
  for (int g0 = 0; g0 < G; g0 += kMtChunk) {
    const int kc = min(kMtChunk, G - g0);
    if (g0 > 0) __syncthreads();  // the previous chunk's LDS reads are done
    // activations: load m = 2 gl + h covers k blocks 2h, 2h + 1 of group gl for rows 0..31
    for (int m = wave; m < 2 * kc; m += 4) {
      const int gl = m >> 1, h = m & 1;
      if (arow < 16 * nrt)
        lds_direct16(reinterpret_cast<const uint8_t*>(xrow + 32 * (g0 + gl) + 16 * h), al + 256 * m);
    }
    // weights: unit position p = (tile * 4 + j) * kMtRun + u
#pragma unroll
    for (int i = wave; i < kMtBLoads; i += 4) {
      const int pos = 64 * i + lane;
      const int tj = pos / kMtRun, u = pos - tj * kMtRun;
      const int tt = tj >> 2, jr = tj & 3;
      if (tt < T && u < 4 * kc)
        lds_direct16(units + (uint64_t)tt * 256 * G + (uint64_t)jr * 64 * G + 64 * g0 + 16 * u, bl + 256 * i);
    }
    // records: quad r of tile tt (4 records of group r / 4), as dwords
    {
      const int tt = t / (4 * kMtChunk), rem = t - tt * (4 * kMtChunk);
      const bool on = tt < T && rem < 4 * kc;
      typedef uint32_t u32x3 __attribute__((ext_vector_type(3), aligned(4)));
      const uint8_t* rp = recs + (on ? (uint64_t)tt * 16 * G * RB + (16 * g0 + 4 * rem) * RB : 0);
      const u32x3 d = *reinterpret_cast<const u32x3*>(rp);
      uint4 v;
      if constexpr (RB == 4) {
        v = make_uint4(d.x, d.y, d.z, *reinterpret_cast<const uint32_t*>(rp + 12));
      } else {
        v = make_uint4(d.x & 0xFFFFFFu, (d.x >> 24) | ((d.y & 0xFFFFu) << 8), (d.y >> 16) | ((d.z & 0xFFu) << 16),
                       d.z >> 8);
      }
      if (on) *reinterpret_cast<uint4*>(rl + tt * kMtRecDw + 4 * rem) = v;
    }
    // the barrier waits for every load of the workgroup, the LDS-direct ones included
    __syncthreads();
    if (wave < T) {
      const uint32_t* bw = bl + wave * 4 * kMtRun * 4;
      const uint32_t* rw = rl + wave * kMtRecDw;
      for (int gl = 0; gl < kc; ++gl) {
        const uint32_t w = bw[(j * kMtRun + 4 * gl + quad) * 4 + kb];
        const uint32_t r = rw[16 * gl + 4 * quad + j];
        const float sc = (float)__builtin_bit_cast(_Float16, (uint16_t)(r & 0xFFFFu));
        const h8_t b = qz_operand(w, (r >> 16) & 0xFFu, m1024);
        const h8_t a0 = *reinterpret_cast<const h8_t*>(al + ((gl * 4 + kb) * 32 + c) * 4);
        scale_add(acc0, sc, mfma16(a0, b));
        if (nrt == 2) {
          const h8_t a1 = *reinterpret_cast<const h8_t*>(al + ((gl * 4 + kb) * 32 + 16 + c) * 4);
          scale_add(acc1, sc, mfma16(a1, b));
        }
      }
    }
  }
  if (wave >= T) return;
  const int nt = nt0 + wave;
  for (int rt = 0; rt < nrt; ++rt) {
    const f4_t d = rt == 0 ? acc0 : acc1;
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
  // runs of 8 items per XCD from 64 rows per expert on average (2 items or more each)
  const int run_log2 = n >= 64 * a.E ? 3 : 0;
  const int round = 8 << run_log2;
  const int items8 = (max_items + round - 1) / round * round;  // whole XCD rounds (see xcd_item_tile)
  const dim3 g13((2 * a.I) / 16, items8), g2(((a.H / 16) + 7) / 8, items8);
  if (a.M >= kMtMinTokens) {
    // many rows per expert: four tiles per workgroup share the staged activations
    const dim3 g13m(((2 * a.I) / 16 + 3) / 4, items8);
    if (a.RB == 4)
      hipLaunchKernelGGL(prefill_w13_mt_kernel<4>, g13m, dim3(256), 0, stream, w.items, w.num_items, w.row_slot, a.bank,
                         x, a.expert_bytes, a.w13_off, a.w13_meta_off, a.H, a.I, a.topk, w.act, run_log2);
    else
      hipLaunchKernelGGL(prefill_w13_mt_kernel<3>, g13m, dim3(256), 0, stream, w.items, w.num_items, w.row_slot, a.bank,
                         x, a.expert_bytes, a.w13_off, a.w13_meta_off, a.H, a.I, a.topk, w.act, run_log2);
  } else if (a.RB == 4) {
    hipLaunchKernelGGL(prefill_w13_kernel<4>, g13, dim3(256), 0, stream, w.items, w.num_items, w.row_slot, a.bank, x,
                       a.expert_bytes, a.w13_off, a.w13_meta_off, a.H, a.I, a.topk, w.act, run_log2);
  } else {
    hipLaunchKernelGGL(prefill_w13_kernel<3>, g13, dim3(256), 0, stream, w.items, w.num_items, w.row_slot, a.bank, x,
                       a.expert_bytes, a.w13_off, a.w13_meta_off, a.H, a.I, a.topk, w.act, run_log2);
  }
  if ((err = hipGetLastError()) != hipSuccess) return err;
  if (a.RB == 4) {
    hipLaunchKernelGGL(prefill_w2_kernel<4>, g2, dim3(256), 0, stream, w.items, w.num_items, a.bank, a.expert_bytes,
                       a.w2_off, a.w2_meta_off, a.H, a.I, w.act, w.y, run_log2);
  } else {
    hipLaunchKernelGGL(prefill_w2_kernel<3>, g2, dim3(256), 0, stream, w.items, w.num_items, a.bank, a.expert_bytes,
                       a.w2_off, a.w2_meta_off, a.H, a.I, w.act, w.y, run_log2);
  }
  if ((err = hipGetLastError()) != hipSuccess) return err;
  hipLaunchKernelGGL(prefill_reduce_kernel, dim3((a.H + 511) / 512, a.M), dim3(64), 0, stream, a.topk_ids, topk_w,
                     w.slot_row, w.y, a.H, a.topk, a.E, out);
  return hipGetLastError();
}

}  // namespace awq_moe
