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

// Cross-lane sums in the VALU (DPP and gfx950 permlane swaps), no LDS round trip.
template <int CTRL>
__device__ __forceinline__ float dpp(float v) {
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), CTRL, 0xF, 0xF, false));
}
constexpr int kRowRor4 = 0x124, kRowRor8 = 0x128;
constexpr int kQuadSwap1 = 0xB1;  // quad_perm [1,0,3,2]
constexpr int kQuadSwap2 = 0x4E;  // quad_perm [2,3,0,1]
constexpr int kRowHalfMirror = 0x141;

// Sum four per-lane values over the 16 lanes that share lane bits 0..1 (one
// column quad of a wave): two DPP row rotations sum within each 16-lane row
// in the VALU; then a reduce-scatter across rows: the xor-16 exchange trades
// two of the four values, the xor-32 exchange one, so lane l ends with the
// full sum of value 2*b4 + b5 (b4, b5 = lane bits 4, 5). The lanes with
// (lane & 12) == 0 carry the four results of their quad.
__device__ __forceinline__ float sum4_lane_bits_2to5(float p0, float p1, float p2, float p3) {
  p0 += dpp<kRowRor4>(p0);
  p1 += dpp<kRowRor4>(p1);
  p2 += dpp<kRowRor4>(p2);
  p3 += dpp<kRowRor4>(p3);
  p0 += dpp<kRowRor8>(p0);
  p1 += dpp<kRowRor8>(p1);
  p2 += dpp<kRowRor8>(p2);
  p3 += dpp<kRowRor8>(p3);
  const int lane = threadIdx.x & 63;
  const bool b4 = (lane & 16) != 0, b5 = (lane & 32) != 0;
  float k0 = b4 ? p2 : p0, k1 = b4 ? p3 : p1;
  k0 += __shfl_xor(b4 ? p0 : p2, 16);
  k1 += __shfl_xor(b4 ? p1 : p3, 16);
  float k = b5 ? k1 : k0;
  k += __shfl_xor(b5 ? k0 : k1, 32);
  return k;
}

// Sum over aligned groups of 8 lanes (lane bits 0..2); every lane gets the sum.
__device__ __forceinline__ float sum_lane_bits_0to2(float v) {
  v += dpp<kQuadSwap1>(v);
  v += dpp<kQuadSwap2>(v);
  v += dpp<kRowHalfMirror>(v);
  return v;
}

// ---------------------------------------------------------------------------
// routing compaction of n <= 256 slots inside one workgroup (LDS only).
// Canonical order: experts ascending, rows of a segment by ascending slot,
// invalid slots (ids outside [0, E)) after all valid ones in slot order.
// Every stage kernel runs this in its prologue, so the only global-memory
// round trip before the weight loads is the read of the n routed ids.
// ---------------------------------------------------------------------------
constexpr int kMaxSlots = AWQ_MOE_KMAX_SLOTS;
constexpr int kNoKey = 0x7FFFFFFF;

struct __attribute__((aligned(16))) Compact {
  int key[kMaxSlots + 4];       // valid id, -1 invalid, -2 padding
  int firstkey[kMaxSlots + 4];  // id when the slot is its id's first valid slot, else kNoKey
  int rank[kMaxSlots];          // slot -> row
  int sorted[kMaxSlots];        // row -> slot
  int seg_e[kMaxSlots];         // segment -> expert
  int seg_off[kMaxSlots + 1];   // segment -> first row; [num_active] = number of valid slots
  int num_active, nvalid;
};

__device__ void block_compact(const int32_t* __restrict__ ids, int n, int E, Compact& C) {
  const int t = threadIdx.x, bd = blockDim.x;
  const int n4 = (n + 3) & ~3;
  for (int s = t; s < n4; s += bd) {
    int k = -2;
    if (s < n) {
      const int v = ids[s];
      k = (v >= 0 && v < E) ? v : -1;
    }
    C.key[s] = k;
    C.firstkey[s] = kNoKey;
  }
  __syncthreads();
  for (int s = t; s < n; s += bd) {
    const int id = C.key[s];
    int before = 0, inv_before = 0, nvalid = 0, dup_before = 0;
    for (int s2 = 0; s2 < n4; s2 += 4) {
      const int4 k4 = *reinterpret_cast<const int4*>(&C.key[s2]);
      const int kk[4] = {k4.x, k4.y, k4.z, k4.w};
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int k2 = kk[q];
        const bool earlier = (s2 + q) < s;
        nvalid += (k2 >= 0);
        before += (k2 >= 0) & ((k2 < id) | ((k2 == id) & earlier));
        dup_before += (k2 == id) & earlier;
        inv_before += (k2 == -1) & earlier;
      }
    }
    const int r = (id >= 0) ? before : nvalid + inv_before;
    C.rank[s] = r;
    C.sorted[r] = s;
    if (id >= 0 && dup_before == 0) C.firstkey[s] = id;
    if (s == 0) C.nvalid = nvalid;
  }
  __syncthreads();
  for (int s = t; s < n; s += bd) {
    const int fk = C.firstkey[s];
    int below = 0, nseg = 0;
    for (int s2 = 0; s2 < n4; s2 += 4) {
      const int4 f4 = *reinterpret_cast<const int4*>(&C.firstkey[s2]);
      const int ff[4] = {f4.x, f4.y, f4.z, f4.w};
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        below += ff[q] < fk;
        nseg += ff[q] != kNoKey;
      }
    }
    if (fk != kNoKey) {
      C.seg_e[below] = fk;
      C.seg_off[below] = C.rank[s];
    }
    if (s == 0) {
      C.num_active = nseg;
      C.seg_off[nseg] = C.nvalid;
    }
  }
  __syncthreads();
}

// Write the compacted arrays of the workgroup to global memory.
__device__ void store_route(const Compact& C, int n, const RouteOut& o) {
  const int t = threadIdx.x, bd = blockDim.x;
  const int A = C.num_active, V = C.nvalid;
  for (int i = t; i < n; i += bd) {
    o.sorted_slots[i] = C.sorted[i];
    o.active_ids[i] = i < A ? C.seg_e[i] : -1;
  }
  for (int i = t; i <= n; i += bd) o.offsets[i] = i <= A ? C.seg_off[i] : V;
  if (t == 0) {
    *o.num_active = A;
    *o.status = (V == n) ? 0u : AWQ_MOE_STATUS_BAD_ID_BIT;
  }
}

__global__ __launch_bounds__(256) void route_compact_kernel(const int32_t* __restrict__ ids, int n, int E,
                                                            RouteOut o) {
  __shared__ Compact C;
  block_compact(ids, n, E, C);
  store_route(C, n, o);
}

// ---------------------------------------------------------------------------
// Segment discovery inside the stage kernels, without sorting. Each wave
// holds the routed ids of up to 256 slots in registers (slot c*64 + lane in
// chunk c); a ballot gives the 64-bit mask of slots that share an id, so the
// rows of a segment come out in ascending slot order for free.
// ---------------------------------------------------------------------------
struct SlotIds {
  int v[4];  // id of slot c*64 + lane, -1 when invalid or past n
};

__device__ __forceinline__ SlotIds load_slot_ids(const int32_t* __restrict__ ids, int n, int E) {
  SlotIds r;
  const int lane = threadIdx.x & 63;
#pragma unroll
  for (int c = 0; c < 4; ++c) {
    const int l = c * 64 + lane;
    int v = -1;
    if (l < n) {
      v = ids[l];
      if (v < 0 || v >= E) v = -1;
    }
    r.v[c] = v;
  }
  return r;
}

__device__ __forceinline__ void same_id_masks(const SlotIds& ids, int id, int n, uint64_t (&m)[4]) {
#pragma unroll
  for (int c = 0; c < 4; ++c) m[c] = (c * 64 < n) ? __ballot(ids.v[c] == id) : 0ull;
}

// Pop the lowest slot of a 256-bit mask (-1 when empty). Uniform.
__device__ __forceinline__ int pop_slot(uint64_t (&m)[4]) {
  int res = -1;
#pragma unroll
  for (int c = 0; c < 4; ++c) {
    if (res < 0 && m[c] != 0ull) {
      res = c * 64 + __builtin_ctzll(m[c]);
      m[c] &= m[c] - 1;
    }
  }
  return res;
}

// ---------------------------------------------------------------------------
// The routing plan for W2, built by one workgroup of the W13 launch while the
// other workgroups stream W13. All phases are parallel over slots:
//  1. insert every valid slot's expert into an LDS hash table (open
//     addressing, atomicCAS), keeping the lowest slot and the count per expert;
//  2. wave 0 numbers the segments in order of their lowest slot (ballots) and
//     turns the counts into offsets (wave prefix sums);
//  3. every slot takes a place in its segment's slot list (atomic fill; the
//     order inside a segment does not change any result, since every slot is
//     computed independently) and ranks itself inside its token by
//     (expert, slot), which fixes the order of the token's final sum.
// ---------------------------------------------------------------------------
constexpr int kHashBits = 9;
constexpr int kHash = 1 << kHashBits;  // > kMaxSlots, so probing always ends
static_assert(kHash > kMaxSlots, "hash table must exceed the slot count");

struct PlanLds {
  int tab_key[kHash];   // expert id, -1 empty
  int tab_min[kHash];   // lowest slot of the expert; then its segment index
  int tab_cnt[kHash];   // slots of the expert
  int tab_fill[kHash];  // placement counter
  int entry[kMaxSlots];  // slot -> table entry, -1 invalid
  int key[kMaxSlots];    // slot -> expert id, -1 invalid
  int seg_off[kMaxSlots + 1];
};

__device__ __forceinline__ int hash_slot(int k) {
  return (int)(((uint32_t)k * 2654435761u) >> (32 - kHashBits));
}

__device__ __forceinline__ int wave_inclusive_sum(int v) {
  const int lane = threadIdx.x & 63;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int u = __shfl_up(v, o);
    if (lane >= o) v += u;
  }
  return v;
}

__device__ void build_plan(const int32_t* __restrict__ topk_ids, int M, int topk, int E, Plan* __restrict__ plan,
                           uint32_t* __restrict__ status, PlanLds& P) {
  const int n = M * topk;
  const int t = threadIdx.x, lane = t & 63, bd = blockDim.x;
  for (int i = t; i < kHash; i += bd) {
    P.tab_key[i] = -1;
    P.tab_min[i] = 0x7FFFFFFF;
    P.tab_cnt[i] = 0;
    P.tab_fill[i] = 0;
  }
  __syncthreads();
  int bad = 0;
  for (int s = t; s < n; s += bd) {
    const int v = topk_ids[s];
    const int k = (v >= 0 && v < E) ? v : -1;
    P.key[s] = k;
    int h = -1;
    if (k >= 0) {
      h = hash_slot(k);
      for (;;) {
        const int old = atomicCAS(&P.tab_key[h], -1, k);
        if (old == -1 || old == k) break;
        h = (h + 1) & (kHash - 1);
      }
      atomicMin(&P.tab_min[h], s);
      atomicAdd(&P.tab_cnt[h], 1);
    } else {
      bad = 1;
    }
    P.entry[s] = h;
  }
  bad = __syncthreads_or(bad);
  if (t == 0 && status != nullptr) *status = bad ? AWQ_MOE_STATUS_BAD_ID_BIT : 0u;
  if (t < 64) {
    int nseg = 0, off = 0;
    for (int c = 0; c * 64 < n; ++c) {
      const int sl = c * 64 + lane;
      const int h = sl < n ? P.entry[sl] : -1;
      const bool leader = h >= 0 && P.tab_min[h] == sl;
      const uint64_t lm = __ballot(leader);
      const int cnt = leader ? P.tab_cnt[h] : 0;
      const int incl = wave_inclusive_sum(cnt);
      if (leader) {
        const int seg = nseg + (int)__builtin_amdgcn_mbcnt_hi((uint32_t)(lm >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)lm, 0));
        const int o = off + incl - cnt;
        P.tab_min[h] = seg;  // from here on: the expert's segment index
        P.seg_off[seg] = o;
        plan->seg_off[seg] = o;
        plan->seg_e[seg] = P.key[sl];
      }
      nseg += __builtin_popcountll(lm);
      off += __shfl(incl, 63);
    }
    if (lane == 0) {
      P.seg_off[nseg] = off;
      plan->seg_off[nseg] = off;
      plan->num_segments = nseg;
    }
  }
  __syncthreads();
  for (int s = t; s < n; s += bd) {
    const int h = P.entry[s];
    const int tok = s / topk, j = s - tok * topk, base = tok * topk;
    if (h >= 0) {
      const int pos = P.seg_off[P.tab_min[h]] + atomicAdd(&P.tab_fill[h], 1);
      plan->seg_slots[pos] = s;
      const int id = P.key[s];
      int r = 0;
      for (int j2 = 0; j2 < topk; ++j2) {
        const int k2 = P.key[base + j2];
        r += (k2 >= 0) & ((k2 < id) | ((k2 == id) & (j2 < j)));
      }
      plan->order[base + r] = s;
    }
    if (j == 0) {
      int c = 0;
      for (int j2 = 0; j2 < topk; ++j2) c += P.key[base + j2] >= 0;
      plan->cnt[tok] = c;
    }
  }
}

// ---------------------------------------------------------------------------
// W13 + SwiGLU: grid (2I/16 column tiles, 1 + n). Row 0 of the grid builds
// the routing plan (tile 0 only). The workgroup of slot s = blockIdx.y - 1
// works only when s is the lowest slot routed to its expert: it streams one
// 16-column tile of that expert over all of K once and applies it to every
// slot routed to the expert (a multi-row segment). act is indexed by slot.
// ---------------------------------------------------------------------------
template <int RB>
__global__ __launch_bounds__(1024) void w13_swiglu_kernel(StageArgs a, const uint16_t* __restrict__ x,
                                                          uint16_t* __restrict__ act, Plan* __restrict__ plan,
                                                          uint32_t* __restrict__ status) {
  constexpr int R = 2;  // rows per pass
  __shared__ float red[16][R][16];  // [wave][row][column]
  __shared__ PlanLds plan_lds;
  const int n = a.M * a.topk;
  const int nt = blockIdx.x;
  if (blockIdx.y == 0) {
    if (nt == 0) build_plan(a.topk_ids, a.M, a.topk, a.E, plan, status, plan_lds);
    return;
  }
  const int s = blockIdx.y - 1;
  const int t = threadIdx.x;
  const int lane = t & 63, wave = t >> 6, nwaves = blockDim.x >> 6;
  const int H = a.H, I = a.I, topk = a.topk;
  const int G = H >> 5;
  const int L = 4 * G;
  const bool active = t < L;
  const int g = t >> 2;
  const int my = a.topk_ids[s];
  const SlotIds ids = load_slot_ids(a.topk_ids, n, a.E);
  if (my < 0 || my >= a.E) return;
  const uint8_t* blk = a.bank + (uint64_t)my * a.expert_bytes;
  uint4 w[4];
  Records<RB> rec;
  Act32 x0;
  // With one token every slot reads the same activation row and an expert
  // repeats only when the caller passes duplicate ids, so the tile and the
  // row are requested before the leader check (which needs all n ids).
  const bool early = (a.M == 1);
  if (early && active) {
    const uint8_t* units = blk + a.w13_off + (uint64_t)nt * 256u * G;
#pragma unroll
    for (int j = 0; j < 4; ++j) w[j] = *reinterpret_cast<const uint4*>(units + ((uint64_t)j * L + t) * 16u);
    rec = load_records<RB>(blk + a.w13_meta_off + (uint64_t)nt * 16u * G * RB + (uint64_t)t * 4u * RB);
    x0 = load_act32(x + 32 * g);
  }
  uint64_t rows[4];
  same_id_masks(ids, my, n, rows);
  {
    uint64_t probe[4] = {rows[0], rows[1], rows[2], rows[3]};
    if (pop_slot(probe) != s) return;  // another slot leads this expert
  }
  if (!early && active) {
    const uint8_t* units = blk + a.w13_off + (uint64_t)nt * 256u * G;
#pragma unroll
    for (int j = 0; j < 4; ++j) w[j] = *reinterpret_cast<const uint4*>(units + ((uint64_t)j * L + t) * 16u);
    rec = load_records<RB>(blk + a.w13_meta_off + (uint64_t)nt * 16u * G * RB + (uint64_t)t * 4u * RB);
  }
  for (;;) {
    int slot[R];
    int rowsn = 0;
#pragma unroll
    for (int rr = 0; rr < R; ++rr) {
      slot[rr] = pop_slot(rows);
      rowsn += slot[rr] >= 0;
    }
    if (rowsn == 0) break;
    float part[R][4];
#pragma unroll
    for (int rr = 0; rr < R; ++rr) {
#pragma unroll
      for (int j = 0; j < 4; ++j) part[rr][j] = 0.f;
      if (active && rr < rowsn) {
        const Act32 av = early ? x0 : load_act32(x + (uint64_t)(slot[rr] / topk) * H + 32 * g);
        float S, Cs;
        group_sums(av, S, Cs);
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const float acc = unit_dot(w[j], av);
          part[rr][j] = rec.s[j] * (acc - fmaf(rec.z[j], S, Cs));
        }
      }
    }
    // Sum over the 16 groups of this wave (lane bits 2..5): lane l ends with
    // column 4*(l & 3) + 2*b4 + b5 of the tile.
#pragma unroll
    for (int rr = 0; rr < R; ++rr) {
      if (rr < rowsn) {
        const float v = sum4_lane_bits_2to5(part[rr][0], part[rr][1], part[rr][2], part[rr][3]);
        if ((lane & 12) == 0) red[wave][rr][4 * (lane & 3) + 2 * ((lane >> 4) & 1) + (lane >> 5)] = v;
      }
    }
    __syncthreads();
    if (t < 16 * R) {  // wave 0 (R <= 4)
      const int col = t & 15, rr = t >> 4;
      float h = 0.f;
      for (int wv = 0; wv < nwaves; ++wv) h += red[wv][rr][col];
      const float other = __shfl_xor(h, 1);  // partner column: gate <-> up
      int sl = -1;
#pragma unroll
      for (int q = 0; q < R; ++q)
        if (q == rr) sl = slot[q];
      if (!(col & 1) && rr < rowsn) {
        const float v = silu_mul(h, other);
        act[(uint64_t)sl * I + nt * 8 + (col >> 1)] = __builtin_bit_cast(uint16_t, (_Float16)v);
      }
    }
    if (rowsn < R) break;
    __syncthreads();
  }
}

// ---------------------------------------------------------------------------
// W2 + router-weighted reduction: grid (H/8 column tiles). One workgroup owns
// 8 output columns for all tokens. It loads the routing plan in one round
// trip; lane groups stream each segment's W2 tile once and apply it to every
// slot of the segment; the K groups of a slot are summed by shuffles into one
// partial per slot; each token then sums its slots' partials in ascending
// expert order (ties by slot), so the result depends only on the set of
// (expert, weight) pairs of the token.
// Lanes: slot group sl (SS of them) x column quad (2) x group gp (GP, the
// power of two >= I/32; lanes with gp >= I/32 idle at the loads).
// ---------------------------------------------------------------------------
template <int RB>
__global__ __launch_bounds__(512) void w2_reduce_kernel(StageArgs a, const uint16_t* __restrict__ act,
                                                        const float* __restrict__ topk_w,
                                                        const Plan* __restrict__ plan, int SS, int GP,
                                                        uint16_t* __restrict__ out) {
  __shared__ int seg_e[kMaxSlots];
  __shared__ int seg_off[kMaxSlots + 1];
  __shared__ int seg_slots[kMaxSlots];
  __shared__ int order[kMaxSlots];
  __shared__ float wts[kMaxSlots];
  __shared__ float ybuf[kMaxSlots][8];
  __shared__ int cnt[AWQ_MOE_KMAX_TOKENS];
  __shared__ int nseg_s;
  const int M = a.M, topk = a.topk, H = a.H, I = a.I;
  const int n = M * topk;
  const int nt = blockIdx.x;
  const int t = threadIdx.x;

  for (int i = t; i < n; i += blockDim.x) {
    seg_e[i] = plan->seg_e[i];
    seg_off[i] = plan->seg_off[i];
    seg_slots[i] = plan->seg_slots[i];
    order[i] = plan->order[i];
    wts[i] = topk_w[i];
  }
  if (t == 0) {
    seg_off[n] = plan->seg_off[n];
    nseg_s = plan->num_segments;
  }
  if (t < M) cnt[t] = plan->cnt[t];
  __syncthreads();

  const int G2 = I >> 5;
  const int L2p = 2 * GP;
  const int sl = t / L2p, tl = t - sl * L2p;
  const int quad = tl / GP, gp = tl - quad * GP;
  const int nseg = nseg_s;
  const bool loader = (sl < SS) && (gp < G2);
  // Segment tiles are software-pipelined: the next segment's W2 tile and first
  // activation row are requested before the current segment is computed.
  const int tli = 2 * gp + quad;  // lane of the bank layout
  auto issue = [&](int seg, uint4 (&w)[4], Records<RB>& rec, Act32& first) {
    const uint8_t* blk = a.bank + (uint64_t)seg_e[seg] * a.expert_bytes;
    const uint8_t* units = blk + a.w2_off + (uint64_t)nt * 128u * G2;
#pragma unroll
    for (int j = 0; j < 4; ++j) w[j] = *reinterpret_cast<const uint4*>(units + ((uint64_t)j * (2 * G2) + tli) * 16u);
    rec = load_records<RB>(blk + a.w2_meta_off + (uint64_t)nt * 8u * G2 * RB + (uint64_t)tli * 4u * RB);
    first = load_act32(act + (uint64_t)seg_slots[seg_off[seg]] * I + 32 * gp);
  };
  if (sl < SS) {
    uint4 w[4], wn[4];
    Records<RB> rec, recn;
    Act32 cur, curn;
    if (loader && sl < nseg) issue(sl, w, rec, cur);
    for (int seg = sl; seg < nseg; seg += SS) {
      const int r_begin = seg_off[seg], r_end = seg_off[seg + 1];
      const bool more = seg + SS < nseg;
      if (loader && more) issue(seg + SS, wn, recn, curn);
      for (int r = r_begin; r < r_end; ++r) {
        const int slot = seg_slots[r];
        if (loader && r > r_begin) cur = load_act32(act + (uint64_t)slot * I + 32 * gp);
        float y[4] = {0.f, 0.f, 0.f, 0.f};
        if (loader) {
          float S, Cs;
          group_sums(cur, S, Cs);
#pragma unroll
          for (int j = 0; j < 4; ++j) y[j] = rec.s[j] * (unit_dot(w[j], cur) - fmaf(rec.z[j], S, Cs));
        }
        if (GP == 8) {
#pragma unroll
          for (int j = 0; j < 4; ++j) y[j] = sum_lane_bits_0to2(y[j]);
        } else {
          for (int o = 1; o < GP; o <<= 1)
#pragma unroll
            for (int j = 0; j < 4; ++j) y[j] += __shfl_xor(y[j], o);
        }
        if (gp == 0) {
#pragma unroll
          for (int j = 0; j < 4; ++j) ybuf[slot][4 * quad + j] = y[j];
        }
      }
      if (more) {
#pragma unroll
        for (int j = 0; j < 4; ++j) w[j] = wn[j];
        rec = recn;
        cur = curn;
      }
    }
  }
  __syncthreads();
  for (int i = t; i < M * 8; i += blockDim.x) {
    const int tt = i >> 3, col = i & 7;
    float v = 0.f;
    const int c = cnt[tt];
    for (int r = 0; r < c; ++r) {
      const int slot = order[tt * topk + r];
      v = fmaf(wts[slot], ybuf[slot][col], v);
    }
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
hipError_t launch_route_compact(const int32_t* ids, int n, int E, const RouteOut& o, hipStream_t stream) {
  hipLaunchKernelGGL(route_compact_kernel, dim3(1), dim3(256), 0, stream, ids, n, E, o);
  return hipGetLastError();
}

hipError_t launch_w13_swiglu(const StageArgs& a, const uint16_t* x, uint16_t* act, Plan* plan, uint32_t* status,
                             hipStream_t stream) {
  const int L = 4 * (a.H / 32);
  const dim3 block(((L + 63) / 64) * 64);
  const dim3 grid((2 * a.I) / 16, 1 + a.M * a.topk);
  if (a.RB == 4)
    hipLaunchKernelGGL(w13_swiglu_kernel<4>, grid, block, 0, stream, a, x, act, plan, status);
  else
    hipLaunchKernelGGL(w13_swiglu_kernel<3>, grid, block, 0, stream, a, x, act, plan, status);
  return hipGetLastError();
}

W2Shape w2_shape(int I, int n) {
  W2Shape sh;
  const int G2 = I / 32;
  sh.GP = 1;
  while (sh.GP < G2) sh.GP <<= 1;
  const int L2p = 2 * sh.GP;
  int ss = 256 / L2p;
  if (ss > 16) ss = 16;
  if (ss > n) ss = n;
  if (ss < 1) ss = 1;
  sh.SS = ss;
  sh.threads = ((ss * L2p + 63) / 64) * 64;
  return sh;
}

hipError_t launch_w2_reduce(const StageArgs& a, const uint16_t* act, const float* topk_w, const Plan* plan,
                            uint16_t* out, hipStream_t stream) {
  const W2Shape sh = w2_shape(a.I, a.M * a.topk);
  const dim3 block(sh.threads);
  const dim3 grid(a.H / 8);
  if (a.RB == 4)
    hipLaunchKernelGGL(w2_reduce_kernel<4>, grid, block, 0, stream, a, act, topk_w, plan, sh.SS, sh.GP, out);
  else
    hipLaunchKernelGGL(w2_reduce_kernel<3>, grid, block, 0, stream, a, act, topk_w, plan, sh.SS, sh.GP, out);
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
