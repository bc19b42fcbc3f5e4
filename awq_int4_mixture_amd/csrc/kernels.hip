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

#include <atomic>
#include <mutex>

#include "device_util.h"
#include "kernels.h"

namespace awq_moe {

typedef uint32_t u32x3_a4 __attribute__((ext_vector_type(3), aligned(4)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));

// Weight units (16 or 8 bytes). STREAM marks the load non-temporal: the
// bytes are read once per call, so the caches need not keep them. Measured
// on cold weights (µs per launch, M = 1 / M = 8 with 80 distinct experts):
// W13 3.78 -> 3.53 / 9.6 -> 8.6, W2 3.61 -> 3.43 / 6.41 -> 6.00. Where slots
// share experts and the grid runs in several rounds (the indexed prefill's
// small calls), a later slot's read of the same tile then misses, and W13
// is slower (64 tokens: 69.5 -> 76.6 per call); there W13 keeps plain loads.
template <bool STREAM>
__device__ __forceinline__ uint4 load_unit16(const uint8_t* p) {
  if constexpr (STREAM) {
    const u32x4_t v = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(p));
    return make_uint4(v.x, v.y, v.z, v.w);
  } else {
    return *reinterpret_cast<const uint4*>(p);
  }
}
template <bool STREAM>
__device__ __forceinline__ uint2 load_unit8(const uint8_t* p) {
  if constexpr (STREAM) {
    const u32x2_t v = __builtin_nontemporal_load(reinterpret_cast<const u32x2_t*>(p));
    return make_uint2(v.x, v.y);
  } else {
    return *reinterpret_cast<const uint2*>(p);
  }
}

// Bit pattern constants of the nibble -> fp16 conversion.
constexpr uint32_t kLoMask = 0x000F000Fu;   // values at bits 0 and 16
constexpr uint32_t kHiMask = 0x00F000F0u;   // values at bits 4 and 20

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

// A lane's four records as loaded (one 16- or 12-byte load), decoded only
// where they are used, so that the wait for them can come late.
template <int RB>
struct RawRecords {
  uint32_t d[RB];
};

template <int RB>
__device__ __forceinline__ RawRecords<RB> load_records_raw(const uint8_t* p) {
  RawRecords<RB> r;
  if constexpr (RB == 4) {
    const uint4 v = *reinterpret_cast<const uint4*>(p);
    r.d[0] = v.x; r.d[1] = v.y; r.d[2] = v.z; r.d[3] = v.w;
  } else {
    const u32x3_a4 v = *reinterpret_cast<const u32x3_a4*>(p);
    r.d[0] = v.x; r.d[1] = v.y; r.d[2] = v.z;
  }
  return r;
}

template <int RB>
__device__ __forceinline__ Records<RB> decode_records(const RawRecords<RB>& v) {
  Records<RB> out;
  uint32_t r[4];
  if constexpr (RB == 4) {
    r[0] = v.d[0]; r[1] = v.d[1]; r[2] = v.d[2]; r[3] = v.d[3];
  } else {
    r[0] = v.d[0];
    r[1] = __builtin_amdgcn_alignbyte(v.d[1], v.d[0], 3);
    r[2] = __builtin_amdgcn_alignbyte(v.d[2], v.d[1], 2);
    r[3] = v.d[2] >> 8;
  }
#pragma unroll
  for (int j = 0; j < 4; ++j) decode_record(r[j], out.s[j], out.z[j]);
  return out;
}

template <int RB>
__device__ __forceinline__ Records<RB> load_records(const uint8_t* p) {
  return decode_records<RB>(load_records_raw<RB>(p));
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

// The same 32 values for a quad of lanes (4 adjacent lanes, one group): lane
// q of the quad loads quarter q (16 bytes) and DPP quad broadcasts hand every
// lane all four quarters, so the quad issues one load per lane instead of four.
// All four lanes of the quad must be active.
template <int Q>
__device__ __forceinline__ uint32_t quad_bcast(uint32_t v) {
  return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, Q | (Q << 2) | (Q << 4) | (Q << 6), 0xF, 0xF, false);
}

__device__ __forceinline__ Act32 load_act32_quad(const uint16_t* p, int quad) {
  const uint4 v = *reinterpret_cast<const uint4*>(p + 8 * quad);
  Act32 a;
  a.px[0] = quad_bcast<0>(v.x); a.px[1] = quad_bcast<0>(v.y); a.px[2] = quad_bcast<0>(v.z); a.px[3] = quad_bcast<0>(v.w);
  a.px[4] = quad_bcast<1>(v.x); a.px[5] = quad_bcast<1>(v.y); a.px[6] = quad_bcast<1>(v.z); a.px[7] = quad_bcast<1>(v.w);
  a.px[8] = quad_bcast<2>(v.x); a.px[9] = quad_bcast<2>(v.y); a.px[10] = quad_bcast<2>(v.z); a.px[11] = quad_bcast<2>(v.w);
  a.px[12] = quad_bcast<3>(v.x); a.px[13] = quad_bcast<3>(v.y); a.px[14] = quad_bcast<3>(v.z); a.px[15] = quad_bcast<3>(v.w);
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

// The two exponent patterns live in VGPRs: with the masks in SGPRs each
// (v & mask) | magic is then a single v_and_or_b32 (a VOP3 instruction here
// takes at most one scalar operand and no literal).
struct Magic {
  uint32_t m1024, m64;
};

// 0x6400 is fp16 1024.0 (mantissa ulp 1: a value at bits 0..3 adds itself);
// 0x5400 is fp16 64.0 (ulp 1/16: a value at bits 4..7 adds itself).
__device__ __forceinline__ Magic make_magic() {
  Magic m;
  asm volatile("v_mov_b32 %0, 0x64006400" : "=v"(m.m1024));
  asm volatile("v_mov_b32 %0, 0x54005400" : "=v"(m.m64));
  return m;
}

// acc = sum_k x_k * (offset_k + q_k) over one unit (4 dwords = 32 values).
__device__ __forceinline__ float unit_dot(const uint4& w, const Act32& a, const Magic& mg) {
  float acc = 0.f;
  const uint32_t wd[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
  for (int d = 0; d < 4; ++d) {
    const uint32_t v = wd[d];
    const uint32_t v8 = v >> 8;
    acc = dot2(a.px[4 * d + 0], (v & kLoMask) | mg.m1024, acc);
    acc = dot2(a.px[4 * d + 1], (v & kHiMask) | mg.m64, acc);
    acc = dot2(a.px[4 * d + 2], (v8 & kLoMask) | mg.m1024, acc);
    acc = dot2(a.px[4 * d + 3], (v8 & kHiMask) | mg.m64, acc);
  }
  return acc;
}

// silu(g) * u = g / (1 + e^-g) * u. The division is the hardware reciprocal
// (about 1 ulp of fp32, far below the fp16 rounding of the result): it is
// the last step before each workgroup's store, and the IEEE division there
// measured 0.02-0.05 us per W13 launch.
__device__ __forceinline__ float silu_mul(float g, float u) {
  return g * __builtin_amdgcn_rcpf(1.0f + __expf(-g)) * u;
}

// ---------------------------------------------------------------------------
// routing compaction of n <= 256 slots inside one workgroup (LDS only).
// Canonical order: experts ascending, rows of a segment by ascending slot,
// invalid slots (ids outside [0, E)) after all valid ones in slot order.
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

// Sum over the 4 lanes of a quad (DPP quad permutes); every lane gets the sum.
__device__ __forceinline__ int quad_sum(int v) {
  v += __builtin_amdgcn_update_dpp(0, v, 0xB1, 0xF, 0xF, false);  // quad_perm [1,0,3,2]
  v += __builtin_amdgcn_update_dpp(0, v, 0x4E, 0xF, 0xF, false);  // quad_perm [2,3,0,1]
  return v;
}

// Each slot's comparisons against all n keys are split over the 4 lanes of
// a quad (lane p takes every 4th group of four keys), and the counts are
// summed with quad permutes. blockDim is a multiple of 64 and at least 4n.
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
  const int p = t & 3;
  const int s = t >> 2;  // every lane of a quad has the same slot
  {
    const int id = s < n ? C.key[s] : -2;
    int before = 0, inv_before = 0, nvalid = 0, dup_before = 0;
    for (int s2 = 4 * p; s2 < n4; s2 += 16) {
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
    before = quad_sum(before);
    inv_before = quad_sum(inv_before);
    nvalid = quad_sum(nvalid);
    dup_before = quad_sum(dup_before);
    if (s < n && p == 0) {
      const int r = (id >= 0) ? before : nvalid + inv_before;
      C.rank[s] = r;
      C.sorted[r] = s;
      if (id >= 0 && dup_before == 0) C.firstkey[s] = id;
      if (s == 0) C.nvalid = nvalid;
    }
  }
  __syncthreads();
  {
    const int fk = s < n ? C.firstkey[s] : kNoKey;
    int below = 0, nseg = 0;
    for (int s2 = 4 * p; s2 < n4; s2 += 16) {
      const int4 f4 = *reinterpret_cast<const int4*>(&C.firstkey[s2]);
      const int ff[4] = {f4.x, f4.y, f4.z, f4.w};
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        below += ff[q] < fk;
        nseg += ff[q] != kNoKey;
      }
    }
    below = quad_sum(below);
    nseg = quad_sum(nseg);
    if (s < n && p == 0) {
      if (fk != kNoKey) {
        C.seg_e[below] = fk;
        C.seg_off[below] = C.rank[s];
      }
      if (s == 0) {
        C.num_active = nseg;
        C.seg_off[nseg] = C.nvalid;
      }
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

__global__ __launch_bounds__(1024) void route_compact_kernel(const int32_t* __restrict__ ids, int n, int E,
                                                            RouteOut o) {
  __shared__ Compact C;
  block_compact(ids, n, E, C);
  store_route(C, n, o);
}

// ---------------------------------------------------------------------------
// Shape word of the decode kernels: G = H/32 in bits 0..8, G2 = I/32 in bits
// 9..15, topk in bits 16..21, M in bits 22..27. Together with 32-bit expert
// strides it keeps every argument a kernel needs before its first weight
// load inside the 14 dwords that arrive preloaded in SGPRs, so no wave waits
// on a kernel-argument load.
// ---------------------------------------------------------------------------
__host__ __device__ constexpr uint32_t pack_dims(int H, int I, int topk, int M) {
  return (uint32_t)(H >> 5) | ((uint32_t)(I >> 5) << 9) | ((uint32_t)topk << 16) | ((uint32_t)M << 22);
}
__host__ __device__ __forceinline__ int dims_G(uint32_t d) { return (int)(d & 0x1FFu); }
__host__ __device__ __forceinline__ int dims_G2(uint32_t d) { return (int)((d >> 9) & 0x7Fu); }
__host__ __device__ __forceinline__ int dims_topk(uint32_t d) { return (int)((d >> 16) & 0x3Fu); }
__host__ __device__ __forceinline__ int dims_M(uint32_t d) { return (int)((d >> 22) & 0x3Fu); }

// The bank layout of one expert block, from the shape word and the record
// size (the sections of the layout: W13 units, W13 records, W2 units, W2
// records, each padded to 256 bytes). Unit sections are multiples of 256
// already (1024 G G2 and 512 G G2 bytes). Kernels that compute it keep two
// argument registers free; the launcher checks it against the host layout.
struct ExpertGeometry {
  uint32_t expert_bytes, w2_off, w2_meta_delta;
};

template <int RB>
__host__ __device__ __forceinline__ ExpertGeometry expert_geometry(uint32_t d) {
  const uint32_t G = (uint32_t)dims_G(d), G2 = (uint32_t)dims_G2(d);
  const uint32_t w13_units = 1024u * G * G2, w13_meta = 64u * G * G2 * RB;
  const uint32_t w2_units = 512u * G * G2, w2_meta = 32u * G * G2 * RB;
  ExpertGeometry g;
  g.w2_off = w13_units + ((w13_meta + 255u) & ~255u);
  g.w2_meta_delta = w2_units;
  g.expert_bytes = g.w2_off + w2_units + ((w2_meta + 255u) & ~255u);
  return g;
}

// Sum of squares of the activations a lane holds (packed fp16 pairs), for the
// in-kernel RMS norm: v_dot2 of each pair with itself (products exact in
// fp32).
template <int NP>
__device__ __forceinline__ float pairs_sumsq(const uint32_t* px) {
  float ss = 0.f;
#pragma unroll
  for (int i = 0; i < NP; ++i) ss = dot2(px[i], px[i], ss);
  return ss;
}

// ---------------------------------------------------------------------------
// W13 + SwiGLU: grid (2I/16 column tiles, n slots), ceil(H/8 / 64) waves.
// The workgroup of slot s reads its expert id with one scalar load; its
// token's activations are requested before that load returns, and the
// expert's 16-column tile (all of K) right after it, so the slot's chain is
// two memory round trips. It then writes act[s] for that tile. Slots that
// share an expert read the same tile within the same few hundred
// nanoseconds: a later read hits the L2 when it runs on the same XCD and
// otherwise goes to the MALL or HBM (with 8 tokens drawing from shared
// pools, about 1.4 times the distinct bytes are fetched), which still
// measured faster than first electing one workgroup per expert from the
// routed ids.
// The workspace holds the status word at offset 0 and act at offset 256.
// Wave 0 of workgroup (0, 0) also writes the status word; its id loads are
// issued first and consumed after the weight loads are in flight.
// ---------------------------------------------------------------------------
// With NORM, x is a residual row r and the stage consumes r / rms(r), rms(r)
// = sqrt(mean(r^2) + eps): the dot products run on r itself and each
// column's fp32 sum is multiplied by 1/rms(r) before SwiGLU (the norm is a
// per-row scale, so nothing is rounded in between). The sum of squares comes
// from the row every workgroup of the token loads anyway: each wave sums its
// lanes' squares (every group is held by the 4 lanes of a quad, so the
// wave's sum is exactly 4 times the sum over its groups), the waves' sums
// go through LDS with the column sums, and the one barrier serves both.
// With TPB = 2 a workgroup takes two adjacent tiles of the slot (grid.x =
// 2I/32), each on its own ceil(L/64) waves: one id load and one workgroup
// per pair of tiles (a tactic for larger grids). STREAM: non-temporal weight
// loads (load_unit16).
// 1/rms(r) from ss = 4 * sum(r^2) over the row (every value counted by the
// four lanes of its quad): the hardware reciprocal and reciprocal square
// root (about 1 ulp each) instead of an IEEE division and square root. The
// step runs after the workgroup's last barrier, on the critical path of
// every workgroup, where the IEEE sequence measured about 0.3 us per launch
// at 8 tokens x 10 experts (hidden 2560, inter 160).
__device__ __forceinline__ float inv_rms(float ss, int H, float eps) {
  return __builtin_amdgcn_rsqf(fmaf(ss, __builtin_amdgcn_rcpf((float)(4 * H)), eps));
}

template <int RB, bool NORM, int TPB, bool STREAM>
__global__ __launch_bounds__(1024) void w13_swiglu_kernel(const int32_t* __restrict__ ids,
                                                          const uint8_t* __restrict__ units_base,
                                                          const uint16_t* __restrict__ x, uint8_t* __restrict__ ws,
                                                          uint32_t expert_bytes, uint32_t meta_delta, uint32_t dims,
                                                          int E, float eps) {
  static_assert(TPB == 1 || TPB == 2, "one or two tiles per workgroup");
  __shared__ float red[16][16];  // [wave][column]
  const int s = blockIdx.y;
  const int e = ids[s];  // scalar load
  const int G = dims_G(dims), I = 32 * dims_G2(dims), topk = dims_topk(dims);
  const int H = 32 * G, L = 4 * G, nwaves = (L + 63) >> 6;  // waves per tile
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
  const int tile_i = (TPB == 2 && wave >= nwaves) ? 1 : 0;
  const int nt = blockIdx.x * TPB + tile_i;
  const int t = threadIdx.x - tile_i * 64 * nwaves;  // lane index within the tile
  const bool status_wave = blockIdx.x == 0 && s == 0 && wave == 0;
  const int n = topk * dims_M(dims);  // the first 256 slots four per lane of one wave, then the rest
  int sid[4];
  if (status_wave) {
#pragma unroll
    for (int q = 0; q < 4; ++q) sid[q] = lane + 64 * q < n ? ids[lane + 64 * q] : 0;
  }
  // Every load below is issued by every lane (lanes past L and invalid
  // slots read valid addresses they do not use), so the code is
  // straight-line and each wait covers exactly the loads its use needs.
  const int tc = t < L ? t : 0;
  Act32 av = load_act32(x + (uint64_t)(s / topk) * H + 32 * (tc >> 2));
  // the activations are requested before the wait for the id
  __builtin_amdgcn_sched_barrier(0);
  const bool live = e >= 0 && e < E;
  const uint64_t eo = (uint64_t)(uint32_t)(live ? e : 0) * expert_bytes;
  const uint8_t* units = units_base + eo + (uint64_t)nt * 256u * G;
  const RawRecords<RB> rraw =
      load_records_raw<RB>(units_base + eo + meta_delta + (uint64_t)nt * 16u * G * RB + (uint64_t)tc * 4u * RB);
  uint4 w[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) w[j] = load_unit16<STREAM>(units + ((uint64_t)j * L + tc) * 16u);
  if (status_wave) {
    bool bad = false;
#pragma unroll
    for (int q = 0; q < 4; ++q) bad |= lane + 64 * q < n && (sid[q] < 0 || sid[q] >= E);
    for (int b0 = 256; b0 < n; b0 += 64) {  // more than 256 slots (calls of the indexed prefill)
      const int id = b0 + lane < n ? ids[b0 + lane] : 0;
      bad |= id < 0 || id >= E;
    }
    const unsigned long long b = __ballot(bad);
    if (lane == 0) *reinterpret_cast<uint32_t*>(ws + AWQ_MOE_KWS_STATUS_OFFSET) = b ? AWQ_MOE_STATUS_BAD_ID_BIT : 0u;
  }
  if (!live) return;  // invalid slot: no row (uniform over the workgroup)
  __shared__ float norm_part[16];  // [wave] sums of squares (NORM)
  if constexpr (NORM) {
    const float ss = wave_sum_xor_order(t < L ? pairs_sumsq<16>(av.px) : 0.f);
    if (lane == 0) norm_part[wave] = ss;
  }
  float part[4] = {0.f, 0.f, 0.f, 0.f};
  if (t < L) {
    float S, Cs;
    group_sums(av, S, Cs);
    const Records<RB> rec = decode_records<RB>(rraw);
    const Magic mg = make_magic();
#pragma unroll
    for (int j = 0; j < 4; ++j) part[j] = rec.s[j] * (unit_dot(w[j], av, mg) - fmaf(rec.z[j], S, Cs));
  }
  // Sum over the 16 groups of this wave (lane bits 2..5): lane l ends with
  // column 4*(l & 3) + 2*b4 + b5 of the tile.
  const float v = sum4_lane_bits_2to5(part[0], part[1], part[2], part[3]);
  if ((lane & 12) == 0) red[wave][4 * (lane & 3) + 2 * ((lane >> 4) & 1) + (lane >> 5)] = v;
  __syncthreads();
  if (threadIdx.x < 16 * TPB) {
    const int ti = threadIdx.x >> 4, c = threadIdx.x & 15;  // tile of the workgroup, column
    const int w0 = ti * nwaves;
    float h = 0.f, ss = 0.f;
    for (int wv = w0; wv < w0 + nwaves; ++wv) {
      h += red[wv][c];
      if constexpr (NORM) ss += norm_part[wv];
    }
    if constexpr (NORM) h *= inv_rms(ss, H, eps);
    const float other = __shfl_xor(h, 1);  // partner column: gate <-> up
    uint16_t* act = reinterpret_cast<uint16_t*>(ws + AWQ_MOE_KWS_ACT_OFFSET);
    if (!(c & 1))
      act[(uint64_t)s * I + (blockIdx.x * TPB + ti) * 8 + (c >> 1)] =
          __builtin_bit_cast(uint16_t, (_Float16)silu_mul(h, other));
  }
}

// ---------------------------------------------------------------------------
// W13 + SwiGLU with each 32-value group split over a lane pair: the same
// work as w13_swiglu_kernel on twice the lanes (ceil(H/4 / 64) waves, 10 at
// H = 2560), each with half of every unit (an 8-byte load per column) and
// half of the group's activations. With 5 waves a lone workgroup leaves one
// SIMD of its CU with two waves' arithmetic; with 10 the busiest SIMD has
// three half-waves' worth. Used when the grid has at most one workgroup per
// CU (M = 1 at the rank shape: 3.68 -> 3.53 us on cold weights). Lane bits: 0 = half, 1..2 = quad, 3..5 = group
// within the wave. The pair's and the wave's partial sums are combined by a
// reduce-scatter over lane bits 0 and 3 and sums over bits 4 and 5, in a
// fixed order, then the waves' sums in LDS in wave order.
// ---------------------------------------------------------------------------
// 16 fp16 activations of half a group as 8 packed pairs: px[4d + p] holds
// (x[8d + 2p], x[8d + 2p + 1]) of the half's dword d (0, 1).
struct Act16 {
  uint32_t px[8];
};

__device__ __forceinline__ Act16 load_act16(const uint16_t* p) {
  Act16 a;
  const uint4* q = reinterpret_cast<const uint4*>(p);
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const uint4 v = q[i];
    a.px[4 * i + 0] = v.x; a.px[4 * i + 1] = v.y; a.px[4 * i + 2] = v.z; a.px[4 * i + 3] = v.w;
  }
  return a;
}

// S and C of group_sums over the half's 16 values.
__device__ __forceinline__ void half_group_sums(const Act16& a, float& S, float& C) {
  const uint32_t one2 = 0x3C003C00u;  // fp16 (1.0, 1.0)
  float s1024 = 0.f, s64 = 0.f;
#pragma unroll
  for (int d = 0; d < 2; ++d) {
    s1024 = dot2(a.px[4 * d + 0], one2, s1024);
    s64 = dot2(a.px[4 * d + 1], one2, s64);
    s1024 = dot2(a.px[4 * d + 2], one2, s1024);
    s64 = dot2(a.px[4 * d + 3], one2, s64);
  }
  S = s1024 + s64;
  C = fmaf(1024.f, s1024, 64.f * s64);
}

// unit_dot over the half's two dwords.
__device__ __forceinline__ float half_unit_dot(const uint2& w, const Act16& a, const Magic& mg) {
  float acc = 0.f;
  const uint32_t wd[2] = {w.x, w.y};
#pragma unroll
  for (int d = 0; d < 2; ++d) {
    const uint32_t v = wd[d];
    const uint32_t v8 = v >> 8;
    acc = dot2(a.px[4 * d + 0], (v & kLoMask) | mg.m1024, acc);
    acc = dot2(a.px[4 * d + 1], (v & kHiMask) | mg.m64, acc);
    acc = dot2(a.px[4 * d + 2], (v8 & kLoMask) | mg.m1024, acc);
    acc = dot2(a.px[4 * d + 3], (v8 & kHiMask) | mg.m64, acc);
  }
  return acc;
}

// With NORM, as w13_swiglu_kernel (each half group is held by the 4 lanes of
// its quad, so a wave's sum of squares is again exactly 4 times its groups').
template <int RB, bool NORM>
__global__ __launch_bounds__(1024) void w13_swiglu_pair_kernel(const int32_t* __restrict__ ids,
                                                               const uint8_t* __restrict__ units_base,
                                                               const uint16_t* __restrict__ x, uint8_t* __restrict__ ws,
                                                               uint32_t expert_bytes, uint32_t meta_delta,
                                                               uint32_t dims, int E, float eps) {
  __shared__ float red[16][16];  // [wave][column]
  const int nt = blockIdx.x, s = blockIdx.y;
  const int e = ids[s];  // scalar load
  const int G = dims_G(dims), I = 32 * dims_G2(dims), topk = dims_topk(dims);
  const int H = 32 * G, L = 4 * G, nwaves = (2 * L + 63) >> 6;
  const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
  const int tu = t >> 1, hf = t & 1;  // unit lane (4g + quad) and half
  const bool status_wave = nt == 0 && s == 0 && wave == 0;
  const int n = topk * dims_M(dims);  // the first 256 slots four per lane of one wave, then the rest
  int sid[4];
  if (status_wave) {
#pragma unroll
    for (int q = 0; q < 4; ++q) sid[q] = lane + 64 * q < n ? ids[lane + 64 * q] : 0;
  }
  // Every load below is issued by every lane (see w13_swiglu_kernel).
  const int tuc = tu < L ? tu : 0;
  Act16 av = load_act16(x + (uint64_t)(s / topk) * H + 32 * (tuc >> 2) + 16 * hf);
  // the activations are requested before the wait for the id
  __builtin_amdgcn_sched_barrier(0);
  const bool live = e >= 0 && e < E;
  const uint64_t eo = (uint64_t)(uint32_t)(live ? e : 0) * expert_bytes;
  const uint8_t* units = units_base + eo + (uint64_t)nt * 256u * G + 8u * hf;
  const RawRecords<RB> rraw =
      load_records_raw<RB>(units_base + eo + meta_delta + (uint64_t)nt * 16u * G * RB + (uint64_t)tuc * 4u * RB);
  uint2 w[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) w[j] = load_unit8<true>(units + ((uint64_t)j * L + tuc) * 16u);
  if (status_wave) {
    bool bad = false;
#pragma unroll
    for (int q = 0; q < 4; ++q) bad |= lane + 64 * q < n && (sid[q] < 0 || sid[q] >= E);
    for (int b0 = 256; b0 < n; b0 += 64) {  // more than 256 slots (calls of the indexed prefill)
      const int id = b0 + lane < n ? ids[b0 + lane] : 0;
      bad |= id < 0 || id >= E;
    }
    const unsigned long long b = __ballot(bad);
    if (lane == 0) *reinterpret_cast<uint32_t*>(ws + AWQ_MOE_KWS_STATUS_OFFSET) = b ? AWQ_MOE_STATUS_BAD_ID_BIT : 0u;
  }
  if (!live) return;  // invalid slot: no row (uniform over the workgroup)
  __shared__ float norm_part[16];  // [wave] sums of squares (NORM)
  if constexpr (NORM) {
    const float ss = wave_sum_xor_order(tu < L ? pairs_sumsq<8>(av.px) : 0.f);
    if (lane == 0) norm_part[wave] = ss;
  }
  float p0 = 0.f, p1 = 0.f, p2 = 0.f, p3 = 0.f;
  if (tu < L) {
    float S, Cs;
    half_group_sums(av, S, Cs);
    const Records<RB> rec = decode_records<RB>(rraw);
    const Magic mg = make_magic();
    p0 = rec.s[0] * (half_unit_dot(w[0], av, mg) - fmaf(rec.z[0], S, Cs));
    p1 = rec.s[1] * (half_unit_dot(w[1], av, mg) - fmaf(rec.z[1], S, Cs));
    p2 = rec.s[2] * (half_unit_dot(w[2], av, mg) - fmaf(rec.z[2], S, Cs));
    p3 = rec.s[3] * (half_unit_dot(w[3], av, mg) - fmaf(rec.z[3], S, Cs));
  }
  // reduce-scatter over lane bit 0 (the pair): bit 0 keeps columns j = 2 b0, 2 b0 + 1
  const bool b0 = lane & 1, b3 = (lane >> 3) & 1;
  const float ka = (b0 ? p2 : p0) + dpp<kQuadSwap1>(b0 ? p0 : p2);
  const float kb = (b0 ? p3 : p1) + dpp<kQuadSwap1>(b0 ? p1 : p3);
  // over lane bit 3: keeps column j = 2 b0 + b3
  float k = (b3 ? kb : ka) + dpp<kRowRor8>(b3 ? ka : kb);
  // over lane bits 4 and 5
  k += __shfl_xor(k, 16);
  k += __shfl_xor(k, 32);
  if (lane < 16) red[wave][4 * ((lane >> 1) & 3) + 2 * (int)b0 + (int)b3] = k;
  __syncthreads();
  if (t < 16) {
    float h = 0.f, ss = 0.f;
    for (int wv = 0; wv < nwaves; ++wv) {
      h += red[wv][t];
      if constexpr (NORM) ss += norm_part[wv];
    }
    if constexpr (NORM) h *= inv_rms(ss, H, eps);
    const float other = __shfl_xor(h, 1);  // partner column: gate <-> up
    uint16_t* act = reinterpret_cast<uint16_t*>(ws + AWQ_MOE_KWS_ACT_OFFSET);
    if (!(t & 1)) act[(uint64_t)s * I + nt * 8 + (t >> 1)] = __builtin_bit_cast(uint16_t, (_Float16)silu_mul(h, other));
  }
}

// ---------------------------------------------------------------------------
// W2 + router-weighted reduction: grid (H/(16*TPW) column groups, M tokens).
// The workgroup of (group, token) streams TPW adjacent 16-column W2 tiles
// (one contiguous run per expert, all of K = I) of each of the token's
// routed experts and sums the slots in LDS, so no partial result crosses
// workgroups and no workspace is written.
// Lanes: u = slot*(TPW*LS) + tile*LS + t with LS = 4*G2 lanes per tile and
// t = 4g + quad as in the layout; slots beyond what one block holds are
// taken in passes. Slot order of the final sum: ascending (expert, slot)
// over the valid slots, so the result depends only on the set of
// (expert, weight) pairs and not on the order of the token's top-k list.
// Wave 0 ranks the slots with lane shuffles while the weight loads are in
// flight.
// ---------------------------------------------------------------------------
// With RES, out receives fp16(resid + fp16(result)) (the residual update of
// a stacked layer) instead of fp16(result).
template <int RB, int TPW, bool RES>
__global__ __launch_bounds__(1024) void w2_reduce_kernel(const int32_t* __restrict__ topk_ids,
                                                         const uint8_t* __restrict__ units_base,
                                                         const uint8_t* __restrict__ recs_base,
                                                         const uint16_t* __restrict__ act, uint64_t expert_bytes, int H,
                                                         int I, int topk, int E, const float* __restrict__ topk_w,
                                                         uint16_t* __restrict__ out, const uint16_t* __restrict__ resid) {
  constexpr int NC = 16 * TPW;                     // columns per workgroup
  __shared__ float red[4096];                      // [slot in pass][tile][g][16]; <= 4*blockDim
  __shared__ float ys[AWQ_MOE_KMAX_TOPK * NC];     // [rank][NC]: a valid slot's column results
  __shared__ int rk[AWQ_MOE_KMAX_TOPK];            // slot -> rank (-1: invalid slot)
  __shared__ float wr[AWQ_MOE_KMAX_TOPK];          // rank -> router weight
  __shared__ int nvalid_s;
  // Workgroups are handed to the 8 XCDs round robin by linear id, so with
  // the group count a multiple of 8 the x index bx runs on XCD bx % 8 for
  // every token. Give each XCD a contiguous run of groups: the record runs
  // of neighbouring tiles share cache lines, which are then fetched into
  // one L2 only.
  const int NG = H / NC;
  const int grp = (NG & 7) ? (int)blockIdx.x : (int)((blockIdx.x & 7) * (NG >> 3) + (blockIdx.x >> 3));
  const int nt0 = grp * TPW;
  const int tok = blockIdx.y;
  const int t = threadIdx.x;
  const int G2 = I >> 5, LS = 4 * G2, LSW = TPW * LS;
  const int spp = blockDim.x / LSW;                // slots per pass (>= 1)
  const int32_t* ids = topk_ids + tok * topk;
  for (int s0 = 0; s0 < topk; s0 += spp) {
    const int sp = t / LSW, rem = t - sp * LSW;
    const int tt = TPW == 1 ? 0 : rem / LS, tl = rem - tt * LS;
    const int slot = s0 + sp;
    const bool lane_on = sp < spp && slot < topk;
    const int e = lane_on ? ids[slot] : -1;
    const bool live = lane_on && e >= 0 && e < E;
    uint4 w[4];
    Records<RB> rec;
    Act32 av;
    const int g = tl >> 2, quad = tl & 3;
    if (live) {
      const uint64_t eo = (uint64_t)e * expert_bytes;
      const uint8_t* units = units_base + eo + (uint64_t)(nt0 + tt) * 256u * G2;
#pragma unroll
      for (int j = 0; j < 4; ++j) w[j] = *reinterpret_cast<const uint4*>(units + ((uint64_t)j * LS + tl) * 16u);
      rec = load_records<RB>(recs_base + eo + (uint64_t)(nt0 + tt) * 16u * G2 * RB + (uint64_t)tl * 4u * RB);
      av = load_act32_quad(act + (uint64_t)(tok * topk + slot) * I + 32 * g, quad);
    }
    if (s0 == 0 && t < 64) {
      const int id = t < topk ? ids[t] : -1;
      const float wt = t < topk ? topk_w[tok * topk + t] : 0.f;
      const bool v = t < topk && id >= 0 && id < E;
      int r = 0;
      for (int j2 = 0; j2 < topk; ++j2) {
        const int k2 = __builtin_amdgcn_readlane(id, j2);
        r += (k2 >= 0 && k2 < E) & ((k2 < id) | ((k2 == id) & (j2 < t)));
      }
      if (t < topk) rk[t] = v ? r : -1;
      if (v) wr[r] = wt;
      const unsigned long long b = __ballot(v);
      if (t == 0) nvalid_s = (int)__popcll(b);
    }
    if (live) {
      float S, Cs;
      group_sums(av, S, Cs);
      const Magic mg = make_magic();
#pragma unroll
      for (int j = 0; j < 4; ++j)
        red[((sp * TPW + tt) * G2 + g) * 16 + 4 * quad + j] =
            rec.s[j] * (unit_dot(w[j], av, mg) - fmaf(rec.z[j], S, Cs));
    }
    __syncthreads();
    // per-slot column results of this pass, groups summed in ascending g,
    // stored at the slot's rank (invalid slots are skipped)
    for (int u = t; u < spp * NC; u += blockDim.x) {
      const int ps = u / NC, cc = u - ps * NC;
      const int t2 = cc >> 4, c = cc & 15;
      const int r = s0 + ps < topk ? rk[s0 + ps] : -1;
      if (r >= 0) {
        float y = 0.f;
        for (int gg = 0; gg < G2; ++gg) y += red[((ps * TPW + t2) * G2 + gg) * 16 + c];
        ys[r * NC + cc] = y;
      }
    }
    __syncthreads();
  }
  if (t < NC) {
    const int nv = nvalid_s;
    float acc = 0.f;
#pragma unroll 4
    for (int rr = 0; rr < nv; ++rr) acc = fmaf(wr[rr], ys[rr * NC + t], acc);
    const uint64_t o = (uint64_t)tok * H + nt0 * 16 + t;
    _Float16 v = (_Float16)acc;
    if constexpr (RES) v = (_Float16)((float)__builtin_bit_cast(_Float16, resid[o]) + (float)v);
    out[o] = __builtin_bit_cast(uint16_t, v);
  }
}

// ---------------------------------------------------------------------------
// W2 + router-weighted reduction for I <= 512: grid (H/16 tiles, M tokens)
// as above. A slot owns LS = 4*I/32 <= 64 adjacent lanes of a wave (lane =
// 4g + quad inside its segment), and a wave holds SPW = floor(64 / LS)
// slots, so a token's slots take ceil(topk / SPW) waves (at most 16): 4 at
// I = 160 and top-k 10, one per SIMD of the CU (with 5 waves one SIMD runs
// two, and at M = 1, one workgroup per CU, that SIMD sets the kernel's
// time); one slot per wave from I = 288 (LS > 32).
// The wave's ids and router weights arrive as scalar loads; the token's
// ids (for the ranking) and the activations are requested before they
// return, and every load is unconditional with clamped indexes, so the
// code is straight-line and each value is waited for just before its first
// use (exec-masked loads measured slower: the waits after the branch cover
// all of them). Each wave ranks its own slots by (id, slot) with one ballot
// per slot while its weights are in flight and keeps the ranks in SGPRs.
// A slot's groups are summed in ascending g through the wave's own LDS
// rows (no barrier: a wave's LDS operations complete in order), and the
// slot's 16 column results go to LDS at its rank; one barrier, then the
// router-weighted sum in ascending (expert, slot) order.
// ---------------------------------------------------------------------------
// With RES, out receives fp16(resid + fp16(result)) (the residual update of
// a stacked layer); resid's value is requested at the start, off the id
// chain. The expert stride and record offset come from the shape word
// (expert_geometry), which keeps resid within the preloaded argument
// registers.
template <int RB, int SPW, bool RES>
__global__ __launch_bounds__(1024) void w2_reduce_seg_kernel(const int32_t* __restrict__ topk_ids,
                                                             const uint8_t* __restrict__ units_base,
                                                             const uint16_t* __restrict__ act,
                                                             const float* __restrict__ topk_w,
                                                             uint16_t* __restrict__ out, uint32_t dims, int E,
                                                             const uint16_t* __restrict__ resid) {
  // [slot][g][16]: up to 8 groups of 32 slots, or with one slot per wave
  // (at most 16 waves) up to 16 groups of 16 slots
  constexpr int kG2Max = SPW == 1 ? 16 : 8;
  constexpr int kSlots = SPW == 1 ? 16 : AWQ_MOE_KMAX_TOPK;
  __shared__ __attribute__((aligned(16))) float red[kSlots * kG2Max * 16];
  __shared__ __attribute__((aligned(16))) float ys[AWQ_MOE_KMAX_TOPK * 16];       // [rank][16]
  __shared__ float wr[AWQ_MOE_KMAX_TOPK];                                         // rank -> router weight
  __shared__ int nvalid_s;
  const int G2 = dims_G2(dims), LS = 4 * G2;  // SPW * LS <= 64
  const int H = 32 * dims_G(dims), I = 32 * G2, topk = dims_topk(dims);
  const int T2 = H >> 4;
  const int nt = (T2 & 7) ? (int)blockIdx.x : (int)((blockIdx.x & 7) * (T2 >> 3) + (blockIdx.x >> 3));
  const int tok = blockIdx.y;
  const int t = threadIdx.x, lane = t & 63;
  const int s0 = __builtin_amdgcn_readfirstlane(t >> 6) * SPW;  // the wave's first slot
  const int32_t* ids = topk_ids + tok * topk;
  const ExpertGeometry geo = expert_geometry<RB>(dims);
  const uint32_t expert_bytes = geo.expert_bytes, meta_delta = geo.w2_meta_delta;
  uint16_t rv = 0;
  if constexpr (RES) rv = resid[(uint64_t)tok * H + nt * 16 + (t & 15)];  // used by t < 16
  // the wave's ids and router weights, indexes clamped into the token's slots
  int ek[SPW];
  float wk[SPW];
#pragma unroll
  for (int k = 0; k < SPW; ++k) {
    const int sk = s0 + k < topk ? s0 + k : topk - 1;
    ek[k] = ids[sk];
    wk[k] = topk_w[tok * topk + sk];
  }
  // ranking input: lane j holds slot j's id
  const int rid = ids[lane < topk ? lane : topk - 1];
  // the lane's slot inside the wave (kk == SPW: a lane past the segments)
  int kk = 0;
#pragma unroll
  for (int k = 1; k <= SPW; ++k) kk += lane >= k * LS;
  // in [0, LS) for every lane: a lane past the segments is clamped to the
  // segment's last, so that its (unused) loads stay inside the tile, the
  // expert's records and the slot's act row also when SPW * LS + LS < 64
  const int tl = min(lane - kk * LS, LS - 1);
  const int slot = s0 + kk;
  const bool lane_on = kk < SPW && slot < topk;
  const int slotc = slot < topk ? slot : topk - 1;
  const int g = tl >> 2, quad = tl & 3;
  const uint4 araw = *reinterpret_cast<const uint4*>(act + (uint64_t)(tok * topk + slotc) * I + 32 * g + 8 * quad);
  int e = ek[0];
#pragma unroll
  for (int k = 1; k < SPW; ++k) e = kk == k ? ek[k] : e;
  const bool valid_e = e >= 0 && e < E;
  const bool live = lane_on && valid_e;
  const uint64_t eo = (uint64_t)(uint32_t)(valid_e ? e : 0) * expert_bytes;
  const uint8_t* units = units_base + eo + (uint64_t)nt * 256u * G2;
  const RawRecords<RB> rraw =
      load_records_raw<RB>(units_base + eo + meta_delta + (uint64_t)nt * 16u * G2 * RB + (uint64_t)tl * 4u * RB);
  uint4 w[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) w[j] = load_unit16<true>(units + ((uint64_t)j * LS + tl) * 16u);
  // Keep the ranking below the weight loads: it runs while they are in flight.
  __builtin_amdgcn_sched_barrier(0);
  // Ranks of the wave's slots among the token's valid slots by (id, slot):
  // each is the population count of one ballot against a wave-uniform id.
  const bool vj = lane < topk && rid >= 0 && rid < E;
  int rk[SPW];
#pragma unroll
  for (int k = 0; k < SPW; ++k)
    rk[k] = (int)__popcll(__ballot(vj && (rid < ek[k] || (rid == ek[k] && lane < s0 + k))));
  const unsigned long long bv = __ballot(vj);
  if (lane == 0) {
#pragma unroll
    for (int k = 0; k < SPW; ++k)
      if (s0 + k < topk && ek[k] >= 0 && ek[k] < E) wr[rk[k]] = wk[k];
    if (s0 == 0) nvalid_s = (int)__popcll(bv);
  }
  int rank = rk[0];
#pragma unroll
  for (int k = 1; k < SPW; ++k) rank = kk == k ? rk[k] : rank;
  // the quad's four 16-byte quarters of the group's activations, to every lane of the quad
  Act32 av;
  av.px[0] = quad_bcast<0>(araw.x); av.px[1] = quad_bcast<0>(araw.y); av.px[2] = quad_bcast<0>(araw.z); av.px[3] = quad_bcast<0>(araw.w);
  av.px[4] = quad_bcast<1>(araw.x); av.px[5] = quad_bcast<1>(araw.y); av.px[6] = quad_bcast<1>(araw.z); av.px[7] = quad_bcast<1>(araw.w);
  av.px[8] = quad_bcast<2>(araw.x); av.px[9] = quad_bcast<2>(araw.y); av.px[10] = quad_bcast<2>(araw.z); av.px[11] = quad_bcast<2>(araw.w);
  av.px[12] = quad_bcast<3>(araw.x); av.px[13] = quad_bcast<3>(araw.y); av.px[14] = quad_bcast<3>(araw.z); av.px[15] = quad_bcast<3>(araw.w);
  float* rrow = red + (slotc * kG2Max) * 16 + 4 * quad;  // + 16 g: this lane's four columns in group g
  if (live) {
    float S, Cs;
    group_sums(av, S, Cs);
    const Records<RB> rec = decode_records<RB>(rraw);
    const Magic mg = make_magic();
    float4 part;
    part.x = rec.s[0] * (unit_dot(w[0], av, mg) - fmaf(rec.z[0], S, Cs));
    part.y = rec.s[1] * (unit_dot(w[1], av, mg) - fmaf(rec.z[1], S, Cs));
    part.z = rec.s[2] * (unit_dot(w[2], av, mg) - fmaf(rec.z[2], S, Cs));
    part.w = rec.s[3] * (unit_dot(w[3], av, mg) - fmaf(rec.z[3], S, Cs));
    *reinterpret_cast<float4*>(rrow + 16 * g) = part;
  }
  // the writes above come from this wave only; wait for them (and keep the
  // compiler from moving the reads below above them)
  asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
  if (live && g == 0) {
    float4 y = *reinterpret_cast<const float4*>(rrow);
    for (int gg = 1; gg < G2; ++gg) {
      const float4 v = *reinterpret_cast<const float4*>(rrow + 16 * gg);
      y.x += v.x;
      y.y += v.y;
      y.z += v.z;
      y.w += v.w;
    }
    *reinterpret_cast<float4*>(ys + rank * 16 + 4 * quad) = y;
  }
  __syncthreads();
  if (t < 16) {
    const int nv = nvalid_s;
    float acc = 0.f;
#pragma unroll 4
    for (int rr = 0; rr < nv; ++rr) acc = fmaf(wr[rr], ys[rr * 16 + t], acc);
    _Float16 v = (_Float16)acc;
    if constexpr (RES) v = (_Float16)((float)__builtin_bit_cast(_Float16, rv) + (float)v);
    out[(uint64_t)tok * H + nt * 16 + t] = __builtin_bit_cast(uint16_t, v);
  }
}

// The slot-segment W2 for inter 544 to 1024 (at most 16 slots): the work
// of w2_reduce_seg_kernel with one slot per wave, whose 64 lanes each take
// group g = lane / 4 and, below G2, group g + 16 as well; the groups are
// summed in the same ascending order, so the result equals the generic
// kernel's. (A kernel of its own, so that the rank shape's kernel keeps its
// code.)
template <int RB, bool RES>
__global__ __launch_bounds__(1024) void w2_reduce_seg2_kernel(const int32_t* __restrict__ topk_ids,
                                                              const uint8_t* __restrict__ units_base,
                                                              const uint16_t* __restrict__ act,
                                                              const float* __restrict__ topk_w,
                                                              uint16_t* __restrict__ out, uint32_t dims, int E,
                                                              const uint16_t* __restrict__ resid) {
  __shared__ __attribute__((aligned(16))) float red[16 * 32 * 16];  // [slot][g][16]
  __shared__ __attribute__((aligned(16))) float ys[16 * 16];        // [rank][16]
  __shared__ float wr[16];                                           // rank -> router weight
  __shared__ int nvalid_s;
  const int G2 = dims_G2(dims), LS = 4 * G2;  // lanes of a tile row (4 per group): 68 .. 128
  const int H = 32 * dims_G(dims), I = 32 * G2, topk = dims_topk(dims);
  const int T2 = H >> 4;
  const int nt = (T2 & 7) ? (int)blockIdx.x : (int)((blockIdx.x & 7) * (T2 >> 3) + (blockIdx.x >> 3));
  const int tok = blockIdx.y;
  const int t = threadIdx.x, lane = t & 63;
  const int slot = __builtin_amdgcn_readfirstlane(t >> 6);  // the wave's slot (< topk <= 16)
  const int32_t* ids = topk_ids + tok * topk;
  const ExpertGeometry geo = expert_geometry<RB>(dims);
  const uint32_t expert_bytes = geo.expert_bytes, meta_delta = geo.w2_meta_delta;
  uint16_t rv = 0;
  if constexpr (RES) rv = resid[(uint64_t)tok * H + nt * 16 + (t & 15)];  // used by t < 16
  const int e = ids[slot];
  const float we = topk_w[tok * topk + slot];
  const int rid = ids[lane < topk ? lane : topk - 1];  // ranking input: lane j holds slot j's id
  // lane tl takes group g = tl / 4 and, below G2, group g2 = g + 16 (its
  // lane index clamped into the tile row, so the unused loads stay inside)
  const int tl = lane, g = tl >> 2, quad = tl & 3;
  const int tl2 = min(tl + 64, LS - 1), g2 = tl2 >> 2;
  const bool on2 = tl + 64 < LS;
  const uint16_t* arow = act + (uint64_t)(tok * topk + slot) * I + 8 * quad;
  const uint4 araw = *reinterpret_cast<const uint4*>(arow + 32 * g);
  const uint4 araw2 = *reinterpret_cast<const uint4*>(arow + 32 * g2);
  const bool live = e >= 0 && e < E;
  const uint64_t eo = (uint64_t)(uint32_t)(live ? e : 0) * expert_bytes;
  const uint8_t* units = units_base + eo + (uint64_t)nt * 256u * G2;
  const uint8_t* recs = units_base + eo + meta_delta + (uint64_t)nt * 16u * G2 * RB;
  const RawRecords<RB> rraw = load_records_raw<RB>(recs + (uint64_t)tl * 4u * RB);
  const RawRecords<RB> rraw2 = load_records_raw<RB>(recs + (uint64_t)tl2 * 4u * RB);
  uint4 w[4], wb[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) w[j] = load_unit16<true>(units + ((uint64_t)j * LS + tl) * 16u);
#pragma unroll
  for (int j = 0; j < 4; ++j) wb[j] = load_unit16<true>(units + ((uint64_t)j * LS + tl2) * 16u);
  // Keep the ranking below the weight loads: it runs while they are in flight.
  __builtin_amdgcn_sched_barrier(0);
  // The slot's rank among the token's valid slots by (id, slot).
  const bool vj = lane < topk && rid >= 0 && rid < E;
  const int rank = (int)__popcll(__ballot(vj && (rid < e || (rid == e && lane < slot))));
  const unsigned long long bv = __ballot(vj);
  if (lane == 0) {
    if (live) wr[rank] = we;
    if (slot == 0) nvalid_s = (int)__popcll(bv);
  }
  // the quad's four 16-byte quarters of the group's activations, to every
  // lane of the quad (the second group's after the first group's products,
  // so that the two are not live together)
  Act32 av;
  av.px[0] = quad_bcast<0>(araw.x); av.px[1] = quad_bcast<0>(araw.y); av.px[2] = quad_bcast<0>(araw.z); av.px[3] = quad_bcast<0>(araw.w);
  av.px[4] = quad_bcast<1>(araw.x); av.px[5] = quad_bcast<1>(araw.y); av.px[6] = quad_bcast<1>(araw.z); av.px[7] = quad_bcast<1>(araw.w);
  av.px[8] = quad_bcast<2>(araw.x); av.px[9] = quad_bcast<2>(araw.y); av.px[10] = quad_bcast<2>(araw.z); av.px[11] = quad_bcast<2>(araw.w);
  av.px[12] = quad_bcast<3>(araw.x); av.px[13] = quad_bcast<3>(araw.y); av.px[14] = quad_bcast<3>(araw.z); av.px[15] = quad_bcast<3>(araw.w);
  float* rrow = red + (slot * 32) * 16 + 4 * quad;  // + 16 g: this lane's four columns in group g
  if (live) {
    float S, Cs;
    group_sums(av, S, Cs);
    const Records<RB> rec = decode_records<RB>(rraw);
    const Magic mg = make_magic();
    float4 part;
    part.x = rec.s[0] * (unit_dot(w[0], av, mg) - fmaf(rec.z[0], S, Cs));
    part.y = rec.s[1] * (unit_dot(w[1], av, mg) - fmaf(rec.z[1], S, Cs));
    part.z = rec.s[2] * (unit_dot(w[2], av, mg) - fmaf(rec.z[2], S, Cs));
    part.w = rec.s[3] * (unit_dot(w[3], av, mg) - fmaf(rec.z[3], S, Cs));
    *reinterpret_cast<float4*>(rrow + 16 * g) = part;
  }
  Act32 av2;
  av2.px[0] = quad_bcast<0>(araw2.x); av2.px[1] = quad_bcast<0>(araw2.y); av2.px[2] = quad_bcast<0>(araw2.z); av2.px[3] = quad_bcast<0>(araw2.w);
  av2.px[4] = quad_bcast<1>(araw2.x); av2.px[5] = quad_bcast<1>(araw2.y); av2.px[6] = quad_bcast<1>(araw2.z); av2.px[7] = quad_bcast<1>(araw2.w);
  av2.px[8] = quad_bcast<2>(araw2.x); av2.px[9] = quad_bcast<2>(araw2.y); av2.px[10] = quad_bcast<2>(araw2.z); av2.px[11] = quad_bcast<2>(araw2.w);
  av2.px[12] = quad_bcast<3>(araw2.x); av2.px[13] = quad_bcast<3>(araw2.y); av2.px[14] = quad_bcast<3>(araw2.z); av2.px[15] = quad_bcast<3>(araw2.w);
  if (live && on2) {
    float S, Cs;
    group_sums(av2, S, Cs);
    const Records<RB> rec = decode_records<RB>(rraw2);
    const Magic mg = make_magic();
    float4 part;
    part.x = rec.s[0] * (unit_dot(wb[0], av2, mg) - fmaf(rec.z[0], S, Cs));
    part.y = rec.s[1] * (unit_dot(wb[1], av2, mg) - fmaf(rec.z[1], S, Cs));
    part.z = rec.s[2] * (unit_dot(wb[2], av2, mg) - fmaf(rec.z[2], S, Cs));
    part.w = rec.s[3] * (unit_dot(wb[3], av2, mg) - fmaf(rec.z[3], S, Cs));
    *reinterpret_cast<float4*>(rrow + 16 * g2) = part;
  }
  // the writes above come from this wave only; wait for them (and keep the
  // compiler from moving the reads below above them)
  asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
  if (live && g == 0) {
    float4 y = *reinterpret_cast<const float4*>(rrow);
    for (int gg = 1; gg < G2; ++gg) {
      const float4 v = *reinterpret_cast<const float4*>(rrow + 16 * gg);
      y.x += v.x;
      y.y += v.y;
      y.z += v.z;
      y.w += v.w;
    }
    *reinterpret_cast<float4*>(ys + rank * 16 + 4 * quad) = y;
  }
  __syncthreads();
  if (t < 16) {
    const int nv = nvalid_s;
    float acc = 0.f;
#pragma unroll 4
    for (int rr = 0; rr < nv; ++rr) acc = fmaf(wr[rr], ys[rr * 16 + t], acc);
    _Float16 v = (_Float16)acc;
    if constexpr (RES) v = (_Float16)((float)__builtin_bit_cast(_Float16, rv) + (float)v);
    out[(uint64_t)tok * H + nt * 16 + t] = __builtin_bit_cast(uint16_t, v);
  }
}

// ---------------------------------------------------------------------------
// dequantisation (diagnostic): one thread per unit, writes 32 fp32 values
// ---------------------------------------------------------------------------
template <int RB>
__global__ void dequant_kernel(const uint8_t* __restrict__ bank, uint64_t expert_bytes,
                               uint64_t units_off, uint64_t meta_off, int K, int N,
                               int expert_begin, int expert_count, float* __restrict__ out) {
  const int G = K >> 5;
  const uint64_t per_expert = (uint64_t)G * N;
  const uint64_t idx = (uint64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (idx >= per_expert * (uint64_t)expert_count) return;
  const int el = (int)(idx / per_expert);
  const int rem = (int)(idx - (uint64_t)el * per_expert);
  const int g = rem / N, n = rem - g * N;
  // W13 and W2 share the tiled placement (16-column tiles, t = 4g + quad).
  const int L = 4 * G, nt = n >> 4, c = n & 15, quad = c >> 2, j = c & 3, t = 4 * g + quad;
  const uint64_t uo = (uint64_t)nt * 256u * G + ((uint64_t)j * L + t) * 16u;
  const uint64_t ro = (uint64_t)nt * 16u * G * RB + (uint64_t)(4 * t + j) * RB;
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
// Fixed decode scratch for callers that cannot allocate device memory: the
// workspace (status word, fp16 act) of awq_moe_decode_noalloc. One copy per
// device, held until the process ends. In host code the array's name only
// stands for the symbol; kernels get the device address that
// hipGetSymbolAddress returns for the current device.
// ---------------------------------------------------------------------------
static __device__ __attribute__((aligned(256))) uint8_t scratch[AWQ_MOE_KNOALLOC_SCRATCH_BYTES];

namespace {
constexpr int kMaxDevices = 64;
std::atomic<void*> g_scratch_ptr[kMaxDevices];
std::mutex g_scratch_mu;
std::atomic<int> g_resident_waves[kMaxDevices];  // 0: not asked yet
}  // namespace

// Waves the current device holds at once at 8 per SIMD (4 SIMDs per CU):
// 8,192 on a whole MI355X, fewer on a partition of it. Asked once per device.
static int resident_waves() {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return 256 * 32;
  int w = g_resident_waves[dev].load(std::memory_order_relaxed);
  if (w == 0) {
    int cus = 0;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0) cus = 256;
    w = 32 * cus;
    g_resident_waves[dev].store(w, std::memory_order_relaxed);
  }
  return w;
}

hipError_t noalloc_scratch(void** ptr) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  void* p = g_scratch_ptr[dev].load(std::memory_order_acquire);
  if (!p) {
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    p = g_scratch_ptr[dev].load(std::memory_order_relaxed);
    if (!p) {
      e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
      if (e != hipSuccess) return e;
      if (!p || reinterpret_cast<uintptr_t>(p) % 256 != 0) return hipErrorInvalidSymbol;
      g_scratch_ptr[dev].store(p, std::memory_order_release);
    }
  }
  *ptr = p;
  return hipSuccess;
}

// ---------------------------------------------------------------------------
// launchers
// ---------------------------------------------------------------------------
hipError_t launch_route_compact(const int32_t* ids, int n, int E, const RouteOut& o, hipStream_t stream) {
  // four lanes per slot, at least one wave
  const int threads = ((4 * n + 63) / 64) * 64;
  hipLaunchKernelGGL(route_compact_kernel, dim3(1), dim3(threads), 0, stream, ids, n, E, o);
  return hipGetLastError();
}

// The decode kernels take 32-bit expert strides and record offsets; the
// largest admitted shape (hidden 8192, inter 2048) needs about 34 MB per
// expert, so a wider value means the arguments are corrupt.
static bool fits32(const StageArgs& a, uint64_t meta_delta) {
  return a.expert_bytes <= 0xFFFFFFFFull && meta_delta <= 0xFFFFFFFFull;
}

// ---------------------------------------------------------------------------
// Tactic table: the kernel form of each stage per token count M and record
// size, measured on the rank layer (512 experts, hidden 2560, inter 160,
// top-k 10; cold weights, shared expert pools for M >= 2, graphs of 48
// calls). A form the shape cannot run falls back to the general rule: lane
// pairs while the grid has at most one workgroup per CU (256), else single
// lanes; for W2 the most slots per wave.
// ---------------------------------------------------------------------------
struct DecodeTactic {
  int8_t w13, w2;
};
// [record bytes 3, 4][M - 1]. W13 us per launch, 3-byte records (lane pairs /
// single lanes / two tiles per workgroup): M=1 3.51 / 3.61 / 3.91,
// M=2 4.44 / 4.25 / 4.31, M=3 5.50 / 4.84 / 5.64, M=8 9.61 / 8.07 / 9.03;
// 4-byte records rank the same except at M=2 (4.49 / 4.43 / 4.36). W2 with
// the most slots per wave wins at every M (M=1 3.42 against 3.63, M=8 5.69
// against 6.26).
constexpr DecodeTactic kDecodeTable[2][AWQ_MOE_KMAX_TOKENS] = {
    {{kW13Pair, kW2SegMost}, {kW13Single, kW2SegMost}, {kW13Single, kW2SegMost}, {kW13Single, kW2SegMost},
     {kW13Single, kW2SegMost}, {kW13Single, kW2SegMost}, {kW13Single, kW2SegMost}, {kW13Single, kW2SegMost}},
    {{kW13Pair, kW2SegMost}, {kW13Single2, kW2SegMost}, {kW13Single, kW2SegMost}, {kW13Single, kW2SegMost},
     {kW13Single, kW2SegMost}, {kW13Single, kW2SegMost}, {kW13Single, kW2SegMost}, {kW13Single, kW2SegMost}},
};

// The slot-segment W2 kernel's instantiated slots-per-wave values, descending.
constexpr int kSpwChoices[] = {16, 8, 5, 4, 3, 2, 1};

static int w2_spw(int form, int I) {
  const int cap = 64 / (I / 8);  // slots that fit a wave at I/8 lanes each
  int most = -1;
  for (int i = 0; i < (int)(sizeof kSpwChoices / sizeof kSpwChoices[0]); ++i)
    if (kSpwChoices[i] <= cap) {
      most = i;
      break;
    }
  if (most < 0) return 0;
  if (form == kW2SegFewer) return most + 1 < (int)(sizeof kSpwChoices / sizeof kSpwChoices[0]) ? kSpwChoices[most + 1] : 0;
  return kSpwChoices[most];
}

bool w13_form_valid(int form, int H, int I, int topk, int M) {
  const int L = 4 * (H / 32);
  switch (form) {
    case kW13Pair: return 2 * L <= 1024;
    case kW13Single: return L <= 1024;
    case kW13Single2: return 2 * ((L + 63) / 64) * 64 <= 1024 && ((2 * I) / 16) % 2 == 0;
    default: return false;
  }
}

// The slot-segment kernel runs a form when the form's slots per wave fit the
// inter size and the token's slots fit 16 waves (from inter 544 to 1024 the
// most-slots form is its two-groups-per-lane variant); otherwise the
// generic kernel (inter > 1024, or more than 16 waves) serves the shape with
// its one form.
static bool w2_seg_fits(int spw, int topk) { return spw > 0 && (topk + spw - 1) / spw <= 16; }

bool w2_form_valid(int form, int H, int I, int topk, int M) {
  if (form != kW2SegMost && form != kW2SegFewer) return false;
  return w2_seg_fits(w2_spw(form, I), topk) || form == kW2SegMost;
}

void decode_table(int H, int I, int topk, int M, int RB, int* w13_form, int* w2_form) {
  // past the table (the indexed prefill's smallest calls): single lanes, the
  // most slots per wave
  const DecodeTactic d = M <= AWQ_MOE_KMAX_TOKENS ? kDecodeTable[RB == 4 ? 1 : 0][M - 1]
                                                  : DecodeTactic{kW13Single, kW2SegMost};
  int f13 = d.w13, f2 = d.w2;
  const uint64_t grid = (uint64_t)((2 * I) / 16) * M * topk;
  // the table's lane pairs are for grids of up to two workgroups per CU (its
  // rank layer at M <= 2); other shapes take the general rule
  if (!w13_form_valid(f13, H, I, topk, M) || (f13 == kW13Pair && grid > 512))
    f13 = w13_form_valid(kW13Pair, H, I, topk, M) && grid <= 256 ? kW13Pair : kW13Single;
  if (!w2_form_valid(f2, H, I, topk, M)) f2 = kW2SegMost;
  *w13_form = f13;
  *w2_form = f2;
}

template <int RB, bool NORM>
static void launch_w13_t(const StageArgs& a, const uint16_t* x, uint8_t* w, uint32_t md, float eps, int form,
                         hipStream_t stream) {
  const int L = 4 * (a.H / 32);
  const dim3 grid((2 * a.I) / 16, a.M * a.topk);
  const uint32_t dims = pack_dims(a.H, a.I, a.topk, a.M);
  const int bw = ((L + 63) / 64) * 64;  // threads per tile, single lanes
  // non-temporal weights when the whole grid can be resident at once (its
  // waves within the CUs x 4 SIMDs x 8): slots that share an expert then
  // request its tiles together (the same count for two tiles per workgroup)
  const bool nt = (uint64_t)grid.x * grid.y * (bw / 64) <= (uint64_t)resident_waves();
  if (form == kW13Pair)
    hipLaunchKernelGGL((w13_swiglu_pair_kernel<RB, NORM>), grid, dim3(((2 * L + 63) / 64) * 64), 0, stream,
                       a.topk_ids, a.bank + a.w13_off, x, w, (uint32_t)a.expert_bytes, md, dims, a.E, eps);
  else if (form == kW13Single2 && nt)
    hipLaunchKernelGGL((w13_swiglu_kernel<RB, NORM, 2, true>), dim3(grid.x / 2, grid.y), dim3(2 * bw), 0, stream,
                       a.topk_ids, a.bank + a.w13_off, x, w, (uint32_t)a.expert_bytes, md, dims, a.E, eps);
  else if (form == kW13Single2)
    hipLaunchKernelGGL((w13_swiglu_kernel<RB, NORM, 2, false>), dim3(grid.x / 2, grid.y), dim3(2 * bw), 0, stream,
                       a.topk_ids, a.bank + a.w13_off, x, w, (uint32_t)a.expert_bytes, md, dims, a.E, eps);
  else if (nt)
    hipLaunchKernelGGL((w13_swiglu_kernel<RB, NORM, 1, true>), grid, dim3(bw), 0, stream, a.topk_ids,
                       a.bank + a.w13_off, x, w, (uint32_t)a.expert_bytes, md, dims, a.E, eps);
  else
    hipLaunchKernelGGL((w13_swiglu_kernel<RB, NORM, 1, false>), grid, dim3(bw), 0, stream, a.topk_ids,
                       a.bank + a.w13_off, x, w, (uint32_t)a.expert_bytes, md, dims, a.E, eps);
}

hipError_t launch_w13_swiglu(const StageArgs& a, const uint16_t* x, void* ws, bool norm, float eps, int form,
                             hipStream_t stream) {
  const uint64_t md = a.w13_meta_off - a.w13_off;
  if (!fits32(a, md)) return hipErrorInvalidValue;
  if (form == kW13Table) {
    int f2;
    decode_table(a.H, a.I, a.topk, a.M, a.RB, &form, &f2);
  } else if (!w13_form_valid(form, a.H, a.I, a.topk, a.M)) {
    return hipErrorInvalidValue;
  }
  uint8_t* w = static_cast<uint8_t*>(ws);
  if (a.RB == 4) {
    if (norm) launch_w13_t<4, true>(a, x, w, (uint32_t)md, eps, form, stream);
    else launch_w13_t<4, false>(a, x, w, (uint32_t)md, eps, form, stream);
  } else {
    if (norm) launch_w13_t<3, true>(a, x, w, (uint32_t)md, eps, form, stream);
    else launch_w13_t<3, false>(a, x, w, (uint32_t)md, eps, form, stream);
  }
  return hipGetLastError();
}

template <int RB, int TPW, bool RES>
static void launch_w2_t(const StageArgs& a, const uint16_t* act, const float* topk_w, uint16_t* out,
                        const uint16_t* resid, hipStream_t stream) {
  const int lanes = a.topk * TPW * 4 * (a.I / 32);
  const dim3 block(lanes >= 1024 ? 1024 : ((lanes + 63) / 64) * 64);
  const dim3 grid(a.H / (16 * TPW), a.M);
  hipLaunchKernelGGL((w2_reduce_kernel<RB, TPW, RES>), grid, block, 0, stream, a.topk_ids, a.bank + a.w2_off,
                     a.bank + a.w2_meta_off, act, a.expert_bytes, a.H, a.I, a.topk, a.E, topk_w, out, resid);
}

// One 16-column tile per workgroup: groups of 2 or 4 adjacent tiles (longer
// contiguous runs per expert) measured no faster, at 4 slower, on hot and
// on cold weights.
template <int RB, int SPW, bool RES>
static void launch_w2_seg(const StageArgs& a, const uint16_t* act, const float* topk_w, uint16_t* out,
                          const uint16_t* resid, hipStream_t stream) {
  const int waves = (a.topk + SPW - 1) / SPW;
  const dim3 grid(a.H / 16, a.M);
  hipLaunchKernelGGL((w2_reduce_seg_kernel<RB, SPW, RES>), grid, dim3(64 * waves), 0, stream, a.topk_ids,
                     a.bank + a.w2_off, act, topk_w, out, pack_dims(a.H, a.I, a.topk, a.M), a.E, resid);
}

// Inter 544 to 1024 with at most 16 slots: one slot per wave, two groups per lane.
static bool w2_seg2_fits(int I, int topk) { return I > 512 && I <= 1024 && topk <= 16; }

template <int RB, bool RES>
static void launch_w2_seg2(const StageArgs& a, const uint16_t* act, const float* topk_w, uint16_t* out,
                           const uint16_t* resid, hipStream_t stream) {
  const dim3 grid(a.H / 16, a.M);
  hipLaunchKernelGGL((w2_reduce_seg2_kernel<RB, RES>), grid, dim3(64 * a.topk), 0, stream, a.topk_ids,
                     a.bank + a.w2_off, act, topk_w, out, pack_dims(a.H, a.I, a.topk, a.M), a.E, resid);
}

template <int RB, bool RES>
static void launch_w2_seg_rb(const StageArgs& a, const uint16_t* act, const float* topk_w, uint16_t* out,
                             const uint16_t* resid, int spw, hipStream_t stream) {
  // spw: an instantiated slots-per-wave value that fits (I/8 lanes per slot)
  if (spw == 16) launch_w2_seg<RB, 16, RES>(a, act, topk_w, out, resid, stream);
  else if (spw == 8) launch_w2_seg<RB, 8, RES>(a, act, topk_w, out, resid, stream);
  else if (spw == 5) launch_w2_seg<RB, 5, RES>(a, act, topk_w, out, resid, stream);
  else if (spw == 4) launch_w2_seg<RB, 4, RES>(a, act, topk_w, out, resid, stream);
  else if (spw == 3) launch_w2_seg<RB, 3, RES>(a, act, topk_w, out, resid, stream);
  else if (spw == 2) launch_w2_seg<RB, 2, RES>(a, act, topk_w, out, resid, stream);
  else launch_w2_seg<RB, 1, RES>(a, act, topk_w, out, resid, stream);
}

template <bool RES>
static hipError_t launch_w2_res(const StageArgs& a, const uint16_t* act, const float* topk_w, uint16_t* out,
                                const uint16_t* resid, int form, hipStream_t stream) {
  const int spw = w2_spw(form, a.I);
  const bool seg2 = spw == 0 && form == kW2SegMost && w2_seg2_fits(a.I, a.topk);
  if (w2_seg_fits(spw, a.topk) || seg2) {
    // the slot-segment kernels derive the expert geometry from the shape word
    const ExpertGeometry g = a.RB == 4 ? expert_geometry<4>(pack_dims(a.H, a.I, a.topk, a.M))
                                       : expert_geometry<3>(pack_dims(a.H, a.I, a.topk, a.M));
    if (g.expert_bytes != a.expert_bytes || g.w2_off != a.w2_off || g.w2_meta_delta != a.w2_meta_off - a.w2_off)
      return hipErrorInvalidValue;
    if (seg2 && a.RB == 4)
      launch_w2_seg2<4, RES>(a, act, topk_w, out, resid, stream);
    else if (seg2)
      launch_w2_seg2<3, RES>(a, act, topk_w, out, resid, stream);
    else if (a.RB == 4)
      launch_w2_seg_rb<4, RES>(a, act, topk_w, out, resid, spw, stream);
    else
      launch_w2_seg_rb<3, RES>(a, act, topk_w, out, resid, spw, stream);
    return hipGetLastError();
  }
  if (a.RB == 4)
    launch_w2_t<4, 1, RES>(a, act, topk_w, out, resid, stream);
  else
    launch_w2_t<3, 1, RES>(a, act, topk_w, out, resid, stream);
  return hipGetLastError();
}

hipError_t launch_w2_reduce(const StageArgs& a, const uint16_t* act, const float* topk_w, uint16_t* out,
                            const uint16_t* resid, int form, hipStream_t stream) {
  if (form == kW2Table) {
    int f13;
    decode_table(a.H, a.I, a.topk, a.M, a.RB, &f13, &form);
  } else if (!w2_form_valid(form, a.H, a.I, a.topk, a.M)) {
    return hipErrorInvalidValue;
  }
  return resid ? launch_w2_res<true>(a, act, topk_w, out, resid, form, stream)
               : launch_w2_res<false>(a, act, topk_w, out, nullptr, form, stream);
}

hipError_t launch_dequant(const uint8_t* bank, uint64_t expert_bytes, uint64_t units_off,
                          uint64_t meta_off, int RB, int which, int H, int I, int expert_begin,
                          int expert_count, float* out, hipStream_t stream) {
  const int K = which == 0 ? H : I;
  const int N = which == 0 ? 2 * I : H;
  const uint64_t total = (uint64_t)(K / 32) * N * expert_count;
  const dim3 block(256);
  const dim3 grid((unsigned)((total + 255) / 256));
  if (RB == 4)
    hipLaunchKernelGGL(dequant_kernel<4>, grid, block, 0, stream, bank, expert_bytes, units_off,
                       meta_off, K, N, expert_begin, expert_count, out);
  else
    hipLaunchKernelGGL(dequant_kernel<3>, grid, block, 0, stream, bank, expert_bytes, units_off,
                       meta_off, K, N, expert_begin, expert_count, out);
  return hipGetLastError();
}

}  // namespace awq_moe
