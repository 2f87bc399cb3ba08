// Device-side helpers shared by the kernels of the library (gfx950 only).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/varlen.h"

// Instruction-scheduling hints; they only mean something in the device pass
// (the host pass of a kernel template must not see the gfx builtins).
#if defined(__HIP_DEVICE_COMPILE__)
#define VL_SCHED_BARRIER(mask) __builtin_amdgcn_sched_barrier(mask)
#define VL_SCHED_GROUP(mask, n, id) __builtin_amdgcn_sched_group_barrier(mask, n, id)
#else
#define VL_SCHED_BARRIER(mask)
#define VL_SCHED_GROUP(mask, n, id)
#endif

namespace vl {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr int kXcds = 8;          // chiplets; block ids are dealt to them round-robin
constexpr int kLptMaxReqs = 64;   // longest-first request order up to this many requests
constexpr int kMaxSplit = 16;       // key ranges a tile of the last round is cut into, at most
constexpr int kMinSplitKeys = 256;  // and no more ranges than max_kv / this
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.69314718055994531f;

__device__ __forceinline__ int lane_id() { return __lane_id(); }

__device__ __forceinline__ int readlane(int x, int l) { return __builtin_amdgcn_readlane(x, l); }

// Value of x in lane (l xor 32), through the gfx950 lane-half swap (one VALU op).
__device__ __forceinline__ float swap_halves(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return lane_id() < 32 ? __uint_as_float(r[1]) : __uint_as_float(r[0]);
}

// x[lane] combined with x[lane xor 32]; symmetric in the two halves.
// (The max is one v_max_f32: fmaxf would first requiet each permuted value
// with a max of the value with itself, two more VALU ops; the inputs here are
// scores, never signalling NaNs.)
__device__ __forceinline__ float pair_max(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  float m;
  asm("v_max_f32 %0, %1, %2" : "=v"(m) : "v"(__uint_as_float(r[0])), "v"(__uint_as_float(r[1])));
  return m;
}
__device__ __forceinline__ float pair_sum(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// Launched block id -> logical tile: the i-th block chiplet x (= b mod 8)
// receives takes tile ((i div chunk) * 8 + x) * chunk + (i mod chunk).
__device__ __forceinline__ int block_to_logical(int b, int chunk) {
  const int x = b % kXcds;
  const int i = b / kXcds;
  return ((i / chunk) * kXcds + x) * chunk + (i % chunk);
}

// Bounds of the requests, one request per lane (lane r < R <= kLptMaxReqs):
// query rows [qs, qe) and key rows [ks, ke); lanes >= R hold zeros.
struct ReqLanes {
  int qs, qe, ks, ke;
};
__device__ __forceinline__ ReqLanes load_req_lanes(const int32_t* __restrict__ q_cu,
                                                   const int32_t* __restrict__ kv_cu, int R) {
  const int lane = lane_id();
  ReqLanes l{0, 0, 0, 0};
  if (lane < R) {
    l.qs = q_cu[lane];
    l.qe = q_cu[lane + 1];
    l.ks = kv_cu[lane];
    l.ke = kv_cu[lane + 1];
  }
  return l;
}

// Number of tiles (see total_tiles) from bounds in registers (R <= kLptMaxReqs).
__device__ __forceinline__ int total_tiles_lanes(const ReqLanes& l, int R, int H, int block_m) {
  int cnt = lane_id() < R ? ((l.qe - l.qs + block_m - 1) / block_m) * H : 0;
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) cnt += __shfl_xor(cnt, off);
  return cnt;
}

// find_tile (below) for R <= kLptMaxReqs on bounds already in registers:
// requests by key length descending, ties by lower index.
__device__ __forceinline__ void find_tile_lanes(const ReqLanes& l, int R, int H, int block_m, int t, int& req,
                                                int& head, int& qtile) {
  const int lane = lane_id();
  req = -1;
  head = 0;
  qtile = 0;
  int kvlen = -1, nt = 0, cnt = 0;
  if (lane < R) {
    kvlen = l.ke - l.ks;
    nt = (l.qe - l.qs + block_m - 1) / block_m;
    cnt = nt * H;
  }
  int rank = 0;
  for (int s = 0; s < R; ++s) {
    const int kv_s = readlane(kvlen, s);
    rank += (kv_s > kvlen) || (kv_s == kvlen && s < lane);
  }
  int start = 0;
  for (int s = 0; s < R; ++s) {
    const int rank_s = readlane(rank, s);
    const int cnt_s = readlane(cnt, s);
    start += (rank_s < rank) ? cnt_s : 0;
  }
  const bool hit = lane < R && cnt > 0 && t >= start && t < start + cnt;
  const uint64_t m = __ballot(hit);
  if (m) {
    const int r = __ffsll((unsigned long long)m) - 1;
    const int st = readlane(start, r);
    const int ntr = readlane(nt, r);
    const int local = t - st;
    req = r;
    head = local / ntr;
    qtile = local % ntr;
  }
}

// Logical tile t -> (request, head, q-tile) of the varlen schedule; req = -1
// when t is past the last tile.  Requests are visited by key length
// descending (ties: lower index first) when R <= kLptMaxReqs, else in index
// order; inside a request heads ascend, then q-tiles.  Executed by a whole
// wave (all 64 lanes active); the result is wave-uniform.
__device__ __forceinline__ void find_tile(const int32_t* __restrict__ q_cu,
                                          const int32_t* __restrict__ kv_cu, int R, int H,
                                          int block_m, int t, int& req, int& head, int& qtile) {
  const int lane = lane_id();
  req = -1;
  head = 0;
  qtile = 0;
  if (R <= kLptMaxReqs) {
    find_tile_lanes(load_req_lanes(q_cu, kv_cu, R), R, H, block_m, t, req, head, qtile);
  } else {
    int base = 0;
    for (int r0 = 0; r0 < R; r0 += 64) {
      const int r = r0 + lane;
      int nt = 0, cnt = 0;
      if (r < R) {
        nt = (q_cu[r + 1] - q_cu[r] + block_m - 1) / block_m;
        cnt = nt * H;
      }
      int incl = cnt;
#pragma unroll
      for (int off = 1; off < 64; off <<= 1) {
        const int y = __shfl_up(incl, off);
        if (lane >= off) incl += y;
      }
      const int excl = incl - cnt;
      const bool hit = cnt > 0 && t >= base + excl && t < base + incl;
      const uint64_t m = __ballot(hit);
      if (m) {
        const int l = __ffsll((unsigned long long)m) - 1;
        const int st = base + readlane(excl, l);
        const int ntr = readlane(nt, l);
        const int local = t - st;
        req = r0 + l;
        head = local / ntr;
        qtile = local % ntr;
        return;
      }
      base += readlane(incl, 63);
      if (t < base) return;
    }
  }
}

// Number of (request, head, q-tile) tiles.  Executed by a whole wave; the
// result is wave-uniform.
__device__ __forceinline__ int total_tiles(const int32_t* __restrict__ q_cu, int R, int H, int block_m) {
  int sum = 0;
  for (int r0 = 0; r0 < R; r0 += 64) {
    const int r = r0 + lane_id();
    int cnt = r < R ? ((q_cu[r + 1] - q_cu[r] + block_m - 1) / block_m) * H : 0;
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) cnt += __shfl_xor(cnt, off);
    sum += cnt;
  }
  return sum;
}

// Key split of the last, partial round of a launch with `slots` resident
// work-groups.  Logical tiles [0, full) run whole.  When the remaining
// tail = T - full tiles would leave at least half of the slots idle, each of
// them is cut into `parts` key ranges (at most kMaxSplit, and at most
// max_kv / kMinSplitKeys), run as tail * parts separate work items whose
// partial results a second kernel merges.  parts == 1 means no split
// (full == T).  slots <= 0 turns the split off.
struct SplitPlan {
  int full;
  int tail;
  int parts;
};
__host__ __device__ inline SplitPlan split_plan(int T, int slots, int max_kv) {
  SplitPlan p{T, 0, 1};
  if (slots <= 0 || T <= 0) return p;
  const int full = T >= slots ? (T / slots) * slots : 0;
  const int tail = T - full;
  if (tail == 0) return p;
  int parts = slots / tail;
  if (parts > kMaxSplit) parts = kMaxSplit;
  if (parts > max_kv / kMinSplitKeys) parts = max_kv / kMinSplitKeys;
  if (parts < 2) return p;
  p.full = full;
  p.tail = tail;
  p.parts = parts;
  return p;
}

// Key tiles [lo, hi) of part `part` of `parts` of a key range of nkt tiles.
__host__ __device__ inline void split_range(int nkt, int part, int parts, int& lo, int& hi) {
  lo = (int)((int64_t)part * nkt / parts);
  hi = (int)((int64_t)(part + 1) * nkt / parts);
}

// One unit of work of the varlen launch: a whole tile (part 0 of 1, unit -1)
// or key range `part` of `parts` of a tile of the last round (unit = index
// of its partial-result slot).  req = -1: nothing to do.
struct WorkItem {
  int req, head, qt, part, parts, unit;
};

__device__ __forceinline__ WorkItem work_item(const int32_t* __restrict__ q_cu, const int32_t* __restrict__ kv_cu,
                                              int R, int H, int block_m, int slots, int max_kv, int logical) {
  WorkItem w{-1, -1, -1, -1, -1, -1};
  int tile = logical;
  int part = 0, parts = 1, unit = -1;
  if (slots > 0) {
    const SplitPlan sp = split_plan(total_tiles(q_cu, R, H, block_m), slots, max_kv);
    if (sp.parts > 1 && logical >= sp.full) {
      const int u = logical - sp.full;
      if (u >= sp.tail * sp.parts) return w;
      tile = sp.full + u / sp.parts;
      part = u % sp.parts;
      parts = sp.parts;
      unit = u;
    }
  }
  find_tile(q_cu, kv_cu, R, H, block_m, tile, w.req, w.head, w.qt);
  if (w.req < 0) return w;
  w.part = part;
  w.parts = parts;
  w.unit = unit;
  return w;
}

// Host-side launch size: upper bound on the tile count (plus one round of
// slots for the split work items), rounded up to whole groups of
// (chiplets x chunk) so the block -> logical map is a bijection.
inline int64_t grid_blocks(int64_t num_reqs, int64_t max_q, int64_t H, int64_t block_m,
                           int64_t chunk, int64_t slots = 0) {
  const int64_t upper = num_reqs * H * ((max_q + block_m - 1) / block_m) + (slots > 0 ? slots : 0);
  const int64_t group = kXcds * chunk;
  return ((upper + group - 1) / group) * group;
}

// Transposed V (V^T) staged by the workspace launch: per head, D rows of
// vt_ld bf16 columns.  Request r's keys start at column
// 64 * (ceil(kv_cu[r] / 64) + r): a multiple of 64, and at least
// roundup(len_r, 64) columns past request r-1's start, so every request owns
// whole 64-key tiles and no tile overlaps another request's.
constexpr int kVtTile = 64;
__host__ __device__ inline int64_t vt_col_base(int kv_start, int r) {
  return (int64_t)kVtTile * ((kv_start + kVtTile - 1) / kVtTile + r);
}
// Columns per V^T row for kv_rows key rows in num_reqs requests: bounds
// vt_col_base(kv_cu[R-1], R-1) + roundup(len, 64) for any cu_seqlens within kv_rows.
inline int64_t vt_row_len(int64_t kv_rows, int64_t num_reqs) {
  return (kv_rows + kVtTile - 1) / kVtTile * kVtTile + kVtTile * num_reqs;
}

}  // namespace vl
