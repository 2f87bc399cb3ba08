// Flat varlen and block-local attention forward for gfx950 (MI355X).
//
// What is computed (vLLM-Omni PR #6711 "Key changes" / "Reference /
// Acknowledgement", PR #4024 "Correctness model", PR #7975 review of the
// window code and its "Purpose" / "Change" sections): for every query row and
// head, softmax(scale * q K^T) V over the keys the row may see -- all keys of
// its own request (varlen), or the keys of its block window (block-local).
//
// Kernel design (ours; the pages only name library calls):
//  * attn_bf16_pp_kernel (varlen, bf16): 8 waves = 256 query rows of one
//    (request, head), two phase-shifted groups of four so that on each SIMD
//    one wave issues MFMAs while the other does the softmax; K/V tiles rotate
//    through three LDS buffers.  With a caller workspace, vt_transpose_kernel
//    first stages V as V^T (the MFMA's V operand then is a plain 16-byte LDS
//    read; pack_vt_kernel writes the same V^T straight from the padded V
//    pieces, so the pack and the staging are one pass), the work items are
//    taken through per-chiplet queues, and the last, partial round of tiles
//    is cut along the keys, its parts combined by split_merge_kernel;
//    without one, V tiles are read row-major with transposing LDS reads.
//  * block_local_bf16_kernel / block_local_f32_kernel (block-local, D = 64,
//    blocks of <= 32 frames): one wave per query block of one (batch, head),
//    its window in 32-key chunks, V copied straight to LDS.
//  * block_local_tiled_bf16_kernel (bf16) and attn_f32_kernel (fp32): 4
//    waves = 128 query rows, keys double-buffered through LDS; the
//    block-local shapes outside the block-aligned kernels' range, and fp32
//    varlen.
//  * every wave owns 32 query rows; Q lives in registers for the whole key
//    loop.
//  * S^T = K Q^T on MFMA (bf16: v_mfma_f32_32x32x16_bf16; fp32:
//    v_mfma_f32_32x32x2_f32), so each lane holds one query's scores for 16
//    keys and the row max needs one in-lane pass plus one lane-half swap
//    (v_permlane32_swap); the row sum likewise, or (ping-pong kernel) a
//    16x16x32 MFMA over P.
//  * O^T += V^T P^T on MFMA with P taken straight from the score registers:
//    the MFMA k-index -> key permutation of the score layout is absorbed by
//    the order in which V^T is staged (vt_transpose_kernel), written to LDS,
//    or read from LDS.
//  * exp2-domain online softmax with a lazy rescale: the running max used as
//    the exponent offset only moves when a new score exceeds it by more than
//    a factor 2^8, so most tiles skip the O rescale.  O and l always carry the
//    same factor, so the ratio is unaffected.
//  * varlen masks keys only in a request's last, partial tile; block-local
//    masks each row to [lo, hi) computed from integers (no dense mask, no
//    device-to-host decision) and loads only the union of the rows' windows.
#include <cmath>
#include <mutex>
#include <type_traits>

#include "vl_device.h"

namespace vl {

struct AttnArgs {
  const void* q;
  const void* k;
  const void* v;
  void* out;
  float* lse;
  const int32_t* q_cu;
  const int32_t* kv_cu;
  int R;
  int H;
  int chunk;
  float c;      // scale * log2(e)
  // block-local
  int B;
  int n;
  int block;
  int look_back;
  int look_ahead;
  int nqt;      // query tiles per (batch, head)
  // key split of the last round (varlen, bf16): slots = resident
  // work-groups (0 = no split); ws = partial results, per unit BM rows of
  // D floats of O, then per unit BM (offset, sum) pairs
  int slots;
  int max_kv;
  float* ws;
  // V^T staged for the workspace launch: [H][D][vt_ld] bf16, request r's
  // keys from column vt_col_base(kv_cu[r], r) (nullptr: read V directly)
  void* vt;
  int64_t vt_ld;
  // chiplet work queues of the workspace launch: kXcds ticket counters
  // (zeroed by the V^T staging kernel); nullptr = the static block map
  int* dyn;
};

// ---------------------------------------------------------------- tile setup

struct TileRange {
  int h;        // head
  int q0, q1;   // absolute query rows [q0, q1)
  int kv_base;  // absolute row of key 0 of the sequence
  int k_lo, k_hi;  // keys of the tile, relative to kv_base
  int seq_q0;   // row of q0 inside its sequence (block-local windows)
  int unit;     // partial-result slot of a split work item, -1 for a whole tile
  int req;      // request (varlen) or batch row (block-local)
  bool valid;
};

// logical_item: the varlen work item this work-group takes (-1: none), or
// kStaticItem for the static block map.
constexpr int kStaticItem = -2;
template <int BM, int BN, bool kBlockLocal>
__device__ __forceinline__ TileRange tile_range(const AttnArgs& a, int logical_item = kStaticItem) {
  TileRange t{};
  t.valid = true;
  t.unit = -1;
  if (!kBlockLocal) {
    const int logical = logical_item == kStaticItem ? block_to_logical(blockIdx.x, a.chunk) : logical_item;
    if (logical < 0) {
      t.valid = false;
      return t;
    }
    const WorkItem w = work_item(a.q_cu, a.kv_cu, a.R, a.H, BM, a.slots, a.max_kv, logical);
    if (w.req < 0) {
      t.valid = false;
      return t;
    }
    const int qs = a.q_cu[w.req];
    const int qe = a.q_cu[w.req + 1];
    t.h = w.head;
    t.req = w.req;
    t.q0 = qs + w.qt * BM;
    t.q1 = min(qe, t.q0 + BM);
    t.kv_base = a.kv_cu[w.req];
    const int kv_len = a.kv_cu[w.req + 1] - t.kv_base;
    t.k_lo = 0;
    t.k_hi = kv_len;
    if (w.unit >= 0) {
      int lo, hi;
      split_range((kv_len + BN - 1) / BN, w.part, w.parts, lo, hi);
      t.k_lo = min(kv_len, lo * BN);
      t.k_hi = min(kv_len, hi * BN);
      t.unit = w.unit;
    }
    t.seq_q0 = w.qt * BM;
  } else {
    const int id = blockIdx.x;
    const int qt = id % a.nqt;
    const int bh = id / a.nqt;
    t.h = bh % a.H;
    const int b = bh / a.H;
    t.req = b;
    const int i0 = qt * BM;
    const int i1 = min(a.n, i0 + BM);
    t.q0 = b * a.n + i0;
    t.q1 = b * a.n + i1;
    t.kv_base = b * a.n;
    t.seq_q0 = i0;
    const int nb = (a.n + a.block - 1) / a.block;
    const int blo = max(0, i0 / a.block - a.look_back);
    const int blast = (i1 - 1) / a.block;
    const int bhi = blast + min(a.look_ahead, nb - 1 - blast);  // (no overflow for any look_ahead)
    t.k_lo = blo * a.block;
    t.k_hi = min(a.n, (bhi + 1) * a.block);
  }
  return t;
}

// tile_range's varlen branch for a queue item, on request bounds already in
// registers (R <= kLptMaxReqs) and the launch's split plan: the same
// decode with no memory access.  Executed by a whole wave.
template <int BM, int BN>
__device__ __forceinline__ TileRange item_range_lanes(const AttnArgs& a, const ReqLanes& rl, const SplitPlan& sp,
                                                      int logical) {
  TileRange t{};
  t.valid = false;
  t.unit = -1;
  if (logical < 0) return t;
  int tile = logical, part = 0, parts = 1, unit = -1;
  if (sp.parts > 1 && logical >= sp.full) {
    const int u = logical - sp.full;
    if (u >= sp.tail * sp.parts) return t;
    tile = sp.full + u / sp.parts;
    part = u % sp.parts;
    parts = sp.parts;
    unit = u;
  }
  int req, head, qt;
  find_tile_lanes(rl, a.R, a.H, BM, tile, req, head, qt);
  if (req < 0) return t;
  const int qs = readlane(rl.qs, req);
  const int qe = readlane(rl.qe, req);
  const int ks = readlane(rl.ks, req);
  const int kv_len = readlane(rl.ke, req) - ks;
  t.valid = true;
  t.h = head;
  t.req = req;
  t.q0 = qs + qt * BM;
  t.q1 = min(qe, t.q0 + BM);
  t.kv_base = ks;
  t.k_lo = 0;
  t.k_hi = kv_len;
  if (unit >= 0) {
    int lo, hi;
    split_range((kv_len + BN - 1) / BN, part, parts, lo, hi);
    t.k_lo = min(kv_len, lo * BN);
    t.k_hi = min(kv_len, hi * BN);
    t.unit = unit;
  }
  t.seq_q0 = qt * BM;
  return t;
}

// Keys [lo, hi) of sequence row i under the block window.
__device__ __forceinline__ void window_of(const AttnArgs& a, int i, int& lo, int& hi) {
  const int nb = (a.n + a.block - 1) / a.block;
  const int b = i / a.block;
  lo = max(0, b - a.look_back) * a.block;
  hi = min(a.n, (b + min(a.look_ahead, nb - 1 - b) + 1) * a.block);
}

// ---------------------------------------------------------------- online softmax

// Running state of one lane's query row.  m_c is the exponent offset in
// log2 units (score * c), l the partial row sum of this lane's keys.
template <int NKB, int NDB>
struct RowState {
  float m_c;
  float l;
  f32x16 o[NDB];

  __device__ __forceinline__ void init() {
    m_c = -INFINITY;
    l = 0.f;
#pragma unroll
    for (int d = 0; d < NDB; ++d) o[d] = f32x16{};
  }

  // Masks nothing; turns raw scores s into unnormalised probabilities in place.
  __device__ __forceinline__ void softmax_tile(f32x16 (&s)[NKB], float c) {
    float mx = -INFINITY;
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
      for (int j = 0; j < 16; ++j) mx = fmaxf(mx, s[kb][j]);
    mx = pair_max(mx);
    const float mx_c = mx * c;
    const bool need = mx_c > m_c + 8.0f;
    if (__ballot(need)) {
      const float m_new = need ? mx_c : m_c;
      const float alpha = need ? __builtin_amdgcn_exp2f(m_c - m_new) : 1.0f;
      l *= alpha;
#pragma unroll
      for (int d = 0; d < NDB; ++d) o[d] *= alpha;
      m_c = m_new;
    }
    const float neg_m = (m_c == -INFINITY) ? 0.f : -m_c;
    float ls = 0.f;
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
      for (int j = 0; j < 16; ++j) {
        const float p = __builtin_amdgcn_exp2f(fmaf(s[kb][j], c, neg_m));
        s[kb][j] = p;
        ls += p;
      }
    l += ls;
  }
};

// Key (relative to the tile start) held in score register j of a lane in
// lane-half g, sub-block kb: the 32x32 MFMA accumulator layout.
__device__ __forceinline__ int score_key(int kb, int j, int g) {
  return kb * 32 + 8 * (j >> 2) + 4 * g + (j & 3);
}

template <int NKB>
__device__ __forceinline__ void mask_scores(f32x16 (&s)[NKB], int key0, int g, int lo, int hi) {
#pragma unroll
  for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
    for (int j = 0; j < 16; ++j) {
      const int key = key0 + score_key(kb, j, g);
      if (key < lo || key >= hi) s[kb][j] = -INFINITY;
    }
}

// ---------------------------------------------------------------- bf16 kernel

// s_waitcnt immediate (gfx9 encoding) that waits for all vector-memory operations.
constexpr int kWaitVm0 = 0x0F70;
// ... and one that waits until at most n (< 64) of them are outstanding
// (vmcnt bits 3:0 and 15:14).
constexpr int wait_vm(int n) { return kWaitVm0 | (n & 15) | ((n >> 4) << 14); }
// Word 3 of a raw buffer descriptor (32-bit data format, no swizzle).
[[maybe_unused]] constexpr int kBufferFlags = 0x00020000;  // (used in the device pass only)

template <int D, int WAVES, int BN_>
struct Bf16Geo {
  static constexpr int kThreads = 64 * WAVES;
  static constexpr int BN = BN_;                        // keys per tile
  static constexpr int ROW = D * 2;                     // bytes per K / V row in LDS (no padding)
  static constexpr int CPR = D / 8;                     // 16-byte chunks per row
  static constexpr int kTileBytes = BN * ROW;
  static constexpr int RPI = 1024 / ROW;                // rows per wave-wide 16-byte load
  static constexpr int kLoadsPerWave = kTileBytes / 1024 / WAVES;  // per tensor, per tile
  static constexpr int NKB = BN / 32;
  static constexpr int NDS = D / 16;
  static constexpr int NDB = D / 32;
  static constexpr int NKC = BN / 16;
  static_assert(kLoadsPerWave * WAVES * 1024 == kTileBytes, "whole wave-wide loads per tile");
};

// XOR swizzles of the 16-byte chunks of a K / V row in LDS.  Each row is
// written whole by one wave-wide load, so any permutation inside a row is
// free on the write side; on the read side they spread the rows a wave reads
// together over distinct bank groups.
//  K: lanes 0..15 read the same logical chunk of 16 consecutive rows.
//  V: a transposing read covers 64 bytes of each of 8 consecutive rows;
//     rows 4k..4k+3 are moved 0 / 64 / 128 / 192 bytes apart.
template <int CPR>
__device__ __forceinline__ int k_swz(int r) { return r & (CPR - 1); }
template <int CPR>
__device__ __forceinline__ int v_swz(int r) { return ((r & 3) << 2) & (CPR - 1); }
//  V^T (rows of 64 keys = 128 bytes, two rows per 256-byte bank line): the
//  16 rows a wave reads together get distinct 16-byte bank groups.
__device__ __forceinline__ int vt_swz(int r) { return (r >> 1) & 7; }

// Copies N wave-wide 16-byte-per-lane rows of a tile straight into LDS
// (buffer_load ... lds): load i lands at lds + i KB, lane l at +16*l; lane l
// fetches base + voff[i].  The buffer descriptor spans nbytes from base, so
// reads past it return zeros.  Device pass only.
template <int N>
__device__ __forceinline__ void lds_dma_tile(const char* base, int nbytes, char* lds, const uint32_t (&voff)[N]) {
#if defined(__HIP_DEVICE_COMPILE__)
  const __amdgpu_buffer_rsrc_t r = __builtin_amdgcn_make_buffer_rsrc((void*)base, 0, nbytes, kBufferFlags);
#pragma unroll
  for (int i = 0; i < N; ++i)
    __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (__attribute__((address_space(3))) void*)(lds + i * 1024), 16,
                                             voff[i], 0, 0, 0);
#endif
}

// One wave-wide 16-byte-per-lane copy into LDS (see lds_dma_tile).  base and
// nbytes must be the same in every lane; they are read from the first lane
// so the compiler knows the descriptor is uniform (no per-lane loop).
__device__ __forceinline__ void lds_dma_one(const char* base, int nbytes, char* lds, uint32_t voff) {
#if defined(__HIP_DEVICE_COMPILE__)
  const uint64_t b = (uint64_t)base;
  const uint64_t ub = (uint64_t)(uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)b) |
                      ((uint64_t)(uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)(b >> 32)) << 32);
  const int un = __builtin_amdgcn_readfirstlane(nbytes);
  const __amdgpu_buffer_rsrc_t r = __builtin_amdgcn_make_buffer_rsrc((void*)ub, 0, un, kBufferFlags);
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (__attribute__((address_space(3))) void*)lds, 16, voff, 0, 0, 0);
#endif
}

// As lds_dma_one with the copy's LDS destination and source both advanced by
// the immediate IMM: copies of one wave into consecutive 1 KB pieces can share
// one LDS base (one M0 value) and pass voff - IMM.  The hardware range check
// covers voffset + IMM.
template <int IMM>
__device__ __forceinline__ void lds_dma_imm(const char* base, int nbytes, char* lds, uint32_t voff) {
#if defined(__HIP_DEVICE_COMPILE__)
  const uint64_t b = (uint64_t)base;
  const uint64_t ub = (uint64_t)(uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)b) |
                      ((uint64_t)(uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)(b >> 32)) << 32);
  const int un = __builtin_amdgcn_readfirstlane(nbytes);
  const __amdgpu_buffer_rsrc_t r = __builtin_amdgcn_make_buffer_rsrc((void*)ub, 0, un, kBufferFlags);
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (__attribute__((address_space(3))) void*)lds, 16, voff, 0, IMM, 0);
#endif
}

typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) i16x4 lds_i16x4;

// Transposing LDS read (gfx950 ds_read_b64_tr_b16): within each 16-lane
// group, output lane j element e is element (j mod 4) of the 8 bytes input
// lane 4e + j/4 points at.
__device__ __forceinline__ i16x4 lds_read_tr(const char* p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(p));
}

// Block-local bf16 attention for the shapes outside the block-aligned
// kernels' range (D = 128, blocks of more than 32 frames, windows of more
// than 64 keys): 4 waves = 128 query rows of one (batch row, head).  The keys
// of the union of the tile rows' windows stream through two LDS buffer pairs
// in 64-key tiles (K one tile ahead of V), and every row is masked to its own
// window.  Within a tile step the softmax of this tile's scores is
// interleaved with the S MFMAs of the next tile, and the row sums with the PV
// MFMAs.
template <int D>
__global__ void __launch_bounds__(256, 2) block_local_tiled_bf16_kernel(AttnArgs a) {
  constexpr int WAVES = 4;
  using G = Bf16Geo<D, WAVES, 64>;
  constexpr int BM = 32 * WAVES;
  // Two separate buffers (not one indexed array) so that the compiler sees
  // the prefetch into one never aliases the reads of the other.
  __shared__ __attribute__((aligned(16))) char k0[G::kTileBytes];
  __shared__ __attribute__((aligned(16))) char v0[G::kTileBytes];
  __shared__ __attribute__((aligned(16))) char k1[G::kTileBytes];
  __shared__ __attribute__((aligned(16))) char v1[G::kTileBytes];

  const TileRange tr = tile_range<BM, G::BN, true>(a);

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int ql = lane & 31;
  const int g = lane >> 5;
  const int H = a.H;
  const int h = tr.h;
  const int64_t row_stride = (int64_t)H * D;  // elements between consecutive tokens

  // Query row of this lane: wave*32 + ql of the tile, and its key window.
  const int wave_row0 = tr.q0 + wave * 32;
  const bool wave_active = wave_row0 < tr.q1;
  const int my_row = wave_row0 + ql;
  int lo, hi;
  window_of(a, min(tr.seq_q0 + wave * 32 + ql, a.n - 1), lo, hi);

  // Q operand of S^T = K Q^T: lane (ql, g) holds features ds*16 + 8g .. +7.
  bf16x8 qf[G::NDS];
  {
    const int qrow = min(my_row, tr.q1 - 1);
    const bf16x8* qp = (const bf16x8*)((const __bf16*)a.q + (int64_t)qrow * row_stride + (int64_t)h * D + g * 8);
#pragma unroll
    for (int ds = 0; ds < G::NDS; ++ds) qf[ds] = qp[2 * ds];
  }

  // Direct global -> LDS copy of one tile: wave w's load i fills LDS bytes
  // [(L*w + i) KB, +1 KB) (L loads per wave); lane l lands on row
  // (L*w+i)*RPI + l/CPR, physical chunk l % CPR, and so fetches logical chunk
  // (l % CPR) ^ swz(row).
  const int ld_row_in_blk = lane / G::CPR;
  const int ld_pchunk = lane % G::CPR;
  const uint32_t rs_bytes = (uint32_t)(row_stride * 2);
  uint32_t ld_koff[G::kLoadsPerWave], ld_voff[G::kLoadsPerWave];
#pragma unroll
  for (int i = 0; i < G::kLoadsPerWave; ++i) {
    const int row = (G::kLoadsPerWave * wave + i) * G::RPI + ld_row_in_blk;
    ld_koff[i] = (uint32_t)row * rs_bytes + (ld_pchunk ^ k_swz<G::CPR>(row)) * 16;
    ld_voff[i] = (uint32_t)row * rs_bytes + (ld_pchunk ^ v_swz<G::CPR>(row)) * 16;
  }
  const char* kbase = (const char*)a.k + ((int64_t)tr.kv_base * row_stride + (int64_t)h * D) * 2;
  const char* vbase = (const char*)a.v + ((int64_t)tr.kv_base * row_stride + (int64_t)h * D) * 2;

  // Buffer descriptors cover only the tile's valid rows, so the hardware
  // range check returns zeros for rows past the window's end (their scores
  // are masked).  MUBUF loads (not FLAT) keep LDS waits precise.
  auto tile_bytes = [&](int tile) {
    const int valid = min(G::BN, tr.k_hi - (tr.k_lo + tile * G::BN));
    return (valid - 1) * (int)rs_bytes + G::ROW;
  };
  auto issue_k = [&](int tile, char* kdst) {
    lds_dma_tile<G::kLoadsPerWave>(kbase + (int64_t)(tr.k_lo + tile * G::BN) * rs_bytes, tile_bytes(tile),
                                   kdst + G::kLoadsPerWave * wave * 1024, ld_koff);
  };
  auto issue_v = [&](int tile, char* vdst) {
    lds_dma_tile<G::kLoadsPerWave>(vbase + (int64_t)(tr.k_lo + tile * G::BN) * rs_bytes, tile_bytes(tile),
                                   vdst + G::kLoadsPerWave * wave * 1024, ld_voff);
  };

  // Per-lane LDS read offsets.
  //  K operand (rows = keys, k = features): lane (ql, g), step ds reads
  //  logical chunk 2ds+g of row kb*32+ql.
  int k_rd[G::NDS];
#pragma unroll
  for (int ds = 0; ds < G::NDS; ++ds) k_rd[ds] = ql * G::ROW + (((2 * ds + g) ^ k_swz<G::CPR>(ql)) * 16);
  //  V^T operand via transposing reads: in 16-lane group G' (lane-half g =
  //  G'/2, feature half G' % 2), input lane i points at row 4g + i/4 (and
  //  + 8 for elements 4..7) of the 16-key chunk, features
  //  db*32 + 16*(G' % 2) + 4*(i % 4) .. +3.  Element e of output lane j is
  //  then V[key 4g+e (or 8+4g+e-4)][db*32 + 16*(G'%2) + j], which is the k-slot
  //  order of the P operand taken from the score registers.
  const int grp = lane >> 4;
  const int gi = lane & 15;
  const int v_row = 4 * (grp >> 1) + (gi >> 2);
  int v_rd[G::NDB];
#pragma unroll
  for (int db = 0; db < G::NDB; ++db) {
    const int byte_in_row = db * 64 + 32 * (grp & 1) + 8 * (gi & 3);
    const int chunk = (byte_in_row >> 4) ^ v_swz<G::CPR>(v_row);
    v_rd[db] = v_row * G::ROW + chunk * 16 + (byte_in_row & 15);
  }

  RowState<G::NKB, G::NDB> st;
  st.init();

  const int nkeys = tr.k_hi - tr.k_lo;
  const int ntiles = (nkeys + G::BN - 1) / G::BN;

  // ---- S^T = K Q^T.  Step `step` = (ds, kb) with kb fastest.
  constexpr int NSTEP_S = G::NKB * G::NDS;
  constexpr int KPF = 3;  // K operand steps read ahead of their MFMAs
  auto read_k = [&](const char* kl, int step) {
    return *(const bf16x8*)(kl + (step % G::NKB) * 32 * G::ROW + k_rd[step / G::NKB]);
  };
  auto qk = [&](const char* kl, f32x16(&s)[G::NKB]) {
#pragma unroll
    for (int kb = 0; kb < G::NKB; ++kb) s[kb] = f32x16{};
    bf16x8 ka[KPF + 1];
#pragma unroll
    for (int i = 0; i < KPF; ++i) ka[i] = read_k(kl, i);
#pragma unroll
    for (int step = 0; step < NSTEP_S; ++step) {
      if (step + KPF < NSTEP_S) ka[(step + KPF) % (KPF + 1)] = read_k(kl, step + KPF);
      VL_SCHED_BARRIER(0);
      s[step % G::NKB] =
          __builtin_amdgcn_mfma_f32_32x32x16_bf16(ka[step % (KPF + 1)], qf[step / G::NKB], s[step % G::NKB], 0, 0, 0);
      VL_SCHED_BARRIER(0);
    }
  };

  // ---- Row max of the tile's scores and the lazy rescale; returns -offset.
  auto row_max = [&](f32x16(&s)[G::NKB]) {
    float mx = -INFINITY;
#pragma unroll
    for (int kb = 0; kb < G::NKB; ++kb)
#pragma unroll
      for (int j = 0; j < 16; ++j) mx = fmaxf(mx, s[kb][j]);
    mx = pair_max(mx);
    const float mx_c = mx * a.c;
    const bool need = mx_c > st.m_c + 8.0f;
    if (__ballot(need)) {
      const float m_new = need ? mx_c : st.m_c;
      const float alpha = need ? __builtin_amdgcn_exp2f(st.m_c - m_new) : 1.0f;
      st.l *= alpha;
#pragma unroll
      for (int d = 0; d < G::NDB; ++d) st.o[d] *= alpha;
      st.m_c = m_new;
    }
    return (st.m_c == -INFINITY) ? 0.f : -st.m_c;
  };

  // ---- exp2 / bf16 conversion of this tile's scores into the P operands,
  // interleaved with the S MFMAs of the next tile: per S step, one K read,
  // one MFMA and the VALU work of kScoresPerStep scores.  On the window's
  // last tile the next-tile product reads a stale buffer and is never used;
  // keeping it makes the exp work and the MFMAs one block.
  auto softmax_qk = [&](f32x16(&sc)[G::NKB], bf16x8(&pf)[G::NKC], float negm, const char* kl_next,
                        f32x16(&sn)[G::NKB], auto&& load_step) {
    constexpr int kScoresPerStep = G::NKB * 16 / NSTEP_S;  // each lane holds NKB*16 scores
    static_assert(kScoresPerStep * NSTEP_S == G::NKB * 16, "whole scores per step");
    static_assert(NSTEP_S >= 2 * G::kLoadsPerWave, "one tile load per S step at most");
#pragma unroll
    for (int kb = 0; kb < G::NKB; ++kb) sn[kb] = f32x16{};
    bf16x8 ka[KPF + 1];
#pragma unroll
    for (int i = 0; i < KPF; ++i) ka[i] = read_k(kl_next, i);
#pragma unroll
    for (int step = 0; step < NSTEP_S; ++step) {
      if (step + KPF < NSTEP_S) ka[(step + KPF) % (KPF + 1)] = read_k(kl_next, step + KPF);
      const bool dma = load_step(step);
      sn[step % G::NKB] =
          __builtin_amdgcn_mfma_f32_32x32x16_bf16(ka[step % (KPF + 1)], qf[step / G::NKB], sn[step % G::NKB], 0, 0, 0);
#pragma unroll
      for (int t = 0; t < kScoresPerStep; ++t) {
        const int idx = step * kScoresPerStep + t;
        const float p = __builtin_amdgcn_exp2f(fmaf(sc[idx >> 4][idx & 15], a.c, negm));
        sc[idx >> 4][idx & 15] = p;
        if ((idx & 7) == 7) {
          const int kc = idx >> 3;
#pragma unroll
          for (int e = 0; e < 8; ++e) pf[kc][e] = (__bf16)sc[kc >> 1][8 * (kc & 1) + e];
        }
      }
      VL_SCHED_GROUP(0x008, 1, 0);                         // the step's MFMA
      VL_SCHED_GROUP(0x100, 1, 0);                         // 1 LDS read
      if (dma) VL_SCHED_GROUP(0x020, 1, 0);                // 1 tile load into LDS
      // the scores' VALU work: fma and exp per score, one bf16 pair
      // conversion per two scores
      VL_SCHED_GROUP(0x002, 2 * kScoresPerStep + kScoresPerStep / 2, 0);
    }
  };

  // ---- O^T += V^T P^T, V^T operands VPF steps ahead.
  auto read_v = [&](const char* vl, int kc, int db) {
    const char* p = vl + kc * 16 * G::ROW + v_rd[db];
    const i16x4 lo4 = lds_read_tr(p);
    const i16x4 hi4 = lds_read_tr(p + 8 * G::ROW);
    return __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo4, hi4, 0, 1, 2, 3, 4, 5, 6, 7));
  };
  // The row sums of this tile's probabilities (still in the score registers,
  // which the next tile's scores do not overwrite before its softmax) are
  // added here, a few per MFMA, where the VALU is otherwise idle.
  auto pv = [&](const char* vl, const bf16x8(&pf)[G::NKC], const f32x16(&sc)[G::NKB]) {
    constexpr int VPF = 6;
    constexpr int NSTEP = G::NKC * G::NDB;
    constexpr int kSumPerStep = G::NKB * 16 / NSTEP;
    static_assert(kSumPerStep * NSTEP == G::NKB * 16, "whole scores per step");
    float ls[2] = {0.f, 0.f};
    bf16x8 va[VPF + 1];
#pragma unroll
    for (int step = 0; step < VPF; ++step) va[step] = read_v(vl, step / G::NDB, step % G::NDB);
#pragma unroll
    for (int step = 0; step < NSTEP; ++step) {
      if (step + VPF < NSTEP)
        va[(step + VPF) % (VPF + 1)] = read_v(vl, (step + VPF) / G::NDB, (step + VPF) % G::NDB);
      VL_SCHED_BARRIER(0);
      st.o[step % G::NDB] =
          __builtin_amdgcn_mfma_f32_32x32x16_bf16(va[step % (VPF + 1)], pf[step / G::NDB], st.o[step % G::NDB], 0, 0, 0);
#pragma unroll
      for (int t = 0; t < kSumPerStep; ++t) {
        const int idx = step * kSumPerStep + t;
        ls[t & 1] += sc[idx >> 4][idx & 15];
      }
      // an opaque use keeps the adds in this step (they would otherwise
      // sink to the sums' only use after the loop)
      asm volatile("" : "+v"(ls[0]), "+v"(ls[1]));
      VL_SCHED_BARRIER(0);
    }
    st.l += ls[0] + ls[1];
  };

  // One tile: S of this tile is in sc; K of the next tile is in kl_next
  // (when there is one), V of this tile in vl.
  bf16x8 pf[G::NKC];
  // The wave's share of the next tiles' loads (K of tile kt into kdst, V of
  // tile vt into vdst; -1 = none) is spread one load per S step so the
  // copies stream while the MFMAs run instead of stalling issue in a burst.
  auto tile_step = [&](int tile, f32x16(&sc)[G::NKB], f32x16(&sn)[G::NKB], const char* kl_next, const char* vl,
                       int kt, char* kdst, int vt, char* vdst) {
    mask_scores<G::NKB>(sc, tr.k_lo + tile * G::BN, g, lo, hi);
    const float negm = row_max(sc);
    // No next tile (kt or vt < 0): the copy still issues, with a zero-byte
    // descriptor, so it reads nothing; its destination buffer is not read
    // during this step.  Keeping it unconditional keeps the whole step one
    // branch-free region for the instruction-group schedule below.
    const char* ksrc = kt >= 0 ? kbase + (int64_t)(tr.k_lo + kt * G::BN) * rs_bytes : kbase;
    const char* vsrc = vt >= 0 ? vbase + (int64_t)(tr.k_lo + vt * G::BN) * rs_bytes : vbase;
    const int kbytes = kt >= 0 ? tile_bytes(kt) : 0;
    const int vbytes = vt >= 0 ? tile_bytes(vt) : 0;
    auto load_step = [&](int step) {
      constexpr int L = G::kLoadsPerWave;
      if (step < L) {
        lds_dma_one(ksrc, kbytes, kdst + (L * wave + step) * 1024, ld_koff[step]);
        return true;
      }
      if (step < 2 * L) {
        lds_dma_one(vsrc, vbytes, vdst + (L * wave + step - L) * 1024, ld_voff[step - L]);
        return true;
      }
      return false;
    };
    softmax_qk(sc, pf, negm, kl_next, sn, load_step);
    pv(vl, pf, sc);
  };

  // K runs one tile ahead of V: during tile t the waves read K(t+1) and V(t)
  // while K(t+2) and V(t+1) stream into the buffers that held K(t) and
  // V(t-1); one barrier per tile separates the two.
  f32x16 sA[G::NKB], sB[G::NKB];
  if (ntiles > 0) {
    issue_k(0, k0);
    issue_v(0, v0);
  }
  if (ntiles > 1) issue_k(1, k1);
  __builtin_amdgcn_s_waitcnt(kWaitVm0);
  __syncthreads();
  if (wave_active && ntiles > 0) qk(k0, sA);
  __syncthreads();
  for (int it = 0; it < ntiles; it += 2) {
    {
      const int kt = it + 2 < ntiles ? it + 2 : -1;
      const int vt = it + 1 < ntiles ? it + 1 : -1;
      if (wave_active) {
        tile_step(it, sA, sB, k1, v0, kt, k0, vt, v1);
      } else {
        if (kt >= 0) issue_k(kt, k0);
        if (vt >= 0) issue_v(vt, v1);
      }
    }
    __builtin_amdgcn_s_waitcnt(kWaitVm0);
    __syncthreads();
    if (it + 1 >= ntiles) break;
    {
      const int kt = it + 3 < ntiles ? it + 3 : -1;
      const int vt = it + 2 < ntiles ? it + 2 : -1;
      if (wave_active) {
        tile_step(it + 1, sB, sA, k0, v1, kt, k1, vt, v0);
      } else {
        if (kt >= 0) issue_k(kt, k1);
        if (vt >= 0) issue_v(vt, v0);
      }
    }
    __builtin_amdgcn_s_waitcnt(kWaitVm0);
    __syncthreads();
  }

  if (!wave_active) return;
  const float l_tot = pair_sum(st.l);
  const float inv = l_tot > 0.f ? 1.0f / l_tot : 0.f;
  if (my_row < tr.q1) {
    __bf16* op = (__bf16*)a.out + (int64_t)my_row * row_stride + (int64_t)h * D;
#pragma unroll
    for (int db = 0; db < G::NDB; ++db)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int d = db * 32 + 8 * i + 4 * g;
        typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
        bf16x4 w;
#pragma unroll
        for (int e = 0; e < 4; ++e) w[e] = (__bf16)(st.o[db][4 * i + e] * inv);
        *(bf16x4*)(op + d) = w;
      }
    if (a.lse != nullptr && g == 0)
      a.lse[(int64_t)my_row * H + h] = l_tot > 0.f ? (st.m_c + log2f(l_tot)) * kLn2 : -INFINITY;
  }
}

// ---------------------------------------------------------------- bf16 ping-pong kernel

// Chiplet work queues (the workspace launch).  The chiplets of one device
// run at different clocks (the card sits at its power limit; 1.58-1.80 GHz
// measured per chiplet), so a fixed share of the work per chiplet leaves the
// fast ones idle at the end.  Queue x holds, in order, exactly the logical
// items the static map gives chiplet x: item k of the queue is logical
// ((k div chunk) * 8 + x) * chunk + k mod chunk, the item of the k-th block
// on that chiplet.  A work-group takes the next item of its own chiplet's
// queue with one atomic ticket and, once that queue is empty, the next item
// of another queue that still has some, so faster chiplets take on more of
// the work while each run of `chunk` items (one request and head: the same
// K/V) still starts on one chiplet.  Lane j < 8 holds c, its read of queue
// x + j's counter; only queues that still had items get a ticket request, so
// the spare work-groups past the last item take no atomic.  Returns the
// logical item, or -1 when every queue is empty.  n_items: logical items of
// the launch.  Called by a whole wave; the result is wave-uniform.  At most
// eight tickets are tried: no work-group waits on another.
__device__ __forceinline__ int queue_len(int n_items, int chunk, int y) {
  const int per8 = kXcds * chunk;
  const int full = n_items / per8;
  return full * chunk + min(chunk, max(0, n_items - full * per8 - y * chunk));
}
__device__ __forceinline__ int take_item(int* cnt, int n_items, int chunk, int x, int c) {
  const int lane = lane_id();
  uint64_t avail = __ballot(lane < kXcds && c < queue_len(n_items, chunk, (x + lane) % kXcds));
  while (avail != 0) {
    const int j = __ffsll((unsigned long long)avail) - 1;  // own queue first, then the next ones
    const int qy = (x + j) % kXcds;
    int k = 0;
    if (lane == 0) k = atomicAdd(cnt + qy, 1);
    k = __builtin_amdgcn_readfirstlane(k);
    if (k < queue_len(n_items, chunk, qy)) return ((k / chunk) * kXcds + qy) * chunk + k % chunk;
    avail &= ~(1ull << j);
  }
  return -1;
}

// Work-group barrier without a memory fence: LDS copies are waited for
// explicitly (vmcnt) before it, and the "memory" clobber keeps the compiler
// from moving loads or stores across it.
__device__ __forceinline__ void wg_barrier() { asm volatile("s_barrier" ::: "memory"); }

// Varlen bf16 attention with 8 waves in two groups of four.  Waves w and
// w + 4 share a SIMD, so each SIMD runs one wave of each group.  A wave
// handles tile t in two phases: an MFMA phase (O += V(t-1)^T P(t-1)^T with
// the row sums of P(t-1), then S(t) = K(t) Q^T: 36 MFMAs) and a VALU phase
// (mask, row max, lazy rescale, exp2 and bf16 pack of P(t)).  Group 1 runs one phase behind group
// 0 and every phase ends at a work-group barrier, so on each SIMD one wave
// issues MFMAs while the other does the softmax arithmetic.
// K and V tiles rotate through three LDS buffers each.  In phase 2j the
// waves copy K(j+2) and V(j+1) in; those buffers last held K(j-1) and
// V(j-2), which both groups finished in phases 2j-2 and 2j-1.  At the end of
// phase 2j each wave waits for its copies of phase 2j-2, so K(j+1) and V(j)
// are complete for phase 2j+2, where group 0 first reads them.  The phase
// loop is unrolled six times so every LDS access names one __shared__ array
// and the compiler's LDS-copy waits stay precise.
// kVt: V tiles come from the staged V^T (a.vt) as D rows of BN keys, so the
// V^T operands are plain 16-byte LDS reads instead of transposing 8-byte
// reads (which move half as many bytes per LDS cycle and need their
// addresses computed on the VALU).
template <int D, int BN, bool kVt>
__global__ void __launch_bounds__(512, 1) attn_bf16_pp_kernel(AttnArgs a) {
  using G = Bf16Geo<D, 8, BN>;
  static_assert(!kVt || BN == kVtTile, "V^T tiles are whole padded 64-key groups");
  constexpr int VROW = BN * 2;       // bytes per V^T row (one tile's keys of one feature)
  constexpr int VRPI = 1024 / VROW;  // V^T rows per wave-wide 16-byte load
  constexpr int BM = 256;
  constexpr int L = G::kLoadsPerWave;
  __shared__ __attribute__((aligned(16))) char k0[G::kTileBytes];
  __shared__ __attribute__((aligned(16))) char k1[G::kTileBytes];
  __shared__ __attribute__((aligned(16))) char k2[G::kTileBytes];
  __shared__ __attribute__((aligned(16))) char v0[G::kTileBytes];
  __shared__ __attribute__((aligned(16))) char v1[G::kTileBytes];
  __shared__ __attribute__((aligned(16))) char v2[G::kTileBytes];

  // Queue launch: wave 0 takes the ticket, decodes the item once and hands
  // the tile to the other waves through LDS.  With at most kLptMaxReqs
  // requests it loads their bounds beside the queue counters, before the
  // ticket, and decodes from registers; otherwise through tile_range.
  TileRange tr;
  if (a.dyn != nullptr) {
    __shared__ TileRange tr_s;
    if (threadIdx.x < 64) {
      const int x = (int)(blockIdx.x % kXcds);
      int c = 0;
      if (threadIdx.x < kXcds)
        c = __hip_atomic_load(a.dyn + (x + threadIdx.x) % kXcds, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      TileRange t0;
      if (a.R <= kLptMaxReqs) {
        const ReqLanes rl = load_req_lanes(a.q_cu, a.kv_cu, a.R);
        const SplitPlan sp = split_plan(total_tiles_lanes(rl, a.R, a.H, BM), a.slots, a.max_kv);
        const int n_items = sp.parts > 1 ? sp.full + sp.tail * sp.parts : sp.full;
        t0 = item_range_lanes<BM, BN>(a, rl, sp, take_item(a.dyn, n_items, a.chunk, x, c));
      } else {
        const int T = total_tiles(a.q_cu, a.R, a.H, BM);
        const SplitPlan sp = split_plan(T, a.slots, a.max_kv);
        const int n_items = sp.parts > 1 ? sp.full + sp.tail * sp.parts : T;
        t0 = tile_range<BM, BN, false>(a, take_item(a.dyn, n_items, a.chunk, x, c));
      }
      if (threadIdx.x == 0) tr_s = t0;
    }
    __syncthreads();
    tr.valid = tr_s.valid;
    tr.h = __builtin_amdgcn_readfirstlane(tr_s.h);
    tr.q0 = __builtin_amdgcn_readfirstlane(tr_s.q0);
    tr.q1 = __builtin_amdgcn_readfirstlane(tr_s.q1);
    tr.kv_base = __builtin_amdgcn_readfirstlane(tr_s.kv_base);
    tr.k_lo = __builtin_amdgcn_readfirstlane(tr_s.k_lo);
    tr.k_hi = __builtin_amdgcn_readfirstlane(tr_s.k_hi);
    tr.seq_q0 = __builtin_amdgcn_readfirstlane(tr_s.seq_q0);
    tr.unit = __builtin_amdgcn_readfirstlane(tr_s.unit);
    tr.req = __builtin_amdgcn_readfirstlane(tr_s.req);
  } else {
    tr = tile_range<BM, BN, false>(a);
  }
  if (!tr.valid) return;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int grp = wave >> 2;
  const int ql = lane & 31;
  const int g = lane >> 5;
  const int H = a.H;
  const int h = tr.h;
  const int64_t row_stride = (int64_t)H * D;
  const int my_row = tr.q0 + wave * 32 + ql;
  const bool wave_active = tr.q0 + wave * 32 < tr.q1;

  // Q operand of S^T = K Q^T: lane (ql, g) holds features ds*16 + 8g .. +7.
  bf16x8 qf[G::NDS];
  {
    const int qrow = min(my_row, tr.q1 - 1);
    const bf16x8* qp = (const bf16x8*)((const __bf16*)a.q + (int64_t)qrow * row_stride + (int64_t)h * D + g * 8);
#pragma unroll
    for (int ds = 0; ds < G::NDS; ++ds) qf[ds] = qp[2 * ds];
  }

  // Copy offsets (see the 4-wave kernel): wave w's load i fills LDS bytes
  // [(L*w + i) KB, +1 KB) of a tile buffer.
  const int ld_row_in_blk = lane / G::CPR;
  const int ld_pchunk = lane % G::CPR;
  const uint32_t rs_bytes = (uint32_t)(row_stride * 2);
  // Prologue copies: all 8 waves, L loads each per tile.
  // V^T copies: lane l of load i lands on feature row i*VRPI + l/8 at
  // physical chunk l%8 and fetches logical chunk (l%8) ^ vt_swz(row).
  const uint32_t vt_rs = (uint32_t)(a.vt_ld * 2);
  auto vt_off = [&](int load) {
    const int row = load * VRPI + lane / 8;
    return (uint32_t)row * vt_rs + (((lane & 7) ^ vt_swz(row)) * 16);
  };
  uint32_t ld_koff[L], ld_voff[L];
#pragma unroll
  for (int i = 0; i < L; ++i) {
    const int row = (L * wave + i) * G::RPI + ld_row_in_blk;
    ld_koff[i] = (uint32_t)row * rs_bytes + (ld_pchunk ^ k_swz<G::CPR>(row)) * 16;
    ld_voff[i] = kVt ? vt_off(L * wave + i) : (uint32_t)row * rs_bytes + (ld_pchunk ^ v_swz<G::CPR>(row)) * 16;
  }
  // Loop copies: the four waves of one group move a whole tile, 2L loads each;
  // group 1 copies K (rows by K swizzle), group 0 copies V.
  constexpr int L2 = 2 * L;
  const int gw = wave & 3;
  // (ld_goff[i] >= 1024 i: load i starts at row >= i * 1024 / row bytes, and
  // every source row is at least that many bytes apart)
  uint32_t ld_goff[L2];
#pragma unroll
  for (int i = 0; i < L2; ++i) {
    const int row = (L2 * gw + i) * G::RPI + ld_row_in_blk;
    const int swz = grp == 1 ? k_swz<G::CPR>(row) : v_swz<G::CPR>(row);
    ld_goff[i] = (kVt && grp == 0) ? vt_off(L2 * gw + i) : (uint32_t)row * rs_bytes + (ld_pchunk ^ swz) * 16;
  }
  const char* kbase = (const char*)a.k + ((int64_t)tr.kv_base * row_stride + (int64_t)h * D) * 2;
  const char* vbase =
      kVt ? (const char*)a.vt + ((int64_t)h * D * a.vt_ld + vt_col_base(tr.kv_base, tr.req)) * 2
          : (const char*)a.v + ((int64_t)tr.kv_base * row_stride + (int64_t)h * D) * 2;
  const int nkeys = tr.k_hi - tr.k_lo;
  const int ntiles = (nkeys + BN - 1) / BN;
  const bool ragged = (nkeys % BN) != 0;
  // Source and byte count of tile `tile`; past the last tile a zero-byte
  // descriptor reads nothing (the copy still issues, keeping wait counts uniform).
  // A V^T tile is D whole rows of BN keys (zero-filled past the request).
  auto tile_src = [&](const char* base, bool is_vt, int tile, const char*& src, int& nb) {
    const bool ok = tile < ntiles;
    if (is_vt) {
      src = ok ? base + (int64_t)(tr.k_lo + tile * BN) * 2 : base;
      nb = ok ? (D - 1) * (int)vt_rs + VROW : 0;
    } else {
      src = ok ? base + (int64_t)(tr.k_lo + tile * BN) * rs_bytes : base;
      nb = ok ? (min(BN, nkeys - tile * BN) - 1) * (int)rs_bytes + G::ROW : 0;
    }
  };
  // Tile `tile` of K or V into dst, this wave's share of an all-wave copy.
  auto copy_tile = [&](const char* base, bool is_vt, int tile, char* dst, const uint32_t(&off)[L]) {
    const char* src;
    int nb;
    tile_src(base, is_vt, tile, src, nb);
#pragma unroll
    for (int i = 0; i < L; ++i) lds_dma_one(src, nb, dst + (L * wave + i) * 1024, off[i]);
  };

  // LDS read offsets of the MFMA operands (see the 4-wave kernel).
  int k_rd[G::NDS];
#pragma unroll
  for (int ds = 0; ds < G::NDS; ++ds) k_rd[ds] = ql * G::ROW + (((2 * ds + g) ^ k_swz<G::CPR>(ql)) * 16);
  const int vgrp = lane >> 4;
  const int gi = lane & 15;
  const int v_row = 4 * (vgrp >> 1) + (gi >> 2);
  int v_rd[G::NDB];
#pragma unroll
  for (int db = 0; db < G::NDB; ++db) {
    const int byte_in_row = db * 64 + 32 * (vgrp & 1) + 8 * (gi & 3);
    const int chunk = (byte_in_row >> 4) ^ v_swz<G::CPR>(v_row);
    v_rd[db] = v_row * G::ROW + chunk * 16 + (byte_in_row & 15);
  }
  //  V^T operand from a V^T tile: lane (ql, g), step (kc, db) reads logical
  //  chunk 2kc+g (stored keys 16kc + 8g .. +7, in P's k-slot order) of
  //  feature row db*32 + ql.
  // The V buffers sit above the 64 KB that a ds_read immediate offset can
  // reach, so each read offset is kept with a bias of kVtBias in a register
  // the compiler cannot see through; the buffer's address minus the bias plus
  // the feature block's offset then fits the immediate field, and no VALU
  // address add is needed per read.
  constexpr int kVtBias = 3 * G::kTileBytes;
  int vt_rd[G::NKC];
#pragma unroll
  for (int kc = 0; kc < G::NKC; ++kc) {
    vt_rd[kc] = ql * VROW + (((2 * kc + g) ^ vt_swz(ql)) * 16) + kVtBias;
    asm volatile("" : "+v"(vt_rd[kc]));
  }

  RowState<G::NKB, G::NDB> st;
  st.init();
  f32x16 s[G::NKB];
  bf16x8 pf[G::NKC];
#pragma unroll
  for (int kc = 0; kc < G::NKC; ++kc) pf[kc] = bf16x8{};
  // Row sums of P on the matrix cores: a 16x16x32 MFMA reads the P^T operand
  // registers of the 32x32x16 PV step as its B operand (lane l: keys of its
  // lane group l/16, query n = l%16 of lanes l%32 < 16, n + 16 of the others)
  // and an A operand whose row 0 sums lane groups 0 and 2 and row 1 groups 1
  // and 3, so result rows 0 and 1 (lanes 0..15, registers 0 and 1) are the
  // 16-key sums of queries n and n + 16.  lsum holds the sums since the last
  // rescale; st.l takes them over at every rescale and at the end.
  f32x4 lsum = {};
  bf16x8 ones_sel;
  {
    const __bf16 one = (lane & 15) == ((lane >> 4) & 1) ? (__bf16)1.0f : (__bf16)0.0f;
#pragma unroll
    for (int e = 0; e < 8; ++e) ones_sel[e] = one;
  }
  // the lazy rescale threshold (offset + 8) and the negated offset (0 while
  // no score has been seen), both changed only by a rescale
  float m_thr = -INFINITY, neg_m = 0.f;
  // this lane's query's share of lsum (the whole row sum on lane half 0)
  auto lsum_row = [&]() {
    const int src = (ql & 15) * 4;
    const float a0 = __int_as_float(__builtin_amdgcn_ds_bpermute(src, __float_as_int(lsum[0])));
    const float a1 = __int_as_float(__builtin_amdgcn_ds_bpermute(src, __float_as_int(lsum[1])));
    return g == 0 ? (ql < 16 ? a0 : a1) : 0.f;
  };

  // ---- MFMA phase of tile k: PV of tile k-1 (V in vl), then S of tile k (K
  // in kl), as one stream of operand reads running PF steps ahead of the
  // MFMAs, so the S part starts without waiting for its first reads.  Every
  // phase runs both parts: in the first (k = 0) P is still zero (and the V
  // buffer read was zeroed), after the last tile the scores are discarded.
  auto m_phase = [&](const char* kl, const char* vl) {
    constexpr int PF = 6;
    constexpr int NV = G::NKC * G::NDB;
    constexpr int NK = G::NKB * G::NDS;
    auto read_op = [&](int i) {
      if (i < NV) {
        if constexpr (kVt) {
          return *(const bf16x8*)(vl + (((i % G::NDB) * 32 * VROW - kVtBias) + vt_rd[i / G::NDB]));
        } else {
          const char* p = vl + (i / G::NDB) * 16 * G::ROW + v_rd[i % G::NDB];
          const i16x4 lo4 = lds_read_tr(p);
          const i16x4 hi4 = lds_read_tr(p + 8 * G::ROW);
          return __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo4, hi4, 0, 1, 2, 3, 4, 5, 6, 7));
        }
      }
      const int ks = i - NV;  // key step of the S part
      return *(const bf16x8*)(kl + (ks % G::NKB) * 32 * G::ROW + k_rd[ks / G::NKB]);
    };
    bf16x8 op[PF + 1];
#pragma unroll
    for (int i = 0; i < PF; ++i) op[i] = read_op(i);
#pragma unroll
    for (int i = 0; i < NV + NK; ++i) {
      if (i + PF < NV + NK) op[(i + PF) % (PF + 1)] = read_op(i + PF);
      VL_SCHED_BARRIER(0);
      if (i < NV) {
        st.o[i % G::NDB] =
            __builtin_amdgcn_mfma_f32_32x32x16_bf16(op[i % (PF + 1)], pf[i / G::NDB], st.o[i % G::NDB], 0, 0, 0);
        if (i % G::NDB == 0) lsum = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ones_sel, pf[i / G::NDB], lsum, 0, 0, 0);
      } else {
        const int ks = i - NV;
        const f32x16 acc = ks < G::NKB ? f32x16{} : s[ks % G::NKB];
        s[ks % G::NKB] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(op[i % (PF + 1)], qf[ks / G::NKB], acc, 0, 0, 0);
      }
      VL_SCHED_BARRIER(0);
    }
  };

  // ---- VALU phase of tile k: scores -> probabilities P(k) in bf16.  The
  // group's tile copy (copy(i), i < 2L) is issued spread over the exp loop.
  auto v_phase = [&](int k, auto&& copy) {
    if (!wave_active || k < 0 || k >= ntiles) {
#pragma unroll
      for (int i = 0; i < L2; ++i) copy(i);
      return;
    }
    // The empty asm statements keep the two rare paths (the sequence's last,
    // partial tile; a rescale) real branches: if-converted, their compares,
    // selects and 64 multiplies would run on every tile.
    if (ragged && k == ntiles - 1) {
      asm volatile("");
      mask_scores<G::NKB>(s, tr.k_lo + k * BN, g, tr.k_lo, tr.k_hi);
    }
    float mx = -INFINITY;
#pragma unroll
    for (int kb = 0; kb < G::NKB; ++kb)
#pragma unroll
      for (int j = 0; j < 16; ++j) mx = fmaxf(mx, s[kb][j]);
    mx = pair_max(mx);
    const float mx_c = mx * a.c;
    const bool need = mx_c > m_thr;
    if (__ballot(need)) {
      asm volatile("");
      // an integer offset: a weight under any other offset (a later rescale,
      // another key range of the same row) is the same value times a power of
      // two (up to the fp32 rounding of s*c - m), so its bf16 rounding does
      // not depend on where the offset was set; alpha is a power of two
      const float m_new = need ? ceilf(mx_c) : st.m_c;
      const float alpha = need ? __builtin_amdgcn_exp2f(st.m_c - m_new) : 1.0f;
      st.l = (st.l + lsum_row()) * alpha;
      lsum = f32x4{};
#pragma unroll
      for (int d = 0; d < G::NDB; ++d) st.o[d] *= alpha;
      st.m_c = m_new;
      m_thr = m_new + 8.0f;
      neg_m = (m_new == -INFINITY) ? 0.f : -m_new;
    }
    constexpr int kCopyEvery = G::NKB * 16 / L2;
#pragma unroll
    for (int kb = 0; kb < G::NKB; ++kb)
#pragma unroll
      for (int j = 0; j < 16; ++j) {
        if ((kb * 16 + j) % kCopyEvery == 0) copy((kb * 16 + j) / kCopyEvery);
        s[kb][j] = __builtin_amdgcn_exp2f(fmaf(s[kb][j], a.c, neg_m));
      }
#pragma unroll
    for (int kc = 0; kc < G::NKC; ++kc)
#pragma unroll
      for (int e = 0; e < 8; ++e) pf[kc][e] = (__bf16)s[kc >> 1][8 * (kc & 1) + e];
  };

  // ---- phase p0 + I of group GR (I, GR compile-time).  The MFMA phase of
  // phase p works on tile p/2: K buffer (p/2) % 3, V buffer (p/2 - 1) % 3.
  // The group in its VALU phase copies: in even phase p (group 1) K(p/2 + 2),
  // in odd phase p (group 0) V(p/2 + 1); it then waits for the copies it
  // issued two phases before, which the MFMA phase of phase p + 1 or later
  // reads first.  Then the barrier.
  auto phase = [&](int p0, auto I_, auto GR_) {
    constexpr int I = decltype(I_)::value;
    constexpr int GR = decltype(GR_)::value;
    char* const kbuf[3] = {k0, k1, k2};
    char* const vbuf[3] = {v0, v1, v2};
    const int p = p0 + I;
    if constexpr (((I - GR) & 1) == 0) {
      // the MFMA wave wins issue arbitration on its SIMD during its phase
      __builtin_amdgcn_s_setprio(2);
      const int k = (p - GR) / 2;
      if (wave_active && k <= ntiles) m_phase(kbuf[(I / 2) % 3], vbuf[(I / 2 + 2) % 3]);
      __builtin_amdgcn_s_setprio(0);
    } else {
      const char* src;
      int nb;
      char* dst;
      if constexpr ((I & 1) == 0) {
        tile_src(kbase, false, p / 2 + 2, src, nb);
        dst = kbuf[(I / 2 + 2) % 3];
      } else {
        tile_src(vbase, kVt, p / 2 + 1, src, nb);
        dst = vbuf[(I / 2 + 1) % 3];
      }
      // the wave's L2 copies share one LDS base; load i adds i KB as an immediate
      char* const wdst = dst + L2 * gw * 1024;
      v_phase((p - GR - 1) / 2, [&](int i) {
        static_assert(L2 <= 4, "immediate offsets up to 3 KB");
        switch (i) {
          case 0: lds_dma_imm<0>(src, nb, wdst, ld_goff[0]); break;
          case 1: lds_dma_imm<1024>(src, nb, wdst, ld_goff[1] - 1024); break;
          case 2: lds_dma_imm<2048>(src, nb, wdst, ld_goff[L2 > 2 ? 2 : 0] - 2048); break;
          default: lds_dma_imm<3072>(src, nb, wdst, ld_goff[L2 > 3 ? 3 : 0] - 3072); break;
        }
      });
      __builtin_amdgcn_s_waitcnt(kWaitVm0 | L2);
    }
    wg_barrier();
  };
  const int nphase = 2 * ntiles + 2;
  auto run = [&](auto GR) {
    using IC0 = std::integral_constant<int, 0>;
    using IC1 = std::integral_constant<int, 1>;
    using IC2 = std::integral_constant<int, 2>;
    using IC3 = std::integral_constant<int, 3>;
    using IC4 = std::integral_constant<int, 4>;
    using IC5 = std::integral_constant<int, 5>;
    for (int p0 = 0; p0 < nphase; p0 += 6) {
      phase(p0, IC0{}, GR);
      if (p0 + 1 >= nphase) break;
      phase(p0, IC1{}, GR);
      if (p0 + 2 >= nphase) break;
      phase(p0, IC2{}, GR);
      if (p0 + 3 >= nphase) break;
      phase(p0, IC3{}, GR);
      if (p0 + 4 >= nphase) break;
      phase(p0, IC4{}, GR);
      if (p0 + 5 >= nphase) break;
      phase(p0, IC5{}, GR);
    }
  };

  copy_tile(kbase, false, 0, k0, ld_koff);
  copy_tile(kbase, false, 1, k1, ld_koff);
  copy_tile(vbase, kVt, 0, v0, ld_voff);
  // the first MFMA phase of each group multiplies a zero P by buffer v2: it
  // must hold finite values
  for (int i = tid; i < G::kTileBytes / 16; i += 512) *(u32x4*)(v2 + 16 * i) = u32x4{};
  __builtin_amdgcn_s_waitcnt(kWaitVm0);
  __syncthreads();
  if (grp == 0)
    run(std::integral_constant<int, 0>{});
  else
    run(std::integral_constant<int, 1>{});
  __builtin_amdgcn_s_waitcnt(kWaitVm0);

  if (!wave_active) return;
  const float l_tot = pair_sum(st.l + lsum_row());
  if (tr.unit >= 0) {
    float* wo = a.ws + (int64_t)tr.unit * BM * D;
    float2* wml = (float2*)(a.ws + (int64_t)a.slots * BM * D) + (int64_t)tr.unit * BM;
    if (my_row < tr.q1) {
      const int r = my_row - tr.q0;
#pragma unroll
      for (int db = 0; db < G::NDB; ++db)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int d = db * 32 + 8 * i + 4 * g;
          *(f32x4*)(wo + (int64_t)r * D + d) =
              f32x4{st.o[db][4 * i], st.o[db][4 * i + 1], st.o[db][4 * i + 2], st.o[db][4 * i + 3]};
        }
      if (g == 0) wml[r] = make_float2(st.m_c, l_tot);
    }
    return;
  }
  const float inv = l_tot > 0.f ? 1.0f / l_tot : 0.f;
  if (my_row < tr.q1) {
    __bf16* op = (__bf16*)a.out + (int64_t)my_row * row_stride + (int64_t)h * D;
#pragma unroll
    for (int db = 0; db < G::NDB; ++db)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int d = db * 32 + 8 * i + 4 * g;
        typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
        bf16x4 w;
#pragma unroll
        for (int e = 0; e < 4; ++e) w[e] = (__bf16)(st.o[db][4 * i + e] * inv);
        *(bf16x4*)(op + d) = w;
      }
    if (a.lse != nullptr && g == 0)
      a.lse[(int64_t)my_row * H + h] = l_tot > 0.f ? (st.m_c + log2f(l_tot)) * kLn2 : -INFINITY;
  }
}

// ---------------------------------------------------------------- fp32 kernel

template <int D>
struct F32Geo {
  static constexpr int kThreads = 256;
  static constexpr int BM = 128;
  static constexpr int BN = 4096 / D;                   // keys per tile
  static constexpr int kRow = (D + 4) * 4;              // bytes per K / V row in LDS
  static constexpr int kKBytes = BN * kRow;
  static constexpr int kBufBytes = 2 * kKBytes;
  static constexpr int kLdsBytes = 2 * kBufBytes;
  static constexpr int DCH = D / 4;                     // 16-byte chunks per row
  static constexpr int kPasses = BN * DCH / kThreads;
  static constexpr int NKB = BN / 32;
  static constexpr int NDB = D / 32;
  static constexpr int NQ = D / 2;                      // Q features per lane
  static_assert(BN * DCH % kThreads == 0, "whole copy passes");
};

template <int D, bool kBlockLocal>
__global__ void __launch_bounds__(256, 2) attn_f32_kernel(AttnArgs a) {
  using G = F32Geo<D>;
  __shared__ __attribute__((aligned(16))) char smem[G::kLdsBytes];

  const TileRange tr = tile_range<G::BM, G::BN, kBlockLocal>(a);
  if (!tr.valid) return;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int ql = lane & 31;
  const int g = lane >> 5;
  const int H = a.H;
  const int h = tr.h;
  const int64_t row_stride = (int64_t)H * D;

  const float* __restrict__ qg = (const float*)a.q;
  const float* __restrict__ kg = (const float*)a.k;
  const float* __restrict__ vg = (const float*)a.v;

  const int my_row = tr.q0 + wave * 32 + ql;
  const bool row_ok = my_row < tr.q1;
  const bool wave_active = tr.q0 + wave * 32 < tr.q1;
  int lo = tr.k_lo, hi = tr.k_hi;
  if (kBlockLocal) {
    const int i = min(tr.seq_q0 + wave * 32 + ql, a.n - 1);
    window_of(a, i, lo, hi);
  }

  // Lane-half g holds features [g*D/2, (g+1)*D/2) of its query row: the
  // MFMA k-index (0 or 1) of step s is feature g*D/2 + s.
  float qf[G::NQ];
  {
    const float* qp = qg + (int64_t)my_row * row_stride + (int64_t)h * D + g * G::NQ;
#pragma unroll
    for (int s4 = 0; s4 < G::NQ / 4; ++s4) {
      const f32x4 x = row_ok ? *(const f32x4*)(qp + 4 * s4) : f32x4{};
#pragma unroll
      for (int e = 0; e < 4; ++e) qf[4 * s4 + e] = x[e];
    }
  }

  RowState<G::NKB, G::NDB> st;
  st.init();
  const int nkeys = tr.k_hi - tr.k_lo;
  const int ntiles = (nkeys + G::BN - 1) / G::BN;

  f32x4 kr[G::kPasses];
  f32x4 vr[G::kPasses];

  auto gload = [&](int tile) {
    const int key0 = tr.k_lo + tile * G::BN;
    const int valid = min(G::BN, tr.k_hi - key0);
    const int64_t base = (int64_t)(tr.kv_base + key0) * row_stride + (int64_t)h * D;
#pragma unroll
    for (int p = 0; p < G::kPasses; ++p) {
      const int idx = p * G::kThreads + tid;
      const int row = min(idx / G::DCH, valid - 1);   // see the bf16 kernel
      const int ch = idx % G::DCH;
      const int64_t off = base + (int64_t)row * row_stride + ch * 4;
      kr[p] = *(const f32x4*)(kg + off);
      vr[p] = *(const f32x4*)(vg + off);
    }
  };

  auto lstore = [&](int buf) {
    char* kl = smem + buf * G::kBufBytes;
    char* vl = kl + G::kKBytes;
#pragma unroll
    for (int p = 0; p < G::kPasses; ++p) {
      const int idx = p * G::kThreads + tid;
      const int row = idx / G::DCH;
      const int ch = idx % G::DCH;
      *(f32x4*)(kl + row * G::kRow + ch * 16) = kr[p];
      *(f32x4*)(vl + row * G::kRow + ch * 16) = vr[p];
    }
  };

  auto compute = [&](int buf, int tile, bool masked) {
    const char* kl = smem + buf * G::kBufBytes;
    const char* vl = kl + G::kKBytes;
    f32x16 s[G::NKB];
#pragma unroll
    for (int kb = 0; kb < G::NKB; ++kb) {
      s[kb] = f32x16{};
      const char* krow = kl + (kb * 32 + ql) * G::kRow + g * G::NQ * 4;
#pragma unroll
      for (int s4 = 0; s4 < G::NQ / 4; ++s4) {
        const f32x4 ka = *(const f32x4*)(krow + 16 * s4);
#pragma unroll
        for (int e = 0; e < 4; ++e)
          s[kb] = __builtin_amdgcn_mfma_f32_32x32x2f32(ka[e], qf[4 * s4 + e], s[kb], 0, 0, 0);
      }
    }
    if (masked) mask_scores<G::NKB>(s, tr.k_lo + tile * G::BN, g, lo, hi);
    st.softmax_tile(s, a.c);
    // O^T += V^T P^T: step j of sub-block kb contracts the key score_key(kb, j, g)
    // of each lane half, exactly the key whose probability sits in s[kb][j].
#pragma unroll
    for (int kb = 0; kb < G::NKB; ++kb)
#pragma unroll
      for (int j = 0; j < 16; ++j) {
        const float* vrow = (const float*)(vl + score_key(kb, j, g) * G::kRow);
#pragma unroll
        for (int db = 0; db < G::NDB; ++db)
          st.o[db] = __builtin_amdgcn_mfma_f32_32x32x2f32(vrow[db * 32 + ql], s[kb][j], st.o[db], 0, 0, 0);
      }
  };

  if (ntiles > 0) {
    gload(0);
    lstore(0);
  }
  __syncthreads();
  const bool ragged = (nkeys % G::BN) != 0;
  for (int it = 0; it < ntiles; ++it) {
    const bool more = it + 1 < ntiles;
    if (more) gload(it + 1);
    if (wave_active) compute(it & 1, it, kBlockLocal || (ragged && !more));
    if (more) lstore((it + 1) & 1);
    __syncthreads();
  }

  if (!wave_active) return;
  const float l_tot = pair_sum(st.l);
  if (row_ok) {
    float* op = (float*)a.out + (int64_t)my_row * row_stride + (int64_t)h * D;
#pragma unroll
    for (int db = 0; db < G::NDB; ++db)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int d = db * 32 + 8 * i + 4 * g;
        f32x4 w;
#pragma unroll
        for (int e = 0; e < 4; ++e) w[e] = l_tot > 0.f ? st.o[db][4 * i + e] / l_tot : 0.f;
        *(f32x4*)(op + d) = w;
      }
    if (a.lse != nullptr && g == 0)
      a.lse[(int64_t)my_row * H + h] = l_tot > 0.f ? (st.m_c + log2f(l_tot)) * kLn2 : -INFINITY;
  }
}

// ---------------------------------------------------------------- block-local, block-aligned (D = 64)

// Every query of block b sees the same keys, so for blocks of <= 32 frames one
// wave takes one query block of one (batch, head) and exactly its window, in
// chunks of 32 keys: no LDS sharing, no barriers, no masking beyond the
// window's ragged end.  Addressing: the wave's unit decides a uniform base
// pointer per tensor (its batch row and head, its first query / window key),
// lanes add 32-bit row offsets (24-bit multiplies), and buffer descriptors
// spanning only the valid rows make reads past the block or the window
// return zeros (those scores are masked, those query rows never stored).
struct BlockUnit {
  int b, h, r0, nq, k_lo, k_hi;
};

// Grid (ceil(nb / kBlockWaves), H, B): wave w of work-group x takes query
// block kBlockWaves * x + w (neighbouring blocks, which share keys, in
// neighbouring waves) of head y and batch row z.  Two-wave work-groups: the
// vocoder shape's 1,344 waves then reach the 256 CUs as 672 small groups
// rather than 336 of four, which spreads them evenly (-7 to -10 % at the
// vocoder shape, -1 to -3 % at the production shape, against four waves;
// one wave per group measured about the same as two, eight slower).
constexpr int kBlockWaves = 2;
__device__ __forceinline__ BlockUnit block_unit(const AttnArgs& a, int qb, int nb) {
  BlockUnit u;
  u.h = blockIdx.y;
  u.b = blockIdx.z;
  u.r0 = qb * a.block;
  u.nq = min(a.block, a.n - u.r0);
  u.k_lo = max(0, qb - a.look_back) * a.block;
  u.k_hi = min((qb + min(a.look_ahead, nb - 1 - qb)) * a.block + a.block, a.n);
  return u;
}

// Buffer resource over `rows` rows of `rs` bytes (the last one `row_bytes`
// long) from `base`; reads past them return zeros.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t rows_rsrc(const void* base, int rows, int rs, int row_bytes) {
  return __builtin_amdgcn_make_buffer_rsrc((void*)base, 0, rows > 0 ? (rows - 1) * rs + row_bytes : 0, kBufferFlags);
}

// fp32 (the Token2Wav DiT's precision):
//   S^T = K Q^T with v_mfma_f32_32x32x2_f32: lane (ql, g) holds the 16-byte
//   chunks 2i + g (features 8i + 4g .. +3, i = 0..7) of query row ql (B
//   operand) and of key row ql of the chunk (A operand), so the two halves of
//   a load read the same 128-byte lines; step 4i + e contracts feature
//   8i + 4g + e of both halves.  Two accumulators (even and odd steps) halve
//   the dependent chain.  The result gives lane (ql, g) the scores of query
//   ql for keys score_key(0, j, g).
//   O^T += V^T P^T: step j contracts key score_key(0, j, g) of each half, whose
//   probability is the lane's own score register j.  The chunk's V rows are
//   copied straight to LDS (256-byte rows; rows 4..7 of each group of 8 have
//   their two 128-byte halves swapped, so the two lane halves of a read --
//   rows 4 apart -- hit different banks) and each operand is one 4-byte read.
// One LDS buffer per wave (8 KB): the next chunk's V copy starts after this
// chunk's PV reads, and three waves fit on each SIMD (162 VGPRs);
// double-buffering V (two waves per SIMD) was
// slower at every window.
template <int D>
__global__ void __launch_bounds__(64 * kBlockWaves, 3) block_local_f32_kernel(AttnArgs a) {
  static_assert(D == 64, "two lane halves of 32 features");
  constexpr int NQ = D / 2;
  constexpr int NDB = D / 32;
  constexpr int VCH = 32 * D * 4;  // bytes of one chunk of V in LDS
  __shared__ __attribute__((aligned(16))) char vlds[kBlockWaves][VCH];
  const int lane = threadIdx.x & 63;
  const int ql = lane & 31;
  const int g = lane >> 5;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int nb = (a.n + a.block - 1) / a.block;
  const int qb = blockIdx.x * kBlockWaves + wave;
  if (qb >= nb) return;
  const BlockUnit u = block_unit(a, qb, nb);
  const int rs = a.H * D * 4;  // bytes between consecutive frames
  const int64_t hoff = (int64_t)u.b * a.n * a.H * D + (int64_t)u.h * D;
  const float* qb_ = (const float*)a.q + hoff + (int64_t)u.r0 * a.H * D;
  const float* kb_ = (const float*)a.k + hoff + (int64_t)u.k_lo * a.H * D;
  const float* vb_ = (const float*)a.v + hoff + (int64_t)u.k_lo * a.H * D;
  const int nkeys = u.k_hi - u.k_lo;
  const __amdgpu_buffer_rsrc_t rq = rows_rsrc(qb_, u.nq, rs, D * 4);
  const __amdgpu_buffer_rsrc_t rk = rows_rsrc(kb_, nkeys, rs, D * 4);

  // lane (ql, g): row ql, 16-byte chunks 2i + g
  const uint32_t lrow = (uint32_t)__umul24(ql, rs) + 16 * g;
  float qf[NQ];
#pragma unroll
  for (int i = 0; i < NQ / 4; ++i) {
    const f32x4 x = __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(rq, lrow + 32 * i, 0, 0));
#pragma unroll
    for (int e = 0; e < 4; ++e) qf[4 * i + e] = x[e];
  }
  // V copy: lane l of load i fills LDS row 4i + l/16, physical chunk l%16,
  // from logical chunk (l%16) ^ 8(i&1)
  auto copy_v = [&](int c, char* dst) {
    const char* src = (const char*)vb_ + (int64_t)c * 32 * rs;
    const int rows = min(32, nkeys - c * 32);
#pragma unroll
    for (int i = 0; i < VCH / 1024; ++i) {
      const int row = 4 * i + lane / 16;
      const uint32_t voff = (uint32_t)__umul24(row, rs) + (((lane & 15) ^ (8 * (i & 1))) * 16);
      lds_dma_one(src, (rows - 1) * rs + D * 4, dst + i * 1024, voff);
    }
  };
  auto load_k = [&](int c, float (&kf)[NQ]) {
#pragma unroll
    for (int i = 0; i < NQ / 4; ++i) {
      const f32x4 x = __builtin_bit_cast(
          f32x4, __builtin_amdgcn_raw_buffer_load_b128(rk, lrow + (uint32_t)(c * 32) * rs + 32 * i, 0, 0));
#pragma unroll
      for (int e = 0; e < 4; ++e) kf[4 * i + e] = x[e];
    }
  };
  // PV operand reads: key score_key(0, j, g), feature db*32 + ql, at
  // row*256 + (db ^ g)*128 + 4 ql
  const int vrd0 = 4 * g * 256 + g * 128 + 4 * ql;
  const int vrd1 = 4 * g * 256 + (1 - g) * 128 + 4 * ql;

  RowState<1, NDB> st;
  st.init();
  const int nch = (nkeys + 31) / 32;
  float kf[NQ];
  load_k(0, kf);
  char* const vbuf = vlds[wave];
  copy_v(0, vbuf);
  for (int c = 0; c < nch; ++c) {
    f32x16 s0 = f32x16{}, s1 = f32x16{};
#pragma unroll
    for (int st4 = 0; st4 < NQ; st4 += 2) {
      s0 = __builtin_amdgcn_mfma_f32_32x32x2f32(kf[st4], qf[st4], s0, 0, 0, 0);
      s1 = __builtin_amdgcn_mfma_f32_32x32x2f32(kf[st4 + 1], qf[st4 + 1], s1, 0, 0, 0);
    }
    f32x16 s[1] = {s0 + s1};
    const int key0 = u.k_lo + c * 32;
    // the next chunk's K rows stream in while this one computes
    if (c + 1 < nch) load_k(c + 1, kf);
    if (key0 + 32 > u.k_hi) mask_scores<1>(s, key0, g, u.k_lo, u.k_hi);
    st.softmax_tile(s, a.c);
    // this chunk's V copy has landed
    __builtin_amdgcn_s_waitcnt(kWaitVm0);
    // step j contracts keys 8(j/4) + j%4 (lane half 0) and 4 more (half 1):
    // steps whose lower key is past the chunk's last key multiply P = 0
    const int kv = min(32, u.k_hi - key0);
#pragma unroll
    for (int j = 0; j < 16; ++j) {
      if (8 * (j >> 2) + (j & 3) >= kv) continue;
      const int rowoff = (8 * (j >> 2) + (j & 3)) * 256;
      const float v0 = *(const float*)(vbuf + rowoff + vrd0);
      const float v1 = *(const float*)(vbuf + rowoff + vrd1);
      st.o[0] = __builtin_amdgcn_mfma_f32_32x32x2f32(v0, s[0][j], st.o[0], 0, 0, 0);
      st.o[1] = __builtin_amdgcn_mfma_f32_32x32x2f32(v1, s[0][j], st.o[1], 0, 0, 0);
    }
    if (c + 1 < nch) copy_v(c + 1, vbuf);
  }

  const float l_tot = pair_sum(st.l);
  if (ql < u.nq) {
    const float inv = l_tot > 0.f ? 1.0f / l_tot : 0.f;
    float* op = (float*)a.out + hoff + (int64_t)(u.r0 + ql) * a.H * D;
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int d = db * 32 + 8 * i + 4 * g;
        f32x4 w;
#pragma unroll
        for (int e = 0; e < 4; ++e) w[e] = st.o[db][4 * i + e] * inv;
        *(f32x4*)(op + d) = w;
      }
    if (a.lse != nullptr && g == 0)
      a.lse[((int64_t)u.b * a.n + u.r0 + ql) * a.H + u.h] =
          l_tot > 0.f ? (st.m_c + log2f(l_tot)) * kLn2 : -INFINITY;
  }
}

// bf16, same scheme:
//   S^T = K Q^T (v_mfma_f32_32x32x16_bf16, 4 steps over D): lane (ql, g)
//   holds features 16 ds + 8g .. +7 of query row ql (B) and of key row ql of
//   the chunk (A), one 16-byte load each.
//   O^T += V^T P^T (2 key steps x 2 feature blocks): P^T(kc) is the lane's
//   score registers 8kc .. 8kc+7 rounded to bf16, i.e. keys
//   16kc + 4g + (i & 3) + 8(i >> 2), i = 0..7; the chunk's V rows are copied
//   straight to LDS (128-byte rows, 16-byte chunks XOR-swizzled by row) and
//   the V^T operands read back with two transposing reads each
//   (ds_read_b64_tr_b16), which deliver exactly those keys of one feature.
// NBUF = 2 for windows of two or three chunks (a ring of two buffers: the
// next chunk's V streams into the other one while this one computes; a
// buffer is refilled only after the PV reads of the chunk it held have
// returned), 1 for single-chunk windows.
template <int D, int NBUF>
__global__ void __launch_bounds__(64 * kBlockWaves, 3) block_local_bf16_kernel(AttnArgs a) {
  static_assert(D == 64, "four 16-feature MFMA steps");
  constexpr int NDS = D / 16;
  constexpr int NDB = D / 32;
  constexpr int ROW = D * 2;
  constexpr int CPR = D / 8;
  constexpr int VCH = 32 * ROW;
  __shared__ __attribute__((aligned(16))) char vlds[kBlockWaves][NBUF][VCH];
  const int lane = threadIdx.x & 63;
  const int ql = lane & 31;
  const int g = lane >> 5;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int nb = (a.n + a.block - 1) / a.block;
  const int qb = blockIdx.x * kBlockWaves + wave;
  if (qb >= nb) return;
  const BlockUnit u = block_unit(a, qb, nb);
  const int rs = a.H * D * 2;
  const int64_t hoff = (int64_t)u.b * a.n * a.H * D + (int64_t)u.h * D;
  const __bf16* qb_ = (const __bf16*)a.q + hoff + (int64_t)u.r0 * a.H * D;
  const __bf16* kb_ = (const __bf16*)a.k + hoff + (int64_t)u.k_lo * a.H * D;
  const __bf16* vb_ = (const __bf16*)a.v + hoff + (int64_t)u.k_lo * a.H * D;
  const int nkeys = u.k_hi - u.k_lo;
  const __amdgpu_buffer_rsrc_t rq = rows_rsrc(qb_, u.nq, rs, ROW);
  const __amdgpu_buffer_rsrc_t rk = rows_rsrc(kb_, nkeys, rs, ROW);

  const uint32_t lrow = (uint32_t)__umul24(ql, rs) + 16 * g;
  bf16x8 qf[NDS];
#pragma unroll
  for (int ds = 0; ds < NDS; ++ds)
    qf[ds] = __builtin_bit_cast(bf16x8, __builtin_amdgcn_raw_buffer_load_b128(rq, lrow + 32 * ds, 0, 0));
  // V copy: lane l of load i fills LDS row 8i + l/8, physical chunk l%8, from
  // logical chunk (l%8) ^ v_swz(row)
  auto copy_v = [&](int c, char* dst) {
    const char* src = (const char*)vb_ + (int64_t)c * 32 * rs;
    const int rows = min(32, nkeys - c * 32);
#pragma unroll
    for (int i = 0; i < VCH / 1024; ++i) {
      const int row = 8 * i + lane / CPR;
      const uint32_t voff = (uint32_t)__umul24(row, rs) + (((lane % CPR) ^ v_swz<CPR>(row)) * 16);
      lds_dma_one(src, (rows - 1) * rs + ROW, dst + i * 1024, voff);
    }
  };
  auto load_k = [&](int c, bf16x8 (&kf)[NDS]) {
#pragma unroll
    for (int ds = 0; ds < NDS; ++ds)
      kf[ds] = __builtin_bit_cast(
          bf16x8, __builtin_amdgcn_raw_buffer_load_b128(rk, lrow + (uint32_t)(c * 32) * rs + 32 * ds, 0, 0));
  };
  // transposing-read offsets: in 16-lane group G' (lane half g = G'/2,
  // feature half G' % 2) input lane i points at row 4g + i/4 (and + 8) of a
  // 16-key step, features db*32 + 16*(G' % 2) + 4*(i % 4) .. +3
  const int vgrp = lane >> 4;
  const int gi = lane & 15;
  const int v_row = 4 * (vgrp >> 1) + (gi >> 2);
  int v_rd[NDB];
#pragma unroll
  for (int db = 0; db < NDB; ++db) {
    const int byte_in_row = db * 64 + 32 * (vgrp & 1) + 8 * (gi & 3);
    v_rd[db] = v_row * ROW + (((byte_in_row >> 4) ^ v_swz<CPR>(v_row)) * 16) + (byte_in_row & 15);
  }

  RowState<1, NDB> st;
  st.init();
  const int nch = (nkeys + 31) / 32;
  bf16x8 kf[NDS];
  load_k(0, kf);
  copy_v(0, vlds[wave][0]);
  for (int c = 0; c < nch; ++c) {
    char* vbuf = vlds[wave][NBUF > 1 ? (c & 1) : 0];
    f32x16 s[1] = {f32x16{}};
#pragma unroll
    for (int ds = 0; ds < NDS; ++ds) s[0] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf[ds], qf[ds], s[0], 0, 0, 0);
    const int key0 = u.k_lo + c * 32;
    if (c + 1 < nch) {
      load_k(c + 1, kf);
      if (NBUF > 1) copy_v(c + 1, vlds[wave][(c + 1) & 1]);
    }
    if (key0 + 32 > u.k_hi) mask_scores<1>(s, key0, g, u.k_lo, u.k_hi);
    st.softmax_tile(s, a.c);
    bf16x8 pf[2];
#pragma unroll
    for (int kc = 0; kc < 2; ++kc)
#pragma unroll
      for (int e = 0; e < 8; ++e) pf[kc][e] = (__bf16)s[0][8 * kc + e];
    if (NBUF > 1 && c + 1 < nch)
      __builtin_amdgcn_s_waitcnt(wait_vm(NDS + VCH / 1024));  // only the next chunk's loads outstanding
    else
      __builtin_amdgcn_s_waitcnt(kWaitVm0);
#pragma unroll
    for (int kc = 0; kc < 2; ++kc)
#pragma unroll
      for (int db = 0; db < NDB; ++db) {
        const char* p = vbuf + kc * 16 * ROW + v_rd[db];
        const i16x4 lo4 = lds_read_tr(p);
        const i16x4 hi4 = lds_read_tr(p + 8 * ROW);
        const bf16x8 vt = __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo4, hi4, 0, 1, 2, 3, 4, 5, 6, 7));
        st.o[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vt, pf[kc], st.o[db], 0, 0, 0);
      }
    if (NBUF == 1 && c + 1 < nch) copy_v(c + 1, vbuf);
  }

  const float l_tot = pair_sum(st.l);
  if (ql < u.nq) {
    const float inv = l_tot > 0.f ? 1.0f / l_tot : 0.f;
    __bf16* op = (__bf16*)a.out + hoff + (int64_t)(u.r0 + ql) * a.H * D;
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int d = db * 32 + 8 * i + 4 * g;
        typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
        bf16x4 w;
#pragma unroll
        for (int e = 0; e < 4; ++e) w[e] = (__bf16)(st.o[db][4 * i + e] * inv);
        *(bf16x4*)(op + d) = w;
      }
    if (a.lse != nullptr && g == 0)
      a.lse[((int64_t)u.b * a.n + u.r0 + ql) * a.H + u.h] =
          l_tot > 0.f ? (st.m_c + log2f(l_tot)) * kLn2 : -INFINITY;
  }
}

// ---------------------------------------------------------------- V^T staging

// One 64-key tile of one head of V -> V^T: the V rows (bf16) of request r's
// keys key0 .. key0+63 become D rows of 64 columns at
// vt_col_base(kv_cu[r], r) + key0, each 16-key group stored in the P k-slot
// order (vt_pos_of_key), keys past the request zero.  Block b covers column
// tile b mod (vt_ld / 64) of head b / (vt_ld / 64); tiles in the gaps between
// requests are never read and are skipped.  Through LDS so that both the V
// reads (16 lanes per 256-byte row) and the V^T writes (8 lanes per 128-byte
// row) are whole-line accesses.  The rows come from `src`: src.prepare(r) is
// called by every thread once the tile's request r is known (it may use
// __syncthreads), then src.row(f, h) gives head h of flat key row f of the
// request, or nullptr for a row that reads as zero.
template <int D, typename Src>
__device__ __forceinline__ void vt_tile(const int32_t* __restrict__ kv_cu, int R, int H, __bf16* vt, int64_t vt_ld,
                                        Src& src) {
  constexpr int LD = D + 2;  // bf16 per LDS row: an odd dword count, so column reads spread over banks
  constexpr int CPR = D / 8;
  __shared__ uint32_t sm[kVtTile * LD / 2];
  const int ntc = (int)(vt_ld / kVtTile);
  const int h = blockIdx.x / ntc;
  const int64_t col0 = (int64_t)(blockIdx.x % ntc) * kVtTile;
  // request of the tile: the last r whose first column is <= col0
  int lo = 0, hi = R - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (vt_col_base(kv_cu[mid], mid) <= col0)
      lo = mid;
    else
      hi = mid - 1;
  }
  const int kv0 = kv_cu[lo];
  const int len = kv_cu[lo + 1] - kv0;
  const int64_t key0 = col0 - vt_col_base(kv0, lo);
  if (key0 < 0 || key0 >= len) return;
  src.prepare(lo);
  const int valid = min(kVtTile, len - (int)key0);
  const int t = threadIdx.x;
#pragma unroll
  for (int i = t; i < kVtTile * CPR; i += 256) {
    const int k = i / CPR, ch = i % CPR;
    uint4 x = make_uint4(0u, 0u, 0u, 0u);
    if (k < valid) {
      const __bf16* row = src.row(kv0 + (int)key0 + k, h);
      if (row != nullptr) x = *(const uint4*)(row + ch * 8);
    }
    uint32_t* d = sm + (k * LD + ch * 8) / 2;
    d[0] = x.x;
    d[1] = x.y;
    d[2] = x.z;
    d[3] = x.w;
  }
  __syncthreads();
  const uint16_t* sh = (const uint16_t*)sm;
#pragma unroll
  for (int i = t; i < D * 8; i += 256) {
    const int d = i / 8, cc = i % 8;  // feature row, 16-byte chunk (stored positions 8cc .. 8cc+7)
    uint32_t w[4];
#pragma unroll
    for (int j = 0; j < 8; j += 2) {
      // stored position p holds key 4 (p / 8) + (p mod 4) + 8 ((p / 4) mod 2) of its group of 16
      const int p0 = (8 * cc + j) & 15, p1 = (8 * cc + j + 1) & 15;
      const int base = 16 * (cc >> 1);
      const int k0 = base + 4 * (p0 >> 3) + (p0 & 3) + 8 * ((p0 >> 2) & 1);
      const int k1 = base + 4 * (p1 >> 3) + (p1 & 3) + 8 * ((p1 >> 2) & 1);
      w[j / 2] = (uint32_t)sh[k0 * LD + d] | ((uint32_t)sh[k1 * LD + d] << 16);
    }
    *(uint4*)(vt + ((int64_t)h * D + d) * vt_ld + col0 + cc * 8) = make_uint4(w[0], w[1], w[2], w[3]);
  }
}

// V rows of the packed [T, H, D] tensor.
template <int D>
struct FlatVRows {
  const __bf16* v;
  int H;
  __device__ void prepare(int) {}
  __device__ const __bf16* row(int f, int h) const { return v + ((int64_t)f * H + h) * D; }
};

template <int D>
__global__ void __launch_bounds__(256) vt_transpose_kernel(AttnArgs a) {
  // the attention kernel that follows starts its chiplet queues from zero
  if (a.dyn != nullptr && blockIdx.x == 0 && threadIdx.x < kXcds) a.dyn[threadIdx.x] = 0;
  FlatVRows<D> src{(const __bf16*)a.v, a.H};
  vt_tile<D>(a.kv_cu, a.R, a.H, (__bf16*)a.vt, a.vt_ld, src);
}

// V packed straight from padded per-request buffers into V^T (the pack and
// the staging in one pass).  Piece p of request r is the rows
// [0, cu[r+1] - cu[r]) of src + r * max_len rows, which are flat key rows
// off[r] (cu[r] when off is null) onward of the request's packed numbering.
constexpr int kMaxVtPieces = 8;
struct VtPiece {
  const void* src;
  const int32_t* cu;
  const int32_t* off;
  int64_t max_len;
};
struct PackVtArgs {
  VtPiece piece[kMaxVtPieces];
  int count;
  const int32_t* kv_cu;
  int R;
  int H;
  void* vt;
  int64_t vt_ld;
};

// Rows of the pieces: prepare(r) puts each piece's first flat row and length
// for request r in LDS; a key row no piece covers reads as zero.
template <int D>
struct PieceVRows {
  const PackVtArgs* p;
  int r;
  int* s_off;
  int* s_len;
  __device__ void prepare(int req) {
    r = req;
    const int t = threadIdx.x;
    if (t < p->count) {
      const VtPiece& pc = p->piece[t];
      s_off[t] = pc.off != nullptr ? pc.off[req] : pc.cu[req];
      s_len[t] = pc.cu[req + 1] - pc.cu[req];
    }
    __syncthreads();
  }
  __device__ const __bf16* row(int f, int h) const {
    for (int i = 0; i < p->count; ++i) {
      const int d = f - s_off[i];
      if (d >= 0 && d < s_len[i])
        return (const __bf16*)p->piece[i].src + (((int64_t)r * p->piece[i].max_len + d) * p->H + h) * D;
    }
    return nullptr;
  }
};

template <int D>
__global__ void __launch_bounds__(256) pack_vt_kernel(PackVtArgs a) {
  __shared__ int s_off[kMaxVtPieces], s_len[kMaxVtPieces];
  PieceVRows<D> src{&a, 0, s_off, s_len};
  vt_tile<D>(a.kv_cu, a.R, a.H, (__bf16*)a.vt, a.vt_ld, src);
}

// Zeroes the chiplet-queue counters before an attention launch that reads a
// V^T staged by an earlier call.
__global__ void __launch_bounds__(64) zero_counters_kernel(int* cnt) {
  if (threadIdx.x < kXcds) cnt[threadIdx.x] = 0;
}

// ---------------------------------------------------------------- split merge

// Merges the partial results of the split work items.  Tail tile t's key
// ranges ran as units t*parts .. t*parts + parts - 1; a block handles RPB rows
// of one tail tile, a thread one 4-float group of a row.  Per row, with
// exponent offsets m_p (log2 units) and row sums l_p of the parts:
// m = max m_p, w_p = 2^(m_p - m), out = sum_p w_p O_p / sum_p w_p l_p,
// lse = (m + log2 sum_p w_p l_p) ln 2 -- taken in one pass over the parts with
// a running maximum.  Empty parts carry m_p = -inf, l_p = 0 and are skipped.
template <int D, int BM>
__global__ void __launch_bounds__(256) split_merge_kernel(AttnArgs a) {
  constexpr int C4 = D / 4;         // 4-float groups per row
  constexpr int RPB = 256 / C4;     // rows per block
  constexpr int BPT = BM / RPB;     // blocks per tail tile
  const SplitPlan sp = split_plan(total_tiles(a.q_cu, a.R, a.H, BM), a.slots, a.max_kv);
  const int t = (int)blockIdx.x / BPT;
  if (sp.parts < 2 || t >= sp.tail) return;
  int req, head, qt;
  find_tile(a.q_cu, a.kv_cu, a.R, a.H, BM, sp.full + t, req, head, qt);
  if (req < 0) return;
  const int q0 = a.q_cu[req] + qt * BM;
  const int rows = min(a.q_cu[req + 1], q0 + BM) - q0;
  const int r = ((int)blockIdx.x % BPT) * RPB + (int)threadIdx.x / C4;
  const int c = (int)threadIdx.x % C4;
  if (r >= rows) return;
  const int64_t u0 = (int64_t)t * sp.parts;
  const float2* wml = (const float2*)(a.ws + (int64_t)a.slots * BM * D);
  float m = -INFINITY, l = 0.f;
  f32x4 acc = f32x4{};
  for (int p = 0; p < sp.parts; ++p) {
    const float2 ml = wml[(u0 + p) * BM + r];
    if (ml.x == -INFINITY) continue;
    if (ml.x > m) {
      const float sc = __builtin_amdgcn_exp2f(m - ml.x);  // 0 while m = -inf
      acc *= sc;
      l *= sc;
      m = ml.x;
    }
    const float w = __builtin_amdgcn_exp2f(ml.x - m);
    l = fmaf(w, ml.y, l);
    acc += w * *(const f32x4*)(a.ws + ((u0 + p) * BM + r) * D + 4 * c);
  }
  const float inv = l > 0.f ? 1.0f / l : 0.f;
  typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
  bf16x4 y;
#pragma unroll
  for (int e = 0; e < 4; ++e) y[e] = (__bf16)(acc[e] * inv);
  *(bf16x4*)((__bf16*)a.out + (int64_t)(q0 + r) * a.H * D + (int64_t)head * D + 4 * c) = y;
  if (c == 0 && a.lse != nullptr)
    a.lse[(int64_t)(q0 + r) * a.H + head] = l > 0.f ? (m + log2f(l)) * kLn2 : -INFINITY;
}

// ---------------------------------------------------------------- tile-map export

__global__ void __launch_bounds__(64) tile_map_kernel(const int32_t* q_cu, const int32_t* kv_cu, int R, int H,
                                                      int block_m, int chunk, int slots, int max_kv, int32_t* out) {
  const int logical = block_to_logical(blockIdx.x, chunk);
  const WorkItem w = work_item(q_cu, kv_cu, R, H, block_m, slots, max_kv, logical);
  if (threadIdx.x == 0) {
    const bool idle = w.req < 0;
    int32_t* o = out + 5 * (int64_t)blockIdx.x;
    o[0] = idle ? -1 : w.req;
    o[1] = idle ? -1 : w.head;
    o[2] = idle ? -1 : w.qt;
    o[3] = idle ? -1 : w.part;
    o[4] = idle ? -1 : w.parts;
  }
}

}  // namespace vl

// ============================================================================ host side

namespace {

constexpr int kChunk = 32;  // logical tiles kept together on one chiplet
// bf16 varlen: the ping-pong kernel, 8 waves, 256 query rows per work-group,
// 64-key tiles
constexpr int kBf16VarlenThreads = 512;
constexpr int kBf16VarlenBN = 64;
constexpr int kBf16VarlenBM = 256;
constexpr int kF32Waves = 4;
constexpr int kMaxDevices = 64;

inline bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

template <int D>
constexpr auto bf16_varlen_kernel() {
  return &vl::attn_bf16_pp_kernel<D, kBf16VarlenBN, true>;
}

// Work-groups of the bf16 varlen kernel resident at once on the current
// device (occupancy x compute units), 0 if it cannot be queried (no GPU).
// Read once per device and head size, then cached.
int bf16_varlen_slots(int D) {
  static std::mutex mu;
  static int cache[kMaxDevices][2];
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) {
    (void)hipGetLastError();
    return 0;
  }
  const int di = D == 128 ? 1 : 0;
  std::lock_guard<std::mutex> lock(mu);
  if (cache[dev][di] > 0) return cache[dev][di];
  int cus = 0, per_cu = 0;
  hipError_t e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
  if (e == hipSuccess)
    e = D == 128 ? hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, bf16_varlen_kernel<128>(), kBf16VarlenThreads, 0)
                 : hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, bf16_varlen_kernel<64>(), kBf16VarlenThreads, 0);
  if (e != hipSuccess || cus <= 0 || per_cu <= 0) {
    (void)hipGetLastError();
    return 0;
  }
  cache[dev][di] = cus * per_cu;
  return cache[dev][di];
}

// The varlen launch for a dtype: query rows per work-group, threads, grid,
// and the slot count of the key split (0 = none).
struct VarlenPlan {
  int block_m;
  int threads;
  int slots;
  bool queues;
  int64_t blocks;
};

// queues: the launch takes its items through the chiplet work queues (the
// workspace launch); it then gets an eighth more work-groups than the item
// bound, so that chiplets that run faster have work-groups left with which
// to take other chiplets' items.
inline VarlenPlan varlen_plan(bool f32, bool split, bool queues, int64_t num_reqs, int64_t max_q, int64_t max_kv,
                              int64_t H, int D) {
  VarlenPlan p;
  p.block_m = f32 ? 32 * kF32Waves : kBf16VarlenBM;
  p.threads = f32 ? 64 * kF32Waves : kBf16VarlenThreads;
  // a split needs at least two key ranges of kMinSplitKeys keys
  p.slots = (split && !f32 && max_kv / vl::kMinSplitKeys >= 2) ? bf16_varlen_slots(D) : 0;
  p.queues = queues && split && !f32;
  const int64_t upper = num_reqs * H * ((max_q + p.block_m - 1) / p.block_m) + p.slots;
  const int64_t spare = p.queues ? (upper + 7) / 8 : 0;
  p.blocks = (num_reqs == 0 || max_q == 0) ? 0
                                           : vl::grid_blocks(num_reqs, max_q, H, p.block_m, kChunk, p.slots + spare);
  return p;
}

// Workspace of the split launch: the partial results the key split may
// write (per slot, BM rows of D floats and BM (offset, sum) float pairs),
// rounded up to 256 bytes; then V^T ([H][D][vt_ld] bf16), rounded up to 256
// bytes; then 256 bytes holding the kXcds counters of the chiplet queues.
inline int64_t split_partial_bytes(int slots, int D) {
  return ((int64_t)slots * kBf16VarlenBM * ((int64_t)D * 4 + 8) + 255) / 256 * 256;
}
inline int64_t split_vt_bytes(int64_t kv_rows, int64_t num_reqs, int64_t H, int D) {
  return (H * D * vl::vt_row_len(kv_rows, num_reqs) * 2 + 255) / 256 * 256;
}
constexpr int64_t kQueueBytes = 256;
inline int64_t split_workspace_bytes(int slots, int64_t kv_rows, int64_t num_reqs, int64_t H, int D) {
  return split_partial_bytes(slots, D) + split_vt_bytes(kv_rows, num_reqs, H, D) + kQueueBytes;
}

// Where a V^T staged by pack_v_transposed starts in the workspace: after the
// partial results of every resident work-group, whatever max_kv is, so that
// the pack and the attention call that reads it agree without sharing max_kv.
inline int64_t staged_vt_offset(int D) { return split_partial_bytes(bf16_varlen_slots(D), D); }

int launch_status() {
  return hipGetLastError() == hipSuccess ? VL_OK : VL_ELAUNCH;
}

// Device scratch of the allocation-free varlen entry point: the partial
// results of the key split (split_partial_bytes(slots, D)).  Every GPU the
// library runs on holds one copy until the process ends; host code never
// passes the array's name to a kernel (on the host it is only a stand-in) but
// the device address looked up once per device by noalloc_scratch().
static __device__ __align__(256) char scratch[VL_NOALLOC_SCRATCH_BYTES];

// Address of this device's `scratch`, looked up with the device current on
// the first call on that device; nullptr if the lookup fails.
void* noalloc_scratch(int dev) {
  static std::mutex mu;
  static void* addr[kMaxDevices];
  std::lock_guard<std::mutex> lock(mu);
  if (addr[dev] == nullptr) {
    void* ptr = nullptr;
    if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || ptr == nullptr) {
      (void)hipGetLastError();
      return nullptr;
    }
    addr[dev] = ptr;
  }
  return addr[dev];
}

// split: the key split of the last round, with the workspace (V^T staged
// there, partials after it) or, when noalloc, with the partials in the
// device's `scratch` and V read row-major.
template <bool kF32>
int varlen_common(const void* q, const void* k, const void* v, const int32_t* q_cu,
                  const int32_t* kv_cu, int32_t max_q, int32_t max_kv, int32_t num_reqs,
                  int32_t H, int32_t D, float scale, void* out, float* lse, bool split, int64_t kv_rows,
                  void* workspace, int64_t workspace_bytes, hipStream_t stream, bool noalloc = false,
                  bool staged_vt = false) {
  if (num_reqs < 0 || max_q < 0 || max_kv < 0 || H < 1 || kv_rows < 0) return VL_EINVAL;
  if (D != 64 && D != 128) return VL_EUNSUPPORTED;
  if (num_reqs == 0 || max_q == 0) return VL_OK;
  if (!q || !k || (!v && !staged_vt) || !q_cu || !kv_cu || !out) return VL_EINVAL;
  if (!aligned16(q) || !aligned16(k) || (v && !aligned16(v)) || !aligned16(out)) return VL_EINVAL;
  // the online softmax tracks the maximum of the raw scores: that is the
  // maximum of scale * q.k only for scale > 0 (and a masked score, -inf,
  // times a zero scale would be NaN)
  if (!(scale > 0.f) || std::isinf(scale)) return VL_EINVAL;
  const VarlenPlan plan = varlen_plan(kF32, split, split && !noalloc, num_reqs, max_q, max_kv, H, D);
  const int64_t G = plan.blocks;
  if (G > INT32_MAX) return VL_EUNSUPPORTED;
  // the workspace launch stages V^T (or, staged_vt, reads the one
  // pack_v_transposed staged); its copies address a head's V^T with 32-bit offsets
  const bool use_vt = split && !noalloc;
  const bool stage_vt = use_vt && !staged_vt;
  const int64_t vt_ld = use_vt ? vl::vt_row_len(kv_rows, num_reqs) : 0;
  if (use_vt && ((int64_t)D * vt_ld * 2 > INT32_MAX || vt_ld / vl::kVtTile * H > INT32_MAX))
    return VL_EUNSUPPORTED;
  const int64_t vt_off = staged_vt ? staged_vt_offset(D) : split_partial_bytes(plan.slots, D);
  if (use_vt &&
      (!workspace || !aligned16(workspace) ||
       workspace_bytes < vt_off + split_vt_bytes(kv_rows, num_reqs, H, D) + kQueueBytes))
    return VL_EINVAL;
  if (noalloc) {
    // the partials must fit the static scratch; its address is this device's
    if (split_partial_bytes(plan.slots, D) > (int64_t)VL_NOALLOC_SCRATCH_BYTES) return VL_EUNSUPPORTED;
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) {
      (void)hipGetLastError();
      return VL_ELAUNCH;
    }
    workspace = plan.slots > 0 ? noalloc_scratch(dev) : nullptr;
    if (plan.slots > 0 && workspace == nullptr) return VL_ELAUNCH;
  }
  vl::AttnArgs a{};
  a.q = q;
  a.k = k;
  a.v = v;
  a.out = out;
  a.lse = lse;
  a.q_cu = q_cu;
  a.kv_cu = kv_cu;
  a.R = num_reqs;
  a.H = H;
  a.chunk = kChunk;
  a.c = scale * vl::kLog2e;
  a.slots = plan.slots;
  a.max_kv = max_kv;
  a.ws = (float*)workspace;
  if (use_vt) {
    a.vt = (char*)workspace + vt_off;
    a.vt_ld = vt_ld;
    if (plan.queues) a.dyn = (int*)((char*)workspace + vt_off + split_vt_bytes(kv_rows, num_reqs, H, D));
  }
  (void)hipGetLastError();
  if (kF32) {
    if (D == 128)
      hipLaunchKernelGGL((vl::attn_f32_kernel<128, false>), dim3((unsigned)G), dim3(plan.threads), 0, stream, a);
    else
      hipLaunchKernelGGL((vl::attn_f32_kernel<64, false>), dim3((unsigned)G), dim3(plan.threads), 0, stream, a);
    return launch_status();
  }
  if (use_vt) {
    const unsigned tb = (unsigned)(vt_ld / vl::kVtTile * H);
    if (stage_vt) {
      if (D == 128)
        hipLaunchKernelGGL((vl::vt_transpose_kernel<128>), dim3(tb), dim3(256), 0, stream, a);
      else
        hipLaunchKernelGGL((vl::vt_transpose_kernel<64>), dim3(tb), dim3(256), 0, stream, a);
    } else if (a.dyn != nullptr) {
      hipLaunchKernelGGL(vl::zero_counters_kernel, dim3(1), dim3(64), 0, stream, a.dyn);
    }
    if (D == 128)
      hipLaunchKernelGGL((vl::attn_bf16_pp_kernel<128, kBf16VarlenBN, true>), dim3((unsigned)G),
                         dim3(plan.threads), 0, stream, a);
    else
      hipLaunchKernelGGL((vl::attn_bf16_pp_kernel<64, kBf16VarlenBN, true>), dim3((unsigned)G),
                         dim3(plan.threads), 0, stream, a);
  } else if (D == 128) {
    hipLaunchKernelGGL((vl::attn_bf16_pp_kernel<128, kBf16VarlenBN, false>), dim3((unsigned)G), dim3(plan.threads),
                       0, stream, a);
  } else {
    hipLaunchKernelGGL((vl::attn_bf16_pp_kernel<64, kBf16VarlenBN, false>), dim3((unsigned)G), dim3(plan.threads),
                       0, stream, a);
  }
  if (plan.slots > 0) {
    // BM / (256 / (D/4)) blocks per possible tail tile (there are fewer than
    // slots of them); blocks past the tail return at once
    const unsigned mb = (unsigned)plan.slots * (unsigned)(kBf16VarlenBM * D / 4 / 256);
    if (D == 128)
      hipLaunchKernelGGL((vl::split_merge_kernel<128, kBf16VarlenBM>), dim3(mb), dim3(256), 0, stream, a);
    else
      hipLaunchKernelGGL((vl::split_merge_kernel<64, kBf16VarlenBM>), dim3(mb), dim3(256), 0, stream, a);
  }
  return launch_status();
}

template <bool kF32>
int block_local_common(const void* q, const void* k, const void* v, int32_t B, int32_t n, int32_t H,
                       int32_t D, int32_t block, int32_t look_back, int32_t look_ahead, float scale,
                       void* out, float* lse, hipStream_t stream) {
  if (B < 0 || n < 0 || H < 1 || block < 1 || look_back < 0 || look_ahead < 0) return VL_EINVAL;
  if (D != 64 && D != 128) return VL_EUNSUPPORTED;
  if (B == 0 || n == 0) return VL_OK;
  if (!q || !k || !v || !out) return VL_EINVAL;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(out)) return VL_EINVAL;
  // the online softmax tracks the maximum of the raw scores: that is the
  // maximum of scale * q.k only for scale > 0 (and a masked score, -inf,
  // times a zero scale would be NaN)
  if (!(scale > 0.f) || std::isinf(scale)) return VL_EINVAL;
  if ((int64_t)B * n > INT32_MAX) return VL_EUNSUPPORTED;
  const int nqt = (n + 127) / 128;
  const int64_t G = (int64_t)B * H * nqt;
  if (G > INT32_MAX) return VL_EUNSUPPORTED;
  vl::AttnArgs a{};
  a.q = q;
  a.k = k;
  a.v = v;
  a.out = out;
  a.lse = lse;
  a.H = H;
  a.c = scale * vl::kLog2e;
  a.B = B;
  a.n = n;
  a.block = block;
  // windows wider than the sequence are the whole sequence
  const int nblocks = (n + block - 1) / block;
  a.look_back = min(look_back, nblocks);
  a.look_ahead = min(look_ahead, nblocks);
  a.nqt = nqt;
  (void)hipGetLastError();
  // one wave per query block of one (batch, head), its window in 32-key
  // chunks (D = 64, blocks of <= 32 frames); its 32-bit row offsets need the
  // sequence's rows within 2^31 bytes
  const int64_t window = (int64_t)(1 + a.look_back + a.look_ahead) * block;
  const bool aligned = D == 64 && block <= 32 && (int64_t)n * H * D * (kF32 ? 4 : 2) < INT32_MAX && H <= 65535 &&
                       B <= 65535;
  const bool one_chunk = window <= 32;
  const int64_t nblk = (n + block - 1) / block;
  const dim3 ag((unsigned)((nblk + vl::kBlockWaves - 1) / vl::kBlockWaves), (unsigned)H, (unsigned)B);
  if (kF32 && aligned) {
    hipLaunchKernelGGL((vl::block_local_f32_kernel<64>), ag, dim3(64 * vl::kBlockWaves), 0, stream, a);
  } else if (kF32) {
    if (D == 128)
      hipLaunchKernelGGL((vl::attn_f32_kernel<128, true>), dim3((unsigned)G), dim3(256), 0, stream, a);
    else
      hipLaunchKernelGGL((vl::attn_f32_kernel<64, true>), dim3((unsigned)G), dim3(256), 0, stream, a);
  } else if (aligned && window <= 96) {
    // Wider windows go to the tiled kernel, which shares the keys of 128
    // queries' windows through LDS, where each wave here re-reads its own
    // window: at 4-5 chunks the tiled kernel is faster at the production
    // shape (B = 2, n = 4000) though not yet at the vocoder's (B = 1,
    // n = 2003), and the 96-key limit is faster at both.
    if (one_chunk)
      hipLaunchKernelGGL((vl::block_local_bf16_kernel<64, 1>), ag, dim3(64 * vl::kBlockWaves), 0, stream, a);
    else
      hipLaunchKernelGGL((vl::block_local_bf16_kernel<64, 2>), ag, dim3(64 * vl::kBlockWaves), 0, stream, a);
  } else {
    if (D == 128)
      hipLaunchKernelGGL((vl::block_local_tiled_bf16_kernel<128>), dim3((unsigned)G), dim3(256), 0, stream, a);
    else
      hipLaunchKernelGGL((vl::block_local_tiled_bf16_kernel<64>), dim3((unsigned)G), dim3(256), 0, stream, a);
  }
  return launch_status();
}

}  // namespace

extern "C" {

int varlen_attn_fwd(const void* q, const void* k, const void* v, const int32_t* q_cu_seqlens,
                    const int32_t* kv_cu_seqlens, int32_t max_q, int32_t max_kv, int32_t num_reqs,
                    int32_t H, int32_t D, float scale, void* out, float* lse, vl_stream_t stream) {
  return varlen_common<false>(q, k, v, q_cu_seqlens, kv_cu_seqlens, max_q, max_kv, num_reqs, H, D,
                              scale, out, lse, false, 0, nullptr, 0, (hipStream_t)stream);
}

int varlen_attn_fwd_split(const void* q, const void* k, const void* v, const int32_t* q_cu_seqlens,
                          const int32_t* kv_cu_seqlens, int32_t max_q, int32_t max_kv, int32_t num_reqs,
                          int32_t H, int32_t D, float scale, void* out, float* lse, int64_t kv_rows,
                          void* workspace, int64_t workspace_bytes, vl_stream_t stream) {
  return varlen_common<false>(q, k, v, q_cu_seqlens, kv_cu_seqlens, max_q, max_kv, num_reqs, H, D,
                              scale, out, lse, true, kv_rows, workspace, workspace_bytes, (hipStream_t)stream);
}

int varlen_attn_fwd_noalloc(const void* q, const void* k, const void* v, const int32_t* q_cu_seqlens,
                            const int32_t* kv_cu_seqlens, int32_t max_q, int32_t max_kv, int32_t num_reqs,
                            int32_t H, int32_t D, float scale, void* out, float* lse, vl_stream_t stream) {
  return varlen_common<false>(q, k, v, q_cu_seqlens, kv_cu_seqlens, max_q, max_kv, num_reqs, H, D,
                              scale, out, lse, true, 0, nullptr, 0, (hipStream_t)stream, true);
}

int pack_v_transposed(const vl_copy_desc* descs, int32_t count, const int32_t* kv_cu_seqlens, int32_t num_reqs,
                      int32_t H, int32_t D, int64_t kv_rows, void* workspace, int64_t workspace_bytes,
                      vl_stream_t stream) {
  if (num_reqs < 0 || H < 1 || kv_rows < 0 || count < 1 || count > vl::kMaxVtPieces || !descs) return VL_EINVAL;
  if (D != 64 && D != 128) return VL_EUNSUPPORTED;
  vl::PackVtArgs a{};
  for (int i = 0; i < count; ++i) {
    const vl_copy_desc& d = descs[i];
    // a piece of no rows (max_len 0) may have a null source: it is never read
    if ((!d.src && d.max_len > 0) || !d.cu_seqlens || !aligned16(d.src) || d.max_len < 0 ||
        d.num_reqs != num_reqs || d.row_bytes != (int64_t)H * D * 2)
      return VL_EINVAL;
    a.piece[i] = vl::VtPiece{d.src, d.cu_seqlens, d.row_offsets, d.max_len};
  }
  if (num_reqs == 0) return VL_OK;
  const int64_t vt_ld = vl::vt_row_len(kv_rows, num_reqs);
  if ((int64_t)D * vt_ld * 2 > INT32_MAX || vt_ld / vl::kVtTile * H > INT32_MAX) return VL_EUNSUPPORTED;
  const int64_t vt_off = staged_vt_offset(D);
  if (!kv_cu_seqlens || !workspace || !aligned16(workspace) ||
      workspace_bytes < vt_off + split_vt_bytes(kv_rows, num_reqs, H, D) + kQueueBytes)
    return VL_EINVAL;
  a.count = count;
  a.kv_cu = kv_cu_seqlens;
  a.R = num_reqs;
  a.H = H;
  a.vt = (char*)workspace + vt_off;
  a.vt_ld = vt_ld;
  (void)hipGetLastError();
  const unsigned tb = (unsigned)(vt_ld / vl::kVtTile * H);
  if (D == 128)
    hipLaunchKernelGGL((vl::pack_vt_kernel<128>), dim3(tb), dim3(256), 0, (hipStream_t)stream, a);
  else
    hipLaunchKernelGGL((vl::pack_vt_kernel<64>), dim3(tb), dim3(256), 0, (hipStream_t)stream, a);
  return launch_status();
}

int varlen_attn_fwd_vt(const void* q, const void* k, const int32_t* q_cu_seqlens, const int32_t* kv_cu_seqlens,
                       int32_t max_q, int32_t max_kv, int32_t num_reqs, int32_t H, int32_t D, float scale, void* out,
                       float* lse, int64_t kv_rows, void* workspace, int64_t workspace_bytes, vl_stream_t stream) {
  return varlen_common<false>(q, k, nullptr, q_cu_seqlens, kv_cu_seqlens, max_q, max_kv, num_reqs, H, D, scale,
                              out, lse, true, kv_rows, workspace, workspace_bytes, (hipStream_t)stream, false, true);
}

int varlen_split_workspace_bytes(int64_t kv_rows, int32_t num_reqs, int32_t H, int32_t D, int64_t* bytes) {
  if (!bytes || kv_rows < 0 || num_reqs < 0 || H < 1) return VL_EINVAL;
  if (D != 64 && D != 128) return VL_EUNSUPPORTED;
  *bytes = split_workspace_bytes(bf16_varlen_slots(D), kv_rows, num_reqs, H, D);
  return VL_OK;
}

int varlen_attn_fwd_f32(const float* q, const float* k, const float* v,
                        const int32_t* q_cu_seqlens, const int32_t* kv_cu_seqlens, int32_t max_q,
                        int32_t max_kv, int32_t num_reqs, int32_t H, int32_t D, float scale,
                        float* out, float* lse, vl_stream_t stream) {
  return varlen_common<true>(q, k, v, q_cu_seqlens, kv_cu_seqlens, max_q, max_kv, num_reqs, H, D,
                             scale, out, lse, false, 0, nullptr, 0, (hipStream_t)stream);
}

int block_local_attn_fwd(const void* q, const void* k, const void* v, int32_t B, int32_t n,
                         int32_t H, int32_t D, int32_t block, int32_t look_back,
                         int32_t look_ahead, float scale, void* out, float* lse,
                         vl_stream_t stream) {
  return block_local_common<false>(q, k, v, B, n, H, D, block, look_back, look_ahead, scale, out,
                                   lse, (hipStream_t)stream);
}

int block_local_attn_fwd_f32(const float* q, const float* k, const float* v, int32_t B,
                             int32_t n, int32_t H, int32_t D, int32_t block, int32_t look_back,
                             int32_t look_ahead, float scale, float* out, float* lse,
                             vl_stream_t stream) {
  return block_local_common<true>(q, k, v, B, n, H, D, block, look_back, look_ahead, scale, out,
                                  lse, (hipStream_t)stream);
}

int varlen_launch_shape(int32_t max_q, int32_t max_kv, int32_t num_reqs, int32_t H, int32_t D, int dtype_f32,
                        int split, int32_t* block_m, int32_t* chunk, int64_t* blocks, int32_t* slots) {
  if (max_q < 0 || max_kv < 0 || num_reqs < 0 || H < 1) return VL_EINVAL;
  if (D != 64 && D != 128) return VL_EUNSUPPORTED;
  const VarlenPlan plan = varlen_plan(dtype_f32 != 0, split != 0, split != 0, num_reqs, max_q, max_kv, H, D);
  if (block_m) *block_m = plan.block_m;
  if (chunk) *chunk = kChunk;
  if (blocks) *blocks = plan.blocks;
  if (slots) *slots = plan.slots;
  return VL_OK;
}

int varlen_tile_map(const int32_t* q_cu_seqlens, const int32_t* kv_cu_seqlens, int32_t max_q, int32_t max_kv,
                    int32_t num_reqs, int32_t H, int32_t D, int dtype_f32, int split, int32_t* items_out,
                    int64_t max_blocks, vl_stream_t stream) {
  if (max_q < 0 || max_kv < 0 || num_reqs < 0 || H < 1) return VL_EINVAL;
  if (D != 64 && D != 128) return VL_EUNSUPPORTED;
  const VarlenPlan plan = varlen_plan(dtype_f32 != 0, split != 0, split != 0, num_reqs, max_q, max_kv, H, D);
  const int64_t G = plan.blocks;
  if (G == 0) return VL_OK;
  if (!q_cu_seqlens || !kv_cu_seqlens || !items_out || max_blocks < G) return VL_EINVAL;
  if (G > INT32_MAX) return VL_EUNSUPPORTED;
  (void)hipGetLastError();
  hipLaunchKernelGGL(vl::tile_map_kernel, dim3((unsigned)G), dim3(64), 0, (hipStream_t)stream, q_cu_seqlens,
                     kv_cu_seqlens, num_reqs, H, plan.block_m, kChunk, plan.slots, max_kv, items_out);
  return launch_status();
}

}  // extern "C"
