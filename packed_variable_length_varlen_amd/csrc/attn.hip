// Flat varlen and block-local attention forward for gfx950 (MI355X).
//
// What is computed (vLLM-Omni PR #6711 "Key changes" / "Reference /
// Acknowledgement", PR #4024 "Correctness model", PR #7975 review of the
// window code and its "Purpose" / "Change" sections): for every query row and
// head, softmax(scale * q K^T) V over the keys the row may see -- all keys of
// its own request (varlen), or the keys of its block window (block-local).
//
// Kernel design (ours; the pages only name library calls):
//  * one work-group = 4 waves = 128 query rows of one (sequence, head); each
//    wave owns 32 rows.  Q lives in registers for the whole key loop.
//  * keys stream through LDS in tiles of BN rows, double-buffered: the next
//    tile's global loads are in flight while the current one is consumed.
//  * S^T = K Q^T on MFMA (bf16: v_mfma_f32_32x32x16_bf16; fp32:
//    v_mfma_f32_32x32x2_f32), so each lane holds one query's scores for 16
//    keys and the row max / row sum need one in-lane pass plus one lane-half
//    swap (v_permlane32_swap).
//  * O^T += V^T P^T on MFMA with P taken straight from the score registers:
//    the MFMA k-index -> key permutation of the score layout is absorbed by
//    the order V^T is written to LDS (bf16) or read from LDS (fp32).
//  * exp2-domain online softmax with a lazy rescale: the running max used as
//    the exponent offset only moves when a new score exceeds it by more than
//    2^8, so most tiles skip the O rescale.  O and l always carry the same
//    factor, so the ratio is unaffected.
//  * varlen masks keys only in a request's last, partial tile; block-local
//    masks each row to [lo, hi) computed from integers (no dense mask, no
//    device-to-host decision) and loads only the union of the rows' windows.
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
};

// ---------------------------------------------------------------- tile setup

struct TileRange {
  int h;        // head
  int q0, q1;   // absolute query rows [q0, q1)
  int kv_base;  // absolute row of key 0 of the sequence
  int k_lo, k_hi;  // keys of the tile, relative to kv_base
  int seq_q0;   // row of q0 inside its sequence (block-local windows)
  bool valid;
};

template <int BM, bool kBlockLocal>
__device__ __forceinline__ TileRange tile_range(const AttnArgs& a) {
  TileRange t;
  t.valid = true;
  if (!kBlockLocal) {
    const int logical = block_to_logical(blockIdx.x, a.chunk);
    int req, head, qt;
    find_tile(a.q_cu, a.kv_cu, a.R, a.H, BM, logical, req, head, qt);
    if (req < 0) {
      t.valid = false;
      return t;
    }
    const int qs = a.q_cu[req];
    const int qe = a.q_cu[req + 1];
    t.h = head;
    t.q0 = qs + qt * BM;
    t.q1 = min(qe, t.q0 + BM);
    t.kv_base = a.kv_cu[req];
    t.k_lo = 0;
    t.k_hi = a.kv_cu[req + 1] - t.kv_base;
    t.seq_q0 = qt * BM;
  } else {
    const int id = blockIdx.x;
    const int qt = id % a.nqt;
    const int bh = id / a.nqt;
    t.h = bh % a.H;
    const int b = bh / a.H;
    const int i0 = qt * BM;
    const int i1 = min(a.n, i0 + BM);
    t.q0 = b * a.n + i0;
    t.q1 = b * a.n + i1;
    t.kv_base = b * a.n;
    t.seq_q0 = i0;
    const int nb = (a.n + a.block - 1) / a.block;
    const int blo = max(0, i0 / a.block - a.look_back);
    const int bhi = min(nb - 1, (i1 - 1) / a.block + a.look_ahead);
    t.k_lo = blo * a.block;
    t.k_hi = min(a.n, (bhi + 1) * a.block);
  }
  return t;
}

// Keys [lo, hi) of sequence row i under the block window.
__device__ __forceinline__ void window_of(const AttnArgs& a, int i, int& lo, int& hi) {
  const int nb = (a.n + a.block - 1) / a.block;
  const int b = i / a.block;
  lo = max(0, b - a.look_back) * a.block;
  hi = min(a.n, (min(nb - 1, b + a.look_ahead) + 1) * a.block);
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

template <int D>
struct Bf16Geo {
  static constexpr int kThreads = 256;
  static constexpr int BM = 128;
  static constexpr int BN = 8192 / D;                   // keys per tile
  static constexpr int kKStride = D * 2 + 16;           // bytes per K row in LDS
  static constexpr int kKBytes = BN * kKStride;
  static constexpr int kVtRow = BN * 2;                 // bytes per V^T row
  static constexpr int kVBytes = D * kVtRow;
  static constexpr int kBufBytes = kKBytes + kVBytes;
  static constexpr int kLdsBytes = 2 * kBufBytes;
  static constexpr int DCH = D / 8;                     // 16-byte chunks per row
  static constexpr int kKPasses = BN * DCH / kThreads;
  static constexpr int NKB = BN / 32;
  static constexpr int NDS = D / 16;
  static constexpr int NDB = D / 32;
  static constexpr int NKC = BN / 16;
  static_assert((BN / 4) * DCH == kThreads, "one V transpose task per thread");
};

// 16-byte chunk swizzle of a V^T row: rows d..d+7 read the same logical chunk
// from 8 different bank groups, and the transposing writes of one wave land
// at most two to a bank group.
__device__ __forceinline__ int vt_swizzle(int d) { return (d ^ (d >> 3)) & 7; }

template <int D, bool kBlockLocal>
__global__ void __launch_bounds__(256, 2) attn_bf16_kernel(AttnArgs a) {
  using G = Bf16Geo<D>;
  __shared__ __attribute__((aligned(16))) char smem[G::kLdsBytes];

  const TileRange tr = tile_range<G::BM, kBlockLocal>(a);
  if (!tr.valid) return;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int ql = lane & 31;
  const int g = lane >> 5;
  const int H = a.H;
  const int h = tr.h;
  const int64_t row_stride = (int64_t)H * D;  // elements between consecutive tokens

  const __bf16* __restrict__ qg = (const __bf16*)a.q;
  const __bf16* __restrict__ kg = (const __bf16*)a.k;
  const __bf16* __restrict__ vg = (const __bf16*)a.v;

  // Query row of this lane and its key window.
  const int my_row = tr.q0 + wave * 32 + ql;
  const bool row_ok = my_row < tr.q1;
  const bool wave_active = tr.q0 + wave * 32 < tr.q1;
  int lo = tr.k_lo, hi = tr.k_hi;
  if (kBlockLocal) {
    const int i = min(tr.seq_q0 + wave * 32 + ql, a.n - 1);
    window_of(a, i, lo, hi);
  }

  bf16x8 qf[G::NDS];
  {
    const __bf16* qp = qg + (int64_t)my_row * row_stride + (int64_t)h * D + g * 8;
#pragma unroll
    for (int ds = 0; ds < G::NDS; ++ds)
      qf[ds] = row_ok ? *(const bf16x8*)(qp + ds * 16) : bf16x8{};
  }

  RowState<G::NKB, G::NDB> st;
  st.init();

  const int nkeys = tr.k_hi - tr.k_lo;
  const int ntiles = (nkeys + G::BN - 1) / G::BN;

  // Per-thread copy tasks of one tile.
  u32x4 kr[G::kKPasses];
  u32x4 vr[4];
  const int v_dc = tid % G::DCH;   // feature chunk (8 features) of the V task
  const int v_kg = tid / G::DCH;   // key group (4 keys) of the V task

  auto gload = [&](int tile) {
    const int key0 = tr.k_lo + tile * G::BN;
    const int valid = min(G::BN, tr.k_hi - key0);
    const int64_t base = (int64_t)(tr.kv_base + key0) * row_stride + (int64_t)h * D;
    // Rows past the last valid key re-read the last valid row: their scores
    // are masked to -inf, so they carry probability 0 times finite data.
#pragma unroll
    for (int p = 0; p < G::kKPasses; ++p) {
      const int idx = p * G::kThreads + tid;
      const int row = min(idx / G::DCH, valid - 1);
      const int ch = idx % G::DCH;
      kr[p] = *(const u32x4*)(kg + base + (int64_t)row * row_stride + ch * 8);
    }
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      const int row = min(4 * v_kg + c, valid - 1);
      vr[c] = *(const u32x4*)(vg + base + (int64_t)row * row_stride + v_dc * 8);
    }
  };

  auto lstore = [&](int buf) {
    char* kl = smem + buf * G::kBufBytes;
    char* vl = kl + G::kKBytes;
#pragma unroll
    for (int p = 0; p < G::kKPasses; ++p) {
      const int idx = p * G::kThreads + tid;
      const int row = idx / G::DCH;
      const int ch = idx % G::DCH;
      *(u32x4*)(kl + row * G::kKStride + ch * 16) = kr[p];
    }
    // V^T[d][slot]: keys 4*kg..4*kg+3 of feature d, in the slot order the
    // P operand expects (bits 2 and 3 of the key index swapped).
    const int chunk = 2 * (v_kg >> 2) + (v_kg & 1);
    const int half = (v_kg >> 1) & 1;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const int w = e >> 1;
      uint32_t lo2, hi2;
      if ((e & 1) == 0) {
        lo2 = (vr[0][w] & 0xffffu) | (vr[1][w] << 16);
        hi2 = (vr[2][w] & 0xffffu) | (vr[3][w] << 16);
      } else {
        lo2 = (vr[0][w] >> 16) | (vr[1][w] & 0xffff0000u);
        hi2 = (vr[2][w] >> 16) | (vr[3][w] & 0xffff0000u);
      }
      const int d = 8 * v_dc + e;
      const int phys = chunk ^ vt_swizzle(d);
      *(u32x2*)(vl + d * G::kVtRow + phys * 16 + half * 8) = u32x2{lo2, hi2};
    }
  };

  auto compute = [&](int buf, int tile, bool masked) {
    const char* kl = smem + buf * G::kBufBytes;
    const char* vl = kl + G::kKBytes;
    f32x16 s[G::NKB];
#pragma unroll
    for (int kb = 0; kb < G::NKB; ++kb) {
      s[kb] = f32x16{};
#pragma unroll
      for (int ds = 0; ds < G::NDS; ++ds) {
        const bf16x8 ka = *(const bf16x8*)(kl + (kb * 32 + ql) * G::kKStride + ds * 32 + g * 16);
        s[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ka, qf[ds], s[kb], 0, 0, 0);
      }
    }
    if (masked) mask_scores<G::NKB>(s, tr.k_lo + tile * G::BN, g, lo, hi);
    st.softmax_tile(s, a.c);
    bf16x8 pf[G::NKC];
#pragma unroll
    for (int kc = 0; kc < G::NKC; ++kc)
#pragma unroll
      for (int e = 0; e < 8; ++e) pf[kc][e] = (__bf16)s[kc >> 1][8 * (kc & 1) + e];
#pragma unroll
    for (int db = 0; db < G::NDB; ++db) {
      const int d = db * 32 + ql;
      const char* vrow = vl + d * G::kVtRow;
      const int sw = vt_swizzle(d);
#pragma unroll
      for (int kc = 0; kc < G::NKC; ++kc) {
        const bf16x8 va = *(const bf16x8*)(vrow + (((2 * kc + g) ^ sw) * 16));
        st.o[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(va, pf[kc], st.o[db], 0, 0, 0);
      }
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
  const float inv = l_tot > 0.f ? 1.0f / l_tot : 0.f;
  if (row_ok) {
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

  const TileRange tr = tile_range<G::BM, kBlockLocal>(a);
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

// ---------------------------------------------------------------- tile-map export

template <int BM>
__global__ void __launch_bounds__(64) tile_map_kernel(const int32_t* q_cu, const int32_t* kv_cu,
                                                      int R, int H, int chunk, int32_t* out) {
  const int logical = block_to_logical(blockIdx.x, chunk);
  int req, head, qt;
  find_tile(q_cu, kv_cu, R, H, BM, logical, req, head, qt);
  if (threadIdx.x == 0) {
    out[3 * (int64_t)blockIdx.x + 0] = req;
    out[3 * (int64_t)blockIdx.x + 1] = req < 0 ? -1 : head;
    out[3 * (int64_t)blockIdx.x + 2] = req < 0 ? -1 : qt;
  }
}

}  // namespace vl

// ============================================================================ host side

namespace {

constexpr int kChunk = 16;  // logical tiles kept together on one chiplet

inline bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

int launch_status() {
  return hipGetLastError() == hipSuccess ? VL_OK : VL_ELAUNCH;
}

template <bool kF32>
int varlen_common(const void* q, const void* k, const void* v, const int32_t* q_cu,
                  const int32_t* kv_cu, int32_t max_q, int32_t max_kv, int32_t num_reqs,
                  int32_t H, int32_t D, float scale, void* out, float* lse, hipStream_t stream) {
  if (num_reqs < 0 || max_q < 0 || max_kv < 0 || H < 1) return VL_EINVAL;
  if (D != 64 && D != 128) return VL_EUNSUPPORTED;
  if (num_reqs == 0 || max_q == 0) return VL_OK;
  if (!q || !k || !v || !q_cu || !kv_cu || !out) return VL_EINVAL;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(out)) return VL_EINVAL;
  if (!(scale == scale)) return VL_EINVAL;
  const int64_t G = vl::grid_blocks(num_reqs, max_q, H, 128, kChunk);
  if (G > INT32_MAX) return VL_EUNSUPPORTED;
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
  (void)hipGetLastError();
  if (kF32) {
    if (D == 128)
      hipLaunchKernelGGL((vl::attn_f32_kernel<128, false>), dim3((unsigned)G), dim3(256), 0, stream, a);
    else
      hipLaunchKernelGGL((vl::attn_f32_kernel<64, false>), dim3((unsigned)G), dim3(256), 0, stream, a);
  } else {
    if (D == 128)
      hipLaunchKernelGGL((vl::attn_bf16_kernel<128, false>), dim3((unsigned)G), dim3(256), 0, stream, a);
    else
      hipLaunchKernelGGL((vl::attn_bf16_kernel<64, false>), dim3((unsigned)G), dim3(256), 0, stream, a);
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
  if (!(scale == scale)) return VL_EINVAL;
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
  a.look_back = look_back;
  a.look_ahead = look_ahead;
  a.nqt = nqt;
  (void)hipGetLastError();
  if (kF32) {
    if (D == 128)
      hipLaunchKernelGGL((vl::attn_f32_kernel<128, true>), dim3((unsigned)G), dim3(256), 0, stream, a);
    else
      hipLaunchKernelGGL((vl::attn_f32_kernel<64, true>), dim3((unsigned)G), dim3(256), 0, stream, a);
  } else {
    if (D == 128)
      hipLaunchKernelGGL((vl::attn_bf16_kernel<128, true>), dim3((unsigned)G), dim3(256), 0, stream, a);
    else
      hipLaunchKernelGGL((vl::attn_bf16_kernel<64, true>), dim3((unsigned)G), dim3(256), 0, stream, a);
  }
  return launch_status();
}

}  // namespace

extern "C" {

int varlen_attn_fwd(const void* q, const void* k, const void* v, const int32_t* q_cu_seqlens,
                    const int32_t* kv_cu_seqlens, int32_t max_q, int32_t max_kv, int32_t num_reqs,
                    int32_t H, int32_t D, float scale, void* out, float* lse, vl_stream_t stream) {
  return varlen_common<false>(q, k, v, q_cu_seqlens, kv_cu_seqlens, max_q, max_kv, num_reqs, H, D,
                              scale, out, lse, (hipStream_t)stream);
}

int varlen_attn_fwd_f32(const float* q, const float* k, const float* v,
                        const int32_t* q_cu_seqlens, const int32_t* kv_cu_seqlens, int32_t max_q,
                        int32_t max_kv, int32_t num_reqs, int32_t H, int32_t D, float scale,
                        float* out, float* lse, vl_stream_t stream) {
  return varlen_common<true>(q, k, v, q_cu_seqlens, kv_cu_seqlens, max_q, max_kv, num_reqs, H, D,
                             scale, out, lse, (hipStream_t)stream);
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

int varlen_launch_shape(int32_t max_q, int32_t num_reqs, int32_t H, int32_t D, int dtype_f32,
                        int32_t* block_m, int32_t* chunk, int64_t* blocks) {
  (void)dtype_f32;
  if (max_q < 0 || num_reqs < 0 || H < 1) return VL_EINVAL;
  if (D != 64 && D != 128) return VL_EUNSUPPORTED;
  if (block_m) *block_m = 128;
  if (chunk) *chunk = kChunk;
  if (blocks) *blocks = (num_reqs == 0 || max_q == 0) ? 0 : vl::grid_blocks(num_reqs, max_q, H, 128, kChunk);
  return VL_OK;
}

int varlen_tile_map(const int32_t* q_cu_seqlens, const int32_t* kv_cu_seqlens, int32_t max_q,
                    int32_t num_reqs, int32_t H, int32_t D, int dtype_f32, int32_t* triples_out,
                    int64_t max_blocks, vl_stream_t stream) {
  int64_t G = 0;
  const int rc = varlen_launch_shape(max_q, num_reqs, H, D, dtype_f32, nullptr, nullptr, &G);
  if (rc != VL_OK) return rc;
  if (G == 0) return VL_OK;
  if (!q_cu_seqlens || !kv_cu_seqlens || !triples_out || max_blocks < G) return VL_EINVAL;
  if (G > INT32_MAX) return VL_EUNSUPPORTED;
  (void)hipGetLastError();
  hipLaunchKernelGGL((vl::tile_map_kernel<128>), dim3((unsigned)G), dim3(64), 0, (hipStream_t)stream,
                     q_cu_seqlens, kv_cu_seqlens, num_reqs, H, kChunk, triples_out);
  return launch_status();
}

}  // extern "C"
