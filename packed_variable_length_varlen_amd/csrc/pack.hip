// Boundaries (cu_seqlens) and pack / unpack gathers for gfx950.
//
// pack: only real tokens of each request enter the flat buffer (vLLM-Omni
// PR #4024 "How batching works"); unpack scatters flat rows back to the
// per-request padded layout (PR #6711 "Key changes": output unpacked by
// cu_seqlens).  A request's rows are contiguous on both sides, so each request
// is one contiguous copy of len_r * row_bytes bytes: the kernels stream it
// with the widest aligned vector, several independent loads in flight per
// thread, and no per-row index arithmetic.
#include "vl_device.h"

namespace vl {

constexpr int kCopyThreads = 256;
// 16-byte loads in flight per thread.  Unpack: 2 (beats 4 and 8 on large
// copies).  Pack: 4; its padded source slabs can be mostly empty (requests
// far shorter than the slab), and every block past a request's end still
// launches its waves before exiting: at four loads per thread half as many
// waves are launched, which lifts a sparse batch (requests of 4,096-16,384
// rows in 16,384-row slabs) from 65 to 73 % of HBM while dense batches stay
// within 1.5-3 points.
template <bool kPack>
constexpr int copy_unroll() { return kPack ? 4 : 2; }
template <bool kPack>
constexpr int units_per_block() { return kCopyThreads * copy_unroll<kPack>(); }
constexpr int kCfgUnroll = 2;  // the CFG combine (two source rows per output row)
constexpr int kCfgUnitsPerBlock = kCopyThreads * kCfgUnroll;

// Request r = blockIdx.y copies units [0, len_r*row_units) of its slab in
// src (starting at r * src_slab_units) to dst starting at off_r * row_units;
// with zero_tail, units [len_r*row_units, slab_units) of the destination slab
// are zeroed (unpack).  For pack, the destination is flat (dst_flat = true).
template <typename U, bool kPack>
__global__ void __launch_bounds__(kCopyThreads) copy_segments_kernel(
    const U* __restrict__ src, U* __restrict__ dst, const int32_t* __restrict__ cu,
    const int32_t* __restrict__ offsets, int64_t row_units, int64_t slab_rows, int zero_tail) {
  const int r = blockIdx.y;
  const int64_t len = (int64_t)(cu[r + 1] - cu[r]);
  const int64_t off = offsets != nullptr ? (int64_t)offsets[r] : (int64_t)cu[r];
  const int64_t real_units = len * row_units;
  const int64_t span_units = (!kPack && zero_tail) ? slab_rows * row_units : real_units;
  constexpr int UN = copy_unroll<kPack>();
  const int64_t u0 = (int64_t)blockIdx.x * units_per_block<kPack>();
  if (u0 >= span_units) return;
  const U* s;
  U* d;
  if (kPack) {
    s = src + (int64_t)r * slab_rows * row_units;
    d = dst + off * row_units;
  } else {
    s = src + off * row_units;
    d = dst + (int64_t)r * slab_rows * row_units;
  }
  U buf[UN];
#pragma unroll
  for (int i = 0; i < UN; ++i) {
    const int64_t u = u0 + i * kCopyThreads + threadIdx.x;
    buf[i] = u < real_units ? (kPack ? __builtin_nontemporal_load(s + u) : s[u]) : U{};
  }
  // Streaming stores: the destination is not re-read by this kernel.
#pragma unroll
  for (int i = 0; i < UN; ++i) {
    const int64_t u = u0 + i * kCopyThreads + threadIdx.x;
    if (u < span_units) __builtin_nontemporal_store(buf[i], d + u);
  }
}

// Up to kMaxBatch pack (or unpack) copies in one launch, 16-byte units.
// Blocks are numbered flat: copy i owns blocks [b0[i], b0[i+1]), bx[i] per
// request; block b0[i] + r*bx[i] + j streams units [j, j+1) * units_per_block
// of request r.  The descriptors travel by value in the kernel arguments.
constexpr int kMaxBatch = 8;
struct CopyBatch {
  const u32x4* src[kMaxBatch];
  u32x4* dst[kMaxBatch];
  const int32_t* cu[kMaxBatch];
  const int32_t* offsets[kMaxBatch];
  int64_t row_units[kMaxBatch];
  int64_t slab_rows[kMaxBatch];
  int64_t bx[kMaxBatch];
  int64_t b0[kMaxBatch + 1];
  int zero_tail[kMaxBatch];
  int count;
};

template <bool kPack>
__global__ void __launch_bounds__(kCopyThreads) copy_batch_kernel(CopyBatch cb) {
  // the host caps the grid at INT32_MAX blocks: 32-bit block arithmetic
  const uint32_t b = blockIdx.x;
  int i = 0;
  while (i + 1 < cb.count && b >= (uint32_t)cb.b0[i + 1]) ++i;
  const uint32_t local = b - (uint32_t)cb.b0[i];
  const uint32_t bxi = (uint32_t)cb.bx[i];
  const int r = (int)(local / bxi);
  const int64_t row_units = cb.row_units[i];
  const int64_t slab_rows = cb.slab_rows[i];
  const int32_t* cu = cb.cu[i];
  const int64_t len = (int64_t)(cu[r + 1] - cu[r]);
  const int64_t off = cb.offsets[i] != nullptr ? (int64_t)cb.offsets[i][r] : (int64_t)cu[r];
  const int64_t real_units = len * row_units;
  const int64_t span_units = (!kPack && cb.zero_tail[i]) ? slab_rows * row_units : real_units;
  constexpr int UN = copy_unroll<kPack>();
  const int64_t u0 = (int64_t)(local - (uint32_t)r * bxi) * units_per_block<kPack>();
  if (u0 >= span_units) return;
  const u32x4* s = kPack ? cb.src[i] + (int64_t)r * slab_rows * row_units : cb.src[i] + off * row_units;
  u32x4* d = kPack ? cb.dst[i] + off * row_units : cb.dst[i] + (int64_t)r * slab_rows * row_units;
  u32x4 buf[UN];
#pragma unroll
  for (int k = 0; k < UN; ++k) {
    const int64_t u = u0 + k * kCopyThreads + threadIdx.x;
    // pack sources (the padded slabs) are streamed once: non-temporal loads
    // (+2.5-3.5 points of HBM); an unpack source is the attention output just
    // written, often still in the last-level cache, which they would pass by
    buf[k] = u < real_units ? (kPack ? __builtin_nontemporal_load(s + u) : s[u]) : u32x4{};
  }
#pragma unroll
  for (int k = 0; k < UN; ++k) {
    const int64_t u = u0 + k * kCopyThreads + threadIdx.x;
    if (u < span_units) __builtin_nontemporal_store(buf[k], d + u);
  }
}

// fp64 -> bf16 with a single rounding (nearest even): round to odd into fp32,
// which keeps every discarded bit as a sticky bit, then nearest-even to bf16.
__device__ __forceinline__ uint32_t f64_to_bf16_bits(double x) {
  const float f = (float)x;
  uint32_t b = __float_as_uint(f);
  const double back = (double)f;
  if (back != x) {
    if (fabs(back) > fabs(x)) b -= 1u;  // the value truncated toward zero
    b |= 1u;
  }
  return (uint32_t)__builtin_bit_cast(uint16_t, (__bf16)__uint_as_float(b));
}

// CFG combine fused into unpack: request r = blockIdx.y, 8 bf16 elements
// (16 bytes) per unit.  dst = neg + s * (pos - neg) in fp64: the difference of
// two bf16 values is exact there (unless their exponents lie more than 45
// apart), so the result is rounded once, and scale 0 / 1 return neg / pos
// bit for bit.  In fp32 the difference rounds as soon as the exponents lie
// more than 16 apart, and scale 1 then misses pos by an ulp.
__global__ void __launch_bounds__(kCopyThreads) cfg_combine_kernel(
    const u32x4* __restrict__ src, const int32_t* __restrict__ seg_cu, const int32_t* __restrict__ pos_rows,
    const int32_t* __restrict__ neg_rows, const float* __restrict__ scale, int64_t row_units,
    u32x4* __restrict__ dst, int64_t slab_rows, int zero_tail) {
  const int r = blockIdx.y;
  const int64_t len = (int64_t)(seg_cu[r + 1] - seg_cu[r]);
  const int64_t real_units = len * row_units;
  const int64_t span_units = zero_tail ? slab_rows * row_units : real_units;
  const int64_t u0 = (int64_t)blockIdx.x * kCfgUnitsPerBlock;
  if (u0 >= span_units) return;
  const u32x4* ps = src + (int64_t)pos_rows[r] * row_units;
  const u32x4* ns = src + (int64_t)neg_rows[r] * row_units;
  u32x4* d = dst + (int64_t)r * slab_rows * row_units;
  const double s = (double)scale[r];
#pragma unroll
  for (int i = 0; i < kCfgUnroll; ++i) {
    const int64_t u = u0 + i * kCopyThreads + threadIdx.x;
    if (u >= span_units) continue;
    u32x4 y = u32x4{};
    if (u < real_units) {
      const u32x4 p = ps[u];
      const u32x4 n = ns[u];
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        // two bf16 per word, widened exactly
        const double p0 = (double)__uint_as_float(p[w] << 16), p1 = (double)__uint_as_float(p[w] & 0xffff0000u);
        const double n0 = (double)__uint_as_float(n[w] << 16), n1 = (double)__uint_as_float(n[w] & 0xffff0000u);
        y[w] = f64_to_bf16_bits(fma(s, p0 - n0, n0)) | (f64_to_bf16_bits(fma(s, p1 - n1, n1)) << 16);
      }
    }
    __builtin_nontemporal_store(y, d + u);
  }
}

// Inclusive scan of one value per thread over a 256-thread block.
__device__ __forceinline__ int block_scan_256(int x, int* lds8) {
  const int lane = lane_id();
  const int wave = threadIdx.x >> 6;
  int incl = x;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const int y = __shfl_up(incl, off);
    if (lane >= off) incl += y;
  }
  if (lane == 63) lds8[wave] = incl;
  __syncthreads();
  int add = 0;
  for (int w = 0; w < wave; ++w) add += lds8[w];
  __syncthreads();
  return incl + add;
}

// One 256-thread block: cu_out[0] = 0, cu_out[r+1] = sum of lengths[0..r].
__global__ void __launch_bounds__(256) cu_from_lengths_kernel(const int32_t* __restrict__ lengths,
                                                              int R, int32_t* __restrict__ cu) {
  __shared__ int lds8[8];
  __shared__ int carry_s;
  if (threadIdx.x == 0) {
    cu[0] = 0;
    carry_s = 0;
  }
  __syncthreads();
  for (int r0 = 0; r0 < R; r0 += 256) {
    const int r = r0 + threadIdx.x;
    const int x = r < R ? lengths[r] : 0;
    const int incl = block_scan_256(x, lds8);
    const int carry = carry_s;
    if (r < R) cu[r + 1] = carry + incl;
    __syncthreads();
    if (threadIdx.x == 255) carry_s = carry + incl;
    __syncthreads();
  }
}

// Number of nonzero bytes of request r's mask row, summed by one wave
// (4-byte words when the row is word-aligned, else bytes).  Wave-uniform.
__device__ __forceinline__ int wave_count_nonzero(const uint8_t* __restrict__ row, int cap) {
  const int lane = lane_id();
  int cnt = 0;
  if ((cap & 3) == 0 && (((uintptr_t)row) & 3) == 0) {
    const uint32_t* w = (const uint32_t*)row;
    for (int i = lane; i < cap / 4; i += 64) {
      const uint32_t x = w[i];
      cnt += ((x & 0xffu) != 0) + ((x & 0xff00u) != 0) + ((x & 0xff0000u) != 0) + ((x & 0xff000000u) != 0);
    }
  } else {
    for (int i = lane; i < cap; i += 64) cnt += row[i] != 0;
  }
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) cnt += __shfl_xor(cnt, off);
  return cnt;
}

// One 256-thread block: text lengths from the mask (one wave per request),
// image tokens from the grids, and the joint / text / image boundaries plus
// each image segment's first packed row, 256 requests at a time.
__global__ void __launch_bounds__(256) joint_cu_kernel(const uint8_t* __restrict__ mask,
                                                       int text_cap, const int32_t* __restrict__ hw,
                                                       int R, int32_t* cu_joint, int32_t* cu_text,
                                                       int32_t* cu_img, int32_t* img_dst) {
  __shared__ int lds8[8];
  __shared__ int carry[3];
  __shared__ int tlen[256];
  const int wave = threadIdx.x >> 6;
  if (threadIdx.x < 3) carry[threadIdx.x] = 0;
  if (threadIdx.x == 0) {
    if (cu_joint) cu_joint[0] = 0;
    if (cu_text) cu_text[0] = 0;
    if (cu_img) cu_img[0] = 0;
  }
  for (int r0 = 0; r0 < R; r0 += 256) {
    const int nr = min(256, R - r0);
    for (int i = wave; i < nr; i += 4) {
      const int c = text_cap > 0 ? wave_count_nonzero(mask + (int64_t)(r0 + i) * text_cap, text_cap) : 0;
      if (lane_id() == 0) tlen[i] = c;
    }
    __syncthreads();
    const int r = r0 + threadIdx.x;
    int t = 0, n = 0;
    if (r < R) {
      t = tlen[threadIdx.x];
      n = hw[2 * r] * hw[2 * r + 1];
    }
    const int it = block_scan_256(t, lds8);
    const int in = block_scan_256(n, lds8);
    const int ij = block_scan_256(t + n, lds8);
    const int ct = carry[0], cn = carry[1], cj = carry[2];
    if (r < R) {
      if (cu_text) cu_text[r + 1] = ct + it;
      if (cu_img) cu_img[r + 1] = cn + in;
      if (cu_joint) cu_joint[r + 1] = cj + ij;
      if (img_dst) img_dst[r] = cj + ij - (t + n) + t;
    }
    __syncthreads();
    if (threadIdx.x == 255) {
      carry[0] = ct + it;
      carry[1] = cn + in;
      carry[2] = cj + ij;
    }
    __syncthreads();
  }
}

}  // namespace vl

// ============================================================================ host side

namespace {

constexpr int kMaxReqs = 65535;  // grid.y bound of the copy kernels

int launch_status() { return hipGetLastError() == hipSuccess ? VL_OK : VL_ELAUNCH; }

template <bool kPack>
int copy_common(const void* src, void* dst, const int32_t* cu, const int32_t* offsets,
                int32_t num_reqs, int64_t row_bytes, int64_t slab_rows, int zero_tail,
                hipStream_t stream) {
  if (num_reqs < 0 || num_reqs > kMaxReqs || row_bytes <= 0 || slab_rows < 0) return VL_EINVAL;
  if (num_reqs == 0 || slab_rows == 0) return VL_OK;
  if (!src || !dst || !cu) return VL_EINVAL;
  const uintptr_t a = (uintptr_t)src | (uintptr_t)dst;
  int64_t unit;
  if (row_bytes % 16 == 0 && (a & 15u) == 0)
    unit = 16;
  else if (row_bytes % 4 == 0 && (a & 3u) == 0)
    unit = 4;
  else
    unit = 1;
  const int64_t row_units = row_bytes / unit;
  const int64_t slab_units = slab_rows * row_units;
  const int64_t bx = (slab_units + vl::units_per_block<kPack>() - 1) / vl::units_per_block<kPack>();
  if (bx > INT32_MAX) return VL_EUNSUPPORTED;
  const dim3 grid((unsigned)bx, (unsigned)num_reqs);
  (void)hipGetLastError();
  if (unit == 16)
    hipLaunchKernelGGL((vl::copy_segments_kernel<vl::u32x4, kPack>), grid, dim3(vl::kCopyThreads), 0,
                       stream, (const vl::u32x4*)src, (vl::u32x4*)dst, cu, offsets, row_units,
                       slab_rows, zero_tail);
  else if (unit == 4)
    hipLaunchKernelGGL((vl::copy_segments_kernel<uint32_t, kPack>), grid, dim3(vl::kCopyThreads), 0,
                       stream, (const uint32_t*)src, (uint32_t*)dst, cu, offsets, row_units,
                       slab_rows, zero_tail);
  else
    hipLaunchKernelGGL((vl::copy_segments_kernel<uint8_t, kPack>), grid, dim3(vl::kCopyThreads), 0,
                       stream, (const uint8_t*)src, (uint8_t*)dst, cu, offsets, row_units,
                       slab_rows, zero_tail);
  return launch_status();
}

// One launch for up to kMaxBatch copies when every one of them can move
// 16-byte units; otherwise one launch per copy.
template <bool kPack>
int copy_batched(const vl_copy_desc* descs, int32_t count, hipStream_t stream) {
  if (count < 0 || count > vl::kMaxBatch || (count > 0 && !descs)) return VL_EINVAL;
  bool wide = true;
  for (int32_t i = 0; i < count; ++i) {
    const vl_copy_desc& c = descs[i];
    if (c.num_reqs < 0 || c.num_reqs > kMaxReqs || c.row_bytes <= 0 || c.max_len < 0) return VL_EINVAL;
    if (c.num_reqs == 0 || c.max_len == 0) continue;
    if (!c.src || !c.dst || !c.cu_seqlens) return VL_EINVAL;
    if (c.row_bytes % 16 != 0 || (((uintptr_t)c.src | (uintptr_t)c.dst) & 15u) != 0) wide = false;
  }
  if (!wide) {
    for (int32_t i = 0; i < count; ++i) {
      const vl_copy_desc& c = descs[i];
      const int rc = copy_common<kPack>(c.src, c.dst, c.cu_seqlens, c.row_offsets, c.num_reqs, c.row_bytes,
                                        c.max_len, kPack ? 0 : c.zero_fill, stream);
      if (rc != VL_OK) return rc;
    }
    return VL_OK;
  }
  vl::CopyBatch cb{};
  int64_t blocks = 0;
  for (int32_t i = 0; i < count; ++i) {
    const vl_copy_desc& c = descs[i];
    const int n = cb.count;
    if (c.num_reqs == 0 || c.max_len == 0) continue;
    cb.src[n] = (const vl::u32x4*)c.src;
    cb.dst[n] = (vl::u32x4*)c.dst;
    cb.cu[n] = c.cu_seqlens;
    cb.offsets[n] = c.row_offsets;
    cb.row_units[n] = c.row_bytes / 16;
    cb.slab_rows[n] = c.max_len;
    cb.bx[n] = (c.max_len * cb.row_units[n] + vl::units_per_block<kPack>() - 1) / vl::units_per_block<kPack>();
    cb.zero_tail[n] = kPack ? 0 : (c.zero_fill != 0);
    cb.b0[n] = blocks;
    blocks += cb.bx[n] * c.num_reqs;
    cb.count = n + 1;
  }
  if (cb.count == 0) return VL_OK;
  cb.b0[cb.count] = blocks;
  if (blocks > INT32_MAX) return VL_EUNSUPPORTED;
  (void)hipGetLastError();
  hipLaunchKernelGGL((vl::copy_batch_kernel<kPack>), dim3((unsigned)blocks), dim3(vl::kCopyThreads), 0, stream, cb);
  return launch_status();
}

}  // namespace

extern "C" {

int vl_version(void) { return 100; }

int pack_by_cu_seqlens_batched(const vl_copy_desc* descs, int32_t count, vl_stream_t stream) {
  return copy_batched<true>(descs, count, (hipStream_t)stream);
}

int unpack_by_cu_seqlens_batched(const vl_copy_desc* descs, int32_t count, vl_stream_t stream) {
  return copy_batched<false>(descs, count, (hipStream_t)stream);
}

int mixfusion_chunk_plan(const int64_t* token_counts, int32_t n, int64_t min_chunk_tokens,
                         int64_t max_chunks, int64_t* chunk_size, int64_t* chunk_count) {
  if (!token_counts || n < 1) return VL_EINVAL;
  int64_t g = 0, total = 0;
  for (int32_t i = 0; i < n; ++i) {
    const int64_t c = token_counts[i];
    if (c < 1) return VL_EINVAL;
    int64_t a = g, b = c;
    while (b != 0) {
      const int64_t t = a % b;
      a = b;
      b = t;
    }
    g = a;
    total += c;
  }
  const int64_t count = total / g;
  if (chunk_size) *chunk_size = g;
  if (chunk_count) *chunk_count = count;
  return (g >= min_chunk_tokens && count <= max_chunks) ? 1 : 0;
}

const char* vl_status_string(int status) {
  switch (status) {
    case VL_OK: return "ok";
    case VL_EINVAL: return "invalid argument";
    case VL_EUNSUPPORTED: return "unsupported size";
    case VL_ELAUNCH: return "kernel launch failed";
    default: return "unknown status";
  }
}

int unpack_cfg_combine(const void* src_flat, const int32_t* seg_cu, const int32_t* pos_rows,
                       const int32_t* neg_rows, const float* scale, int32_t num_reqs,
                       int64_t row_elems, void* dst_padded, int64_t max_len, int zero_fill,
                       vl_stream_t stream) {
  if (num_reqs < 0 || num_reqs > kMaxReqs || row_elems <= 0 || max_len < 0) return VL_EINVAL;
  if (row_elems % 8 != 0) return VL_EUNSUPPORTED;
  if (num_reqs == 0 || max_len == 0) return VL_OK;
  if (!src_flat || !seg_cu || !pos_rows || !neg_rows || !scale || !dst_padded) return VL_EINVAL;
  if ((((uintptr_t)src_flat) | ((uintptr_t)dst_padded)) & 15u) return VL_EINVAL;
  const int64_t row_units = row_elems / 8;
  const int64_t bx = (max_len * row_units + vl::kCfgUnitsPerBlock - 1) / vl::kCfgUnitsPerBlock;
  if (bx > INT32_MAX) return VL_EUNSUPPORTED;
  (void)hipGetLastError();
  hipLaunchKernelGGL(vl::cfg_combine_kernel, dim3((unsigned)bx, (unsigned)num_reqs), dim3(vl::kCopyThreads), 0,
                     (hipStream_t)stream, (const vl::u32x4*)src_flat, seg_cu, pos_rows, neg_rows, scale, row_units,
                     (vl::u32x4*)dst_padded, max_len, zero_fill);
  return launch_status();
}

int cu_seqlens_from_lengths(const int32_t* lengths, int32_t num_reqs, int32_t* cu_out,
                            vl_stream_t stream) {
  if (num_reqs < 0 || num_reqs > kMaxReqs + 1 || !cu_out) return VL_EINVAL;
  if (num_reqs > 0 && !lengths) return VL_EINVAL;
  (void)hipGetLastError();
  hipLaunchKernelGGL(vl::cu_from_lengths_kernel, dim3(1), dim3(256), 0, (hipStream_t)stream,
                     lengths, num_reqs, cu_out);
  return launch_status();
}

int joint_cu_seqlens(const uint8_t* text_mask, int32_t text_cap, const int32_t* img_hw,
                     int32_t num_reqs, int32_t* cu_joint, int32_t* cu_text, int32_t* cu_img,
                     int32_t* img_dst, vl_stream_t stream) {
  if (num_reqs < 0 || num_reqs > kMaxReqs + 1 || text_cap < 0) return VL_EINVAL;
  if (num_reqs > 0 && (!img_hw || (text_cap > 0 && !text_mask))) return VL_EINVAL;
  if (!cu_joint && !cu_text && !cu_img && !img_dst) return VL_OK;
  (void)hipGetLastError();
  hipLaunchKernelGGL(vl::joint_cu_kernel, dim3(1), dim3(256), 0, (hipStream_t)stream, text_mask,
                     text_cap, img_hw, num_reqs, cu_joint, cu_text, cu_img, img_dst);
  return launch_status();
}

int pack_by_cu_seqlens(const void* src_padded, int64_t max_len, const int32_t* cu_seqlens,
                       int32_t num_reqs, int64_t row_bytes, void* dst_flat,
                       const int32_t* dst_row_offsets, vl_stream_t stream) {
  return copy_common<true>(src_padded, dst_flat, cu_seqlens, dst_row_offsets, num_reqs, row_bytes,
                           max_len, 0, (hipStream_t)stream);
}

int unpack_by_cu_seqlens(const void* src_flat, const int32_t* src_row_offsets,
                         const int32_t* cu_seqlens, int32_t num_reqs, int64_t row_bytes,
                         void* dst_padded, int64_t max_len, int zero_fill, vl_stream_t stream) {
  return copy_common<false>(src_flat, dst_padded, cu_seqlens, src_row_offsets, num_reqs, row_bytes,
                            max_len, zero_fill, (hipStream_t)stream);
}

}  // extern "C"
