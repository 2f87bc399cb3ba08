/*
 * varlen.h -- C ABI of the MI355X (gfx950) packed variable-length attention library.
 *
 * All tensor pointers are DEVICE pointers owned by the caller.  Every function
 * enqueues its work on `stream` and returns at once: no allocation, no
 * host<->device copy or synchronisation.  The library keeps no global mutable
 * state with two exceptions: a per-device cache of one occupancy query
 * (resident work-groups of the attention kernel, read once, mutex-guarded),
 * which sizes the key split of varlen_attn_fwd_split, and the static device
 * scratch array of varlen_attn_fwd_noalloc with its per-device address
 * (looked up once, mutex-guarded; see that function).  Device-
 * resident cu_seqlens are trusted preconditions (checking them would need a
 * device-to-host read); host scalars are validated and a bad one returns an
 * error code before anything is launched.  Return value: VL_OK (0) on success,
 * a negative vl_status otherwise.
 *
 * Layouts: packed tensors are [T, H, D] row-major (token, head, feature);
 * block-local tensors are [B, n, H, D]; lse tensors are [T, H] / [B, n, H]
 * float32, natural log.  Output buffers must not alias inputs.
 */
#ifndef VARLEN_MI355X_H
#define VARLEN_MI355X_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef struct ihipStream_t* vl_stream_t; /* a hipStream_t; NULL = default stream */

typedef enum {
  VL_OK = 0,
  VL_EINVAL = -1,       /* bad pointer, negative size, misaligned buffer, ... */
  VL_EUNSUPPORTED = -2, /* a size the kernels do not implement (e.g. head_dim not 64/128) */
  VL_ELAUNCH = -3       /* the kernel launch itself failed (hipGetLastError after launch) */
} vl_status;

/* Library version (major*10000 + minor*100 + patch) and a text for a status code. */
int vl_version(void);
const char* vl_status_string(int status);

/* ---------------------------------------------------------------- boundaries
 * cu_seqlens_from_lengths: cu_out[0] = 0, cu_out[r+1] = cu_out[r] + lengths[r].
 *   Flat varlen attention takes request boundaries as cumulative sequence
 *   lengths (vLLM-Omni PR #6711, "Key changes": q_cu_seqlens/kv_cu_seqlens).
 *   lengths: int32 [num_reqs] (device), cu_out: int32 [num_reqs+1] (device).
 *   0 <= num_reqs <= 65536; the sum must fit in int32 (trusted).
 *
 * joint_cu_seqlens: boundaries of a joint [text ; image] packed batch, built
 *   from the real text mask and the image grids (PR #6711 "Key changes":
 *   cu_seqlens from real text lengths via mask.sum; PR #4024 "How batching
 *   works": text lengths from the prompt mask, image grids from img_shapes).
 *   text_mask: uint8 [num_reqs, text_cap] (nonzero = real token);
 *   img_hw: int32 [num_reqs, 2] (grid h, w).  Outputs (device, int32):
 *   cu_joint [num_reqs+1], cu_text [num_reqs+1], cu_img [num_reqs+1] and
 *   img_dst [num_reqs] = cu_joint[r] + text_len[r] (first packed row of the
 *   request's image tokens; text precedes image inside a request).
 *   Any output pointer may be NULL to skip it.
 */
int cu_seqlens_from_lengths(const int32_t* lengths, int32_t num_reqs, int32_t* cu_out,
                            vl_stream_t stream);
int joint_cu_seqlens(const uint8_t* text_mask, int32_t text_cap, const int32_t* img_hw,
                     int32_t num_reqs, int32_t* cu_joint, int32_t* cu_text, int32_t* cu_img,
                     int32_t* img_dst, vl_stream_t stream);

/* ---------------------------------------------------------------- pack / unpack
 * pack_by_cu_seqlens: copy only the real rows of a padded per-request buffer
 *   into a flat one (PR #4024 "How batching works": only real tokens are
 *   packed; padding never enters the attention path).  Request r has
 *   len_r = cu_seqlens[r+1] - cu_seqlens[r] rows at src_padded + r*max_len rows;
 *   they go to dst_flat rows dst_row_offsets[r] + i (dst_row_offsets NULL =>
 *   cu_seqlens[r]).  A row is row_bytes bytes.  Rows of dst no request covers
 *   are left untouched.  len_r <= max_len is trusted.
 *
 * unpack_by_cu_seqlens: the inverse scatter (PR #6711 "Key changes": output
 *   unpacked by cu_seqlens; PR #4024 "Correctness model": outputs scattered back
 *   to request-local state): dst_padded[r*max_len + i] = src_flat[off_r + i] for
 *   i < len_r with off_r = src_row_offsets[r] (NULL => cu_seqlens[r]); rows
 *   i >= len_r are zeroed when zero_fill != 0, else untouched.
 *
 *   Both: row_bytes > 0; 0 <= num_reqs <= 65535; max_len >= 0.  Whole 16-byte
 *   vectors are used when row_bytes and both base pointers are 16-byte aligned,
 *   else 4-byte words (row_bytes and pointers 4-byte aligned), else bytes.
 */
int pack_by_cu_seqlens(const void* src_padded, int64_t max_len, const int32_t* cu_seqlens,
                       int32_t num_reqs, int64_t row_bytes, void* dst_flat,
                       const int32_t* dst_row_offsets, vl_stream_t stream);
int unpack_by_cu_seqlens(const void* src_flat, const int32_t* src_row_offsets,
                         const int32_t* cu_seqlens, int32_t num_reqs, int64_t row_bytes,
                         void* dst_padded, int64_t max_len, int zero_fill, vl_stream_t stream);

/* pack_by_cu_seqlens_batched / unpack_by_cu_seqlens_batched: up to 8 pack
 *   (or unpack) calls in one launch, e.g. the text and image pieces of Q, K
 *   and V of a joint batch.  descs: HOST array of `count` descriptors (read
 *   during the call only); descriptor i means exactly
 *     pack_by_cu_seqlens(src, max_len, cu_seqlens, num_reqs, row_bytes, dst,
 *                        row_offsets)
 *   resp. unpack_by_cu_seqlens(src, row_offsets, cu_seqlens, num_reqs,
 *                              row_bytes, dst, max_len, zero_fill)
 *   with the same argument rules (zero_fill is ignored by pack).  The copies
 *   run in no particular order, so no destination may overlap another copy's
 *   source or destination.  0 <= count <= 8, else VL_EINVAL.  When every copy
 *   moves 16-byte vectors it is one kernel launch, otherwise one per copy.
 */
typedef struct {
  const void* src;
  void* dst;
  const int32_t* cu_seqlens;
  const int32_t* row_offsets;
  int64_t max_len;
  int64_t row_bytes;
  int32_t num_reqs;
  int32_t zero_fill;
} vl_copy_desc;
int pack_by_cu_seqlens_batched(const vl_copy_desc* descs, int32_t count, vl_stream_t stream);
int unpack_by_cu_seqlens_batched(const vl_copy_desc* descs, int32_t count, vl_stream_t stream);

/* unpack_cfg_combine: per-request classifier-free-guidance combine fused into
 *   the unpack (vLLM-Omni PR #4024, "CFG behavior": the combine
 *   negative + true_cfg_scale * (positive - negative) is applied after the
 *   per-request split, and requests with different scales batch together).
 *   Request r has a positive and a negative segment of the same length
 *   len_r = seg_cu[r+1] - seg_cu[r] in the flat buffer, starting at rows
 *   pos_rows[r] and neg_rows[r]; for i < len_r
 *     dst[r*max_len + i] = bf16(neg + scale[r] * (pos - neg))
 *   computed in fp64 and rounded once to bf16 (nearest even), so scale 0 and 1
 *   return neg and pos bit for bit; rows i >= len_r are zeroed when
 *   zero_fill != 0.  src_flat, dst_padded:
 *   bf16 rows of row_elems elements (row_elems % 8 == 0, 16-byte aligned);
 *   seg_cu int32 [num_reqs+1], pos_rows / neg_rows int32 [num_reqs], scale
 *   float32 [num_reqs], all device; len_r <= max_len is trusted.
 */
int unpack_cfg_combine(const void* src_flat, const int32_t* seg_cu, const int32_t* pos_rows,
                       const int32_t* neg_rows, const float* scale, int32_t num_reqs,
                       int64_t row_elems, void* dst_padded, int64_t max_len, int zero_fill,
                       vl_stream_t stream);

/* ---------------------------------------------------------------- varlen attention
 * varlen_attn_fwd: flat non-causal attention over packed [T, H, D] bf16 Q/K/V
 *   (PR #6711 "Key changes" and "Reference / Acknowledgement"; PR #4024
 *   "Correctness model": no token attends across request boundaries).  For
 *   request r (rows q_cu[r]..q_cu[r+1] of q and kv_cu[r]..kv_cu[r+1] of k/v)
 *   and head h: out = softmax(scale * Q K^T) V, fp32 accumulation, output
 *   rounded to bf16 (nearest even); lse = natural-log sum of exp(scale*q.k)
 *   (fp32, may be NULL).  A request with q_len > 0 and kv_len = 0 gives out = 0
 *   and lse = -inf.  padded_tokens must be 0: every row of q/k/v belongs to a
 *   request (there is no argument for padding on purpose).
 *   q, k, v, out: bf16, 16-byte aligned; q_cu/kv_cu: int32 [num_reqs+1] with
 *   cu[0] = 0, non-decreasing (trusted).  max_q / max_kv: upper bounds of the
 *   per-request lengths, used only to size the launch.  D in {64, 128};
 *   H >= 1; num_reqs >= 0; scale finite and > 0 (else VL_EINVAL: the online
 *   softmax follows the maximum of the raw scores q.k, which is that of
 *   scale * q.k only for scale > 0).  The softmax weights are rounded to
 *   bf16 before the product with V, and the row sum behind the normalisation
 *   and lse is the sum of those rounded weights (so the output's weights sum
 *   to one; lse differs from the exact value by at most ln(1 + 2^-8)).
 * varlen_attn_fwd_f32: same contract on float32 q/k/v/out (weights and
 *   their sum stay fp32).
 */
int varlen_attn_fwd(const void* q, const void* k, const void* v, const int32_t* q_cu_seqlens,
                    const int32_t* kv_cu_seqlens, int32_t max_q, int32_t max_kv, int32_t num_reqs,
                    int32_t H, int32_t D, float scale, void* out, float* lse, vl_stream_t stream);
int varlen_attn_fwd_f32(const float* q, const float* k, const float* v,
                        const int32_t* q_cu_seqlens, const int32_t* kv_cu_seqlens, int32_t max_q,
                        int32_t max_kv, int32_t num_reqs, int32_t H, int32_t D, float scale,
                        float* out, float* lse, vl_stream_t stream);

/* varlen_attn_fwd_split: varlen_attn_fwd (same contract; results equal up to
 *   fp32 summation order and the order of the keys inside each MFMA step)
 *   with a caller-provided workspace that serves three purposes.
 *   1. V^T staging: a first kernel writes V transposed, per head D rows of
 *      vt_ld = roundup(kv_rows, 64) + 64 * num_reqs bf16 columns, request r's
 *      keys from column 64 * (ceil(kv_cu_seqlens[r] / 64) + r), each request
 *      padded with zeros to whole 64-key tiles; the attention kernel then
 *      reads its V operands with plain 16-byte LDS reads.  This reads V once
 *      and writes its copy once (HBM traffic of 2 x the V bytes).
 *   2. Key split of the last round: with `slots` work-groups resident at
 *      once on the device and T tiles of 256 query rows, tiles [0, full) run
 *      whole, full = T - T mod slots (0 if T < slots); when the remaining
 *      tail tiles would leave at least half of the slots idle, each is cut
 *      into parts = min(16, slots / tail, max_kv / 256) >= 2 key ranges of
 *      whole 64-key tiles, run as separate work-groups that write
 *      unnormalised partial results to the workspace; a last kernel on the
 *      same stream merges them (log-sum-exp weights) into out / lse.
 *   3. Chiplet work queues: the work items the static schedule below deals
 *      to each of the 8 chiplets form that chiplet's queue, in the same
 *      order; a work-group takes the next item of its own chiplet's queue
 *      (an atomic ticket on a counter in the workspace, zeroed by the V^T
 *      staging kernel) and, once that queue is empty, the next item of
 *      another queue, so chiplets that run at a higher clock take on more
 *      of the work.  The launch has an eighth more work-groups than the
 *      item bound for that; work-groups that find every queue empty exit.
 *      Which work-group runs an item does not change its result: out and
 *      lse are the same bits from call to call.
 *   kv_rows: rows of k and v (>= kv_cu_seqlens[num_reqs]; the Python binding
 *   passes k.shape[0]); it sizes the V^T rows.
 *   workspace: device, 16-byte aligned, at least the bytes
 *   varlen_split_workspace_bytes reports for (kv_rows, num_reqs, H, D): the
 *   partial results (slots * 256 * (4 * D + 8) bytes, rounded up to 256),
 *   V^T (H * D * vt_ld * 2 bytes, rounded up to 256), then 256 bytes of
 *   queue counters; its contents need no initialisation and are scratch
 *   after the call.  Two
 *   calls that share a workspace must be ordered (same stream, or
 *   synchronised).  A missing or short workspace returns VL_EINVAL; a V^T
 *   row of more than 2^31 bytes (D * vt_ld * 2) returns VL_EUNSUPPORTED.
 * varlen_split_workspace_bytes: host-only; the workspace size for these
 *   sizes on the current device (the partial-result part is 0 when no device
 *   can be queried).
 */
int varlen_attn_fwd_split(const void* q, const void* k, const void* v, const int32_t* q_cu_seqlens,
                          const int32_t* kv_cu_seqlens, int32_t max_q, int32_t max_kv, int32_t num_reqs,
                          int32_t H, int32_t D, float scale, void* out, float* lse, int64_t kv_rows,
                          void* workspace, int64_t workspace_bytes, vl_stream_t stream);
int varlen_split_workspace_bytes(int64_t kv_rows, int32_t num_reqs, int32_t H, int32_t D, int64_t* bytes);

/* pack_v_transposed + varlen_attn_fwd_vt: the pack of V and the V^T staging
 *   of varlen_attn_fwd_split in one pass (PR #4024 "How batching works":
 *   only real tokens are packed; PR #6711 "Key changes": K/V of all
 *   requests concatenated with kv_cu_seqlens as their boundaries), so V is
 *   read from its padded buffers and written once, straight in the layout
 *   the attention kernel reads.
 * pack_v_transposed: descs[i] (HOST array, read during the call) names piece
 *   i of V as pack_by_cu_seqlens would copy it: rows [0, len_r) of
 *   src + r * max_len rows (len_r = cu_seqlens[r+1] - cu_seqlens[r]) are
 *   the flat key rows row_offsets[r] (NULL => cu_seqlens[r]) onward; dst and
 *   zero_fill are ignored.  Every descriptor must have num_reqs requests and
 *   row_bytes = H * D * 2 (bf16 rows of H heads of D features) and a 16-byte
 *   aligned src; 1 <= count <= 8.  Instead of flat rows the call writes V^T
 *   into `workspace` (as varlen_attn_fwd_split stages it): request r's keys
 *   kv_cu_seqlens[r] .. kv_cu_seqlens[r+1]-1 take their rows from the piece
 *   that covers them (the first one, where pieces overlap), a key no piece
 *   covers reads as zero, and the columns past each request's last key up
 *   to its next multiple of 64 are zero.  kv_rows, num_reqs, H, D,
 *   workspace, workspace_bytes: as for varlen_attn_fwd_split; len_r <=
 *   max_len is trusted.
 * varlen_attn_fwd_vt: varlen_attn_fwd_split on q, k and the V^T that
 *   pack_v_transposed left in `workspace` (same kv_cu_seqlens, num_reqs, H,
 *   D and kv_rows); out and lse are the same bits as varlen_attn_fwd_split's
 *   on the V those pieces pack.  The V^T is only read, so the call may be
 *   repeated on one staging; it clears the queue counters itself.
 *   Both: the V^T starts after room for the partial results of every
 *   resident work-group (the size varlen_split_workspace_bytes reports),
 *   whatever max_kv is; a workspace shorter than that returns VL_EINVAL.
 */
int pack_v_transposed(const vl_copy_desc* descs, int32_t count, const int32_t* kv_cu_seqlens, int32_t num_reqs,
                      int32_t H, int32_t D, int64_t kv_rows, void* workspace, int64_t workspace_bytes,
                      vl_stream_t stream);
int varlen_attn_fwd_vt(const void* q, const void* k, const int32_t* q_cu_seqlens, const int32_t* kv_cu_seqlens,
                       int32_t max_q, int32_t max_kv, int32_t num_reqs, int32_t H, int32_t D, float scale, void* out,
                       float* lse, int64_t kv_rows, void* workspace, int64_t workspace_bytes, vl_stream_t stream);

/* varlen_attn_fwd_noalloc: for callers that cannot allocate device memory
 *   (code under HIP graph capture, tight serving loops, harnesses that forbid
 *   hipMalloc).  Same arguments and contract as varlen_attn_fwd; it runs the
 *   key split of the last round like varlen_attn_fwd_split, with the same
 *   split plan but the static schedule (no chiplet queues), and keeps the
 *   partial results in a static device array of
 *   VL_NOALLOC_SCRATCH_BYTES per GPU (held until the process ends) and reads V
 *   row-major (no V^T staging, whose buffer grows with the input); its out and
 *   lse are the same bits as varlen_attn_fwd_split's.  It calls no hipMalloc
 *   or hipFree.  The partials need slots * 256 * (4 * D + 8) bytes, slots =
 *   the attention kernel's resident work-groups on the device (256 on an
 *   MI355X: 34 MB at D = 128); a device needing more returns VL_EUNSUPPORTED.
 *   Every call on one GPU shares that GPU's array: calls that overlap on one
 *   GPU (two streams, two threads) race and must be ordered by the caller.
 *   The array needs no clearing: each call writes every partial it reads.
 */
#define VL_NOALLOC_SCRATCH_BYTES (48 * 1024 * 1024)
int varlen_attn_fwd_noalloc(const void* q, const void* k, const void* v, const int32_t* q_cu_seqlens,
                            const int32_t* kv_cu_seqlens, int32_t max_q, int32_t max_kv, int32_t num_reqs,
                            int32_t H, int32_t D, float scale, void* out, float* lse, vl_stream_t stream);

/* ---------------------------------------------------------------- block-local attention
 * block_local_attn_fwd: the block-local ("block-sparse") attention of the
 *   Token2Wav DiT (PR #7975, review of the window code, commit messages,
 *   "Purpose"/"Change"): frames are grouped in blocks of `block`; a query in
 *   block b attends to every frame j < n whose block lies in
 *   [b - look_back, b + look_ahead]; no dense n x n mask is formed and only
 *   the keys of that window are read.  q, k, v, out: bf16 [B, n, H, D];
 *   lse: fp32 [B, n, H] or NULL.  D in {64, 128}; B, n >= 0; H >= 1;
 *   block >= 1; look_back, look_ahead >= 0; scale finite and > 0.
 * block_local_attn_fwd_f32: same contract on float32 tensors.
 */
int block_local_attn_fwd(const void* q, const void* k, const void* v, int32_t B, int32_t n,
                         int32_t H, int32_t D, int32_t block, int32_t look_back,
                         int32_t look_ahead, float scale, void* out, float* lse,
                         vl_stream_t stream);
int block_local_attn_fwd_f32(const float* q, const float* k, const float* v, int32_t B,
                             int32_t n, int32_t H, int32_t D, int32_t block, int32_t look_back,
                             int32_t look_ahead, float scale, float* out, float* lse,
                             vl_stream_t stream);

/* ---------------------------------------------------------------- MixFusion layout check (host)
 * mixfusion_chunk_plan: whether a mixed-resolution batch may take the flat
 *   varlen layout (vLLM-Omni PR #6711, "How to enable MixFusion": the layout
 *   is rejected when the gcd of the token counts is below
 *   mixfusion_min_chunk_tokens, default 256, or when the resulting chunk count
 *   exceeds mixfusion_max_chunks, default 128).  chunk_size = gcd of the
 *   counts, chunk_count = sum / chunk_size.  Host-only, no GPU.
 *   token_counts: int64 [n] (host), n >= 1, every count >= 1.  Writes
 *   *chunk_size / *chunk_count (may be NULL); returns 1 if accepted, 0 if
 *   rejected, VL_EINVAL on bad arguments.
 */
int mixfusion_chunk_plan(const int64_t* token_counts, int32_t n, int64_t min_chunk_tokens,
                         int64_t max_chunks, int64_t* chunk_size, int64_t* chunk_count);

/* ---------------------------------------------------------------- schedule (test export)
 * The tile map serves the contract that no token attends across request
 * boundaries (PR #4024, "Correctness model"; PR #6711, "Key changes": one
 * flat pass over the packed batch): every work item lies inside one request
 * and one head, so the attention kernels never mix requests.
 * varlen_launch_shape: host-only; the launch varlen_attn_fwd (dtype_f32 = 0,
 *   split = 0), varlen_attn_fwd_split (dtype_f32 = 0, split = 1) or
 *   varlen_attn_fwd_f32 (dtype_f32 = 1) uses for these scalars: query rows
 *   per work-group (block_m), chiplet chunk, number of work-groups and the
 *   slot count of the key split (0 = no split possible).  The split = 1
 *   launch adds spare work-groups for its chiplet queues: an eighth of the
 *   item bound (R * H * ceil(max_q / block_m) + slots) before the rounding
 *   up to whole groups of 8 * chunk.  Any output pointer may be NULL.
 * varlen_tile_map: writes, for every launched work-group b of that launch,
 *   (request, head, q-tile, part, parts) into items_out[5*b .. 5*b+4]:
 *   part 0 of 1 for a whole tile, key range `part` of `parts` for a split
 *   one, all -1 for an idle work-group; it runs the same device code as the
 *   attention kernel.  For split = 1 it gives the static map; the items it
 *   assigns to one chiplet's work-groups, in work-group order, are that
 *   chiplet's queue (which work-group takes which entry then follows the
 *   order of their tickets).
 *   items_out: int32 [max_blocks, 5] (device); max_blocks must be >= the
 *   launch size, else VL_EINVAL.
 *   Schedule: requests by key length descending (ties: lower index first) when
 *   num_reqs <= 64, else in index order; heads ascending; q-tiles ascending.
 *   Work-group b runs on chiplet b mod 8 and takes logical item
 *   ((i div chunk)*8 + b mod 8)*chunk + (i mod chunk) with i = b div 8;
 *   logical items [0, full) are the tiles in that order, then item
 *   full + u is part u mod parts of tile full + u div parts.  Part p of a
 *   tile with nkt key tiles covers key tiles [p*nkt/parts, (p+1)*nkt/parts).
 */
int varlen_launch_shape(int32_t max_q, int32_t max_kv, int32_t num_reqs, int32_t H, int32_t D, int dtype_f32,
                        int split, int32_t* block_m, int32_t* chunk, int64_t* blocks, int32_t* slots);
int varlen_tile_map(const int32_t* q_cu_seqlens, const int32_t* kv_cu_seqlens, int32_t max_q, int32_t max_kv,
                    int32_t num_reqs, int32_t H, int32_t D, int dtype_f32, int split, int32_t* items_out,
                    int64_t max_blocks, vl_stream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* VARLEN_MI355X_H */
