/*
 * ffa.h - C ABI of libffa: Flex-Flash-Attention (FFA) on AMD Instinct MI355X (gfx950).
 *
 * FFA is fused attention forward and backward over a list of AttnSlices.  An
 * AttnSlice is (QRange, KRange, MaskType): a contiguous 2-D region of the
 * query x key plane plus the rule that applies inside it (MagiAttention blog
 * deep-dive, section "Flex-Flash-Attention 与 AttnSlice", AttnSlice equation
 * and the list of mask types after it).  A list of such slices expresses
 * varlen, block-causal, sliding-window and patch-and-pack masks in one call.
 *
 * Conventions used by every entry point
 * -------------------------------------
 *  - Slice table: device int32 array [num_slices][5] =
 *      { q_start, q_end, k_start, k_end, mask_type }, half-open token ranges
 *    into the q and k tensors.  For slice s, query i and key j with
 *    r = i - q_start, c = j - k_start, Lq = q_end - q_start, Lk = k_end - k_start,
 *    (i, j) is valid iff it lies in the rectangle and
 *      FFA_FULL:        always
 *      FFA_CAUSAL:      c <= r + (Lk - Lq)       (bottom-right aligned)
 *      FFA_INV_CAUSAL:  c >= r                   (top-left aligned)
 *      FFA_BI_CAUSAL:   both.
 *    Slices must have disjoint valid sets.  A query attends to the union of its
 *    valid keys; a query with none gets O = 0 and LSE = -inf.
 *  - Tensors are token-major ("THD"): q, o, dout, dq are [seqlen_q][num_heads_q][head_dim],
 *    k, v, dk, dv are [seqlen_k][num_heads_kv][head_dim], all bf16, with the
 *    last dimension contiguous and arbitrary token/head strides (in elements).
 *    The rows of an output (one per token and head) must not share elements:
 *    with its axes of more than one element ordered by stride, the inner
 *    stride is at least head_dim and the outer one at least the inner stride
 *    times the inner extent (views into one packed tensor qualify).  Outputs
 *    must not share elements with each other or with the inputs (accumulate
 *    mode reads and writes the same o and lse); the library checks the first
 *    rule, not the second.
 *    Query head h reads key/value head h / (num_heads_q / num_heads_kv).
 *  - lse is fp32 [num_heads_q][seqlen_q], natural log, including the softmax
 *    scale: lse_i = ln sum_{j valid} exp(scale * q_i . k_j).
 *  - Ownership: the caller allocates and frees every buffer.  The library
 *    allocates nothing, never synchronises, and only enqueues work on the
 *    given stream (a hipStream_t passed as void*; NULL is the default
 *    stream).  Its only global state is the per-device address of the static
 *    scratch array of ffa_bwd_static_scratch, looked up once per device.
 *  - Errors: problems visible on the host (null or misaligned pointers, bad
 *    shapes or strides, unsupported head_dim, a buffer that is too small) make
 *    the call return a non-zero ffa_status before anything is enqueued.  A
 *    failed launch returns FFA_ERR_HIP.  Problems in the device-resident slice
 *    table are found by ffa_build_block_meta on the device and recorded in the
 *    metadata's status word (FFA_META_ERR_* flags); ffa_fwd and ffa_bwd then
 *    write nothing.  The same holds when the metadata was built for other
 *    sequence lengths than the call's seqlen_q / seqlen_k (the kernels compare
 *    them with the metadata header on the device): outputs are left as they
 *    were, so a caller that cannot rule this out reads the status word (or
 *    pre-fills its outputs) before trusting them.  No function throws.
 */
#ifndef FFA_H_
#define FFA_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define FFA_ABI_VERSION 6

#if defined(__GNUC__)
#define FFA_API __attribute__((visibility("default")))
#else
#define FFA_API
#endif

typedef enum {
  FFA_FULL = 0,
  FFA_CAUSAL = 1,
  FFA_INV_CAUSAL = 2,
  FFA_BI_CAUSAL = 3
} ffa_mask_type;

typedef enum {
  FFA_OK = 0,
  FFA_ERR_INVALID_ARGUMENT = 1,    /* null/misaligned pointer, bad shape or stride */
  FFA_ERR_UNSUPPORTED = 2,         /* e.g. head_dim not 64 or 128 */
  FFA_ERR_WORKSPACE_TOO_SMALL = 3, /* meta_bytes or ws_bytes below the required size */
  FFA_ERR_HIP = 4,                 /* a kernel launch failed */
  FFA_ERR_BAD_SLICES = 5,          /* host slice table: range out of bounds or unknown type */
  FFA_ERR_TOO_LARGE = 6            /* the shape needs more scratch than the static array holds */
} ffa_status;

/* Flags of the device status word inside the block metadata. */
#define FFA_META_ERR_BOUNDS 1   /* a range outside [0, seqlen] or start > end */
#define FFA_META_ERR_TYPE 2     /* mask_type not in 0..3 */
#define FFA_META_ERR_OVERLAP 4  /* two slices share a valid (query, key) pair */
#define FFA_META_ERR_CAPACITY 8 /* meta buffer too small for this table's CSR lists */

typedef struct {
  const void* ptr;       /* device, 16-byte aligned */
  int64_t token_stride;  /* elements between consecutive tokens: multiple of 8,
                            >= head_dim and < 2^23 for every tensor with a token */
  int64_t head_stride;   /* elements between consecutive heads (multiple of 8) */
} ffa_tensor_in;

typedef struct {
  void* ptr;             /* device, 16-byte aligned; strides as for inputs,  */
  int64_t token_stride;  /* and its (token, head) rows must not overlap      */
  int64_t head_stride;   /* (FFA_ERR_INVALID_ARGUMENT otherwise)             */
} ffa_tensor_out;

typedef struct {
  int32_t seqlen_q;      /* >= 0 */
  int32_t seqlen_k;      /* >= 0 */
  int32_t num_heads_q;   /* >= 1, multiple of num_heads_kv */
  int32_t num_heads_kv;  /* >= 1 */
  int32_t head_dim;      /* 64 or 128 */
  float softmax_scale;   /* finite, > 0; 1/sqrt(head_dim) is the usual choice */
} ffa_shape;

/* Host-side summary of a block-metadata buffer (pure pointer arithmetic; no
 * device access).  Tile shapes are the kernels' own; they are what the CSR
 * lists are built for. */
typedef struct {
  int32_t bm_fwd, bn_fwd;            /* q2k tile: query rows x key cols */
  int32_t bm_bwd, bn_bwd;            /* k2q tile: query rows x key cols */
  int32_t num_qblocks_fwd, num_kblocks_fwd;
  int32_t num_qblocks_bwd, num_kblocks_bwd;
  int64_t header_bytes;              /* the header struct below sits at offset 0 */
  /* device pointers into the buffer */
  const int32_t* status;             /* FFA_META_ERR_* flags, 0 = good */
  const int64_t* area;               /* exact number of valid (query, key) pairs */
  const int32_t* full_block_offset;  /* q2k, [num_qblocks_fwd + 1] */
  const int32_t* mask_block_offset;  /* q2k, [num_qblocks_fwd + 1] */
  const int32_t* k2q_full_block_offset; /* k2q, [num_kblocks_bwd + 1] */
  const int32_t* k2q_mask_block_offset; /* k2q, [num_kblocks_bwd + 1] */
  const int32_t* qblock_slice_offset;   /* [num_qblocks_fwd + 1] */
  const int32_t* schedule_fwd;       /* [num_qblocks_fwd], q-blocks by descending work */
  const int32_t* schedule_bwd;       /* [num_kblocks_bwd], k-blocks by descending work */
  const int32_t* index_base;         /* variable region; see list_offsets */
  const int64_t* list_offsets;       /* device int64[5]: entry offsets from index_base of
                                        full_block_idx, mask_block_idx, k2q_full_block_idx,
                                        k2q_mask_block_idx, qblock_slice_idx */
  /* block records, 16 int32 each, in schedule order (the kernels' first read):
   * fwd: q-block, q2k Full offset, Full count, Partial offset, Partial count,
   *      slice-list offset, slice count, first Full tile, first Partial tile;
   * bwd: k-block, k2q Full offset, Full count, Partial offset, Partial count,
   *      last Full tile, last Partial tile; -1 for a tile of an empty list,
   *      the rest of the 16 unspecified */
  const int32_t* block_records_fwd;  /* [num_qblocks_fwd][16] */
  const int32_t* block_records_bwd;  /* [num_kblocks_bwd][16] */
} ffa_block_meta_view_t;

/* Upper bound on the metadata buffer size for a table of num_slices slices.
 * host_slices (nullable) is a host copy of the table: when given, the bound
 * is tightened from each slice's bounding rectangle, otherwise it assumes
 * every tile may be non-empty.  Block classes and CSR lists follow the
 * create_block_mask / CSR description of the MagiAttention documentation
 * page, "FFA_FA4" optimisations, items 1 and 2. */
FFA_API ffa_status ffa_block_meta_workspace_size(int32_t num_slices, int32_t seqlen_q,
                                                 int32_t seqlen_k, int32_t head_dim,
                                                 const int32_t* host_slices, size_t* bytes);

/* Build the block metadata of a slice table, asynchronously on `stream`.
 * d_slices: device int32 [num_slices][5] (read only; copied into d_meta).
 * d_meta: device buffer of meta_bytes bytes, 256-byte aligned, owned by the caller.
 * For each (query block, key block) tile the valid count v is computed exactly
 * and the tile is classed Empty (v = 0), Full or Partial.  q2k (forward):
 * query rows past seqlen_q are ignored and key columns past seqlen_k count as
 * invalid, so a block out of bounds only in q can be Full.  k2q (backward):
 * the mirror, key columns past seqlen_k ignored, query rows past seqlen_q
 * invalid.  Per block the Full and Partial lists are kept apart, ascending
 * (full_block_offset / mask_block_offset and the k2q mirrors).  The table is
 * validated on the device (bounds, type, disjointness) into the status word;
 * disjointness is tested for the slice pairs that share a 128-row query
 * block, in time proportional to the sum over query blocks of the square of
 * the slices meeting the block (linear in the table when each row meets a
 * bounded number of slices), and only when the lists fit the buffer
 * (otherwise FFA_META_ERR_CAPACITY is set and the table is not checked for
 * overlap).
 * The buffer can be reused by any number of ffa_fwd / ffa_bwd calls with the
 * same seqlens and head_dim until it is rebuilt. */
FFA_API ffa_status ffa_build_block_meta(const int32_t* d_slices, int32_t num_slices,
                                        int32_t seqlen_q, int32_t seqlen_k, int32_t head_dim,
                                        void* d_meta, size_t meta_bytes, void* stream);

/* Fill *out from the layout of a metadata buffer built with these arguments:
 * host pointer arithmetic only, no device access.  The fields are the block
 * classes and CSR lists of the MagiAttention documentation page ("FFA_FA4"
 * optimisations, item 1: Full / Partial / Empty tiles from create_block_mask,
 * a tile out of bounds only in q counted as Full; item 2: full_block_offset /
 * mask_block_offset CSR lists).  d_meta is not read; out receives device
 * pointers into it.  Bad sizes give FFA_ERR_INVALID_ARGUMENT, a head_dim other
 * than 64 or 128 FFA_ERR_UNSUPPORTED. */
FFA_API ffa_status ffa_block_meta_view(const void* d_meta, int32_t num_slices, int32_t seqlen_q,
                                       int32_t seqlen_k, int32_t head_dim,
                                       ffa_block_meta_view_t* out);

/* Forward: o = softmax(scale * q k^T restricted to the valid set) v and lse,
 * the FFA forward kernel of the MagiAttention blog deep-dive (section
 * "Flex-Flash-Attention 与 AttnSlice": the AttnSlice equation defines the valid
 * set as the union of the slices' masks, Fig. 5 the per-slice data loading and
 * on-chip compute), computed with an online softmax over the q2k Full and
 * Partial tiles of each query block, per-element masking only on Partial tiles
 * (documentation page, "FFA_FA4" items 1 and 2).
 * q: [seqlen_q][num_heads_q][head_dim] bf16; k, v: [seqlen_k][num_heads_kv][head_dim]
 * bf16 (read only).  d_meta: built by ffa_build_block_meta for this seqlen_q,
 * seqlen_k (read only).  o: bf16 like q, written.  lse: device fp32
 * [num_heads_q][seqlen_q], 16-byte aligned, written.  Rows with no valid key
 * get o = 0, lse = -inf.  Errors as in the conventions above. */
FFA_API ffa_status ffa_fwd(const ffa_shape* shape, ffa_tensor_in q, ffa_tensor_in k,
                           ffa_tensor_in v, const void* d_meta, ffa_tensor_out o, float* lse,
                           void* stream);

/* Scratch bytes ffa_bwd needs for the backward of the FFA kernel (MagiAttention
 * blog deep-dive, section "Flex-Flash-Attention 与 AttnSlice", Fig. 5: the
 * backward merges partial results; here the only partials are those of split
 * key blocks, see ffa_bwd).  Layout, each region starting at a 256-byte
 * boundary of d_ws:
 *   -D_i = -(dO_i . O_i)      fp32 [num_heads_q][seqlen_q]
 *   LSE_i * log2(e)           fp32 [num_heads_q][seqlen_q]
 *   -LSE_i / softmax_scale    fp32 [num_heads_q][seqlen_q]
 *   split finish counters     int32 [E][num_heads_kv]
 *   split partial dK, dV      fp32 [E][num_heads_kv][2 halves][dK, dV][128 * head_dim]
 * with E = min(ceil(seqlen_k / 128), min(32, max(4, 128 / num_heads_kv))) key
 * blocks of 128 keys per kv head (the longest ones).  Depends on the shape only.
 * Bad shapes give FFA_ERR_INVALID_ARGUMENT / FFA_ERR_UNSUPPORTED; null bytes
 * FFA_ERR_INVALID_ARGUMENT. */
FFA_API ffa_status ffa_bwd_workspace_size(const ffa_shape* shape, size_t* bytes);

/* Backward: dq, dk, dv of the forward above, given its o and lse: the textbook
 * gradient of the FFA forward (MagiAttention blog deep-dive, section
 * "Flex-Flash-Attention 与 AttnSlice", Fig. 5: FFA forward and backward
 * kernels over the slices; documentation page, "FFA_FA4" items 1 and 2 for
 * the k2q / q2k tile lists it walks).  q, k, v, o, dout as for ffa_fwd (dout
 * like o); lse as written by ffa_fwd (read only); dq like q, dk and dv like k,
 * all bf16 and written.
 * dk and dv are accumulated per key block in a fixed order over the k2q tiles
 * and the query heads that share the key head, and dq per query block over
 * its q2k tiles.  A key block whose work exceeds an even share of the
 * device's resident workgroups is done as two halves of that order whose fp32
 * sums are added once (a commutative step), so results are bitwise
 * reproducible on a given device; the split choice depends on the number of
 * compute units.  Calls that share one workspace must not run concurrently,
 * except the DQ-only and DKDV-only calls of ffa_bwd_phases after PRE (they
 * only read the row statistics, and only DKDV uses the split counters).
 * d_ws: device scratch of at least ffa_bwd_workspace_size bytes, 256-byte aligned. */
FFA_API ffa_status ffa_bwd(const ffa_shape* shape, ffa_tensor_in q, ffa_tensor_in k,
                           ffa_tensor_in v, ffa_tensor_in o, const float* lse,
                           ffa_tensor_in dout, const void* d_meta, ffa_tensor_out dq,
                           ffa_tensor_out dk, ffa_tensor_out dv, void* d_ws, size_t ws_bytes,
                           void* stream);

/* Phases of the backward, for ffa_bwd_phases. */
#define FFA_BWD_PRE 1   /* -D_i = -dO_i . O_i and LSE_i log2(e) into d_ws        */
#define FFA_BWD_DKDV 2  /* dk, dv (reads D from d_ws)                             */
#define FFA_BWD_DQ 4    /* dq (reads D from d_ws)                                 */
#define FFA_BWD_ALL 7

/* ffa_bwd restricted to a subset of its phases (bitwise OR of FFA_BWD_*), the
 * same backward of the FFA kernel (blog deep-dive, "Flex-Flash-Attention 与
 * AttnSlice", Fig. 5) split where its kernels meet; arguments as for ffa_bwd.
 * DKDV and DQ read the values that PRE wrote into the same d_ws; once PRE has
 * finished they are independent of each other, so a caller may run them on
 * two streams.  When PRE and DQ are requested together, the dQ kernel
 * computes the PRE values itself, stores them in d_ws, and runs first, then
 * DKDV; otherwise the order is PRE, DKDV, DQ.  phases = FFA_BWD_ALL is
 * ffa_bwd.  Unknown bits give FFA_ERR_INVALID_ARGUMENT. */
FFA_API ffa_status ffa_bwd_phases(const ffa_shape* shape, ffa_tensor_in q, ffa_tensor_in k,
                                  ffa_tensor_in v, ffa_tensor_in o, const float* lse,
                                  ffa_tensor_in dout, const void* d_meta, ffa_tensor_out dq,
                                  ffa_tensor_out dk, ffa_tensor_out dv, void* d_ws,
                                  size_t ws_bytes, int32_t phases, void* stream);

/* Flags of ffa_fwd_ex and ffa_bwd_ex. */
#define FFA_ACCUMULATE 1u  /* merge into / add to the results already in the output buffers */

/* ffa_fwd with flags; flags = 0 is ffa_fwd.  FFA_ACCUMULATE is the partial-result merge that
 * lets one attention be computed in several calls whose valid (query, key) sets are
 * disjoint, e.g. one call per stage of key / value ranges arriving from other GPUs
 * (MagiAttention blog deep-dive, section "通信与重叠", Fig. 13: the forward runs stage by
 * stage; section "Flex-Flash-Attention 与 AttnSlice", Fig. 5: partial results are merged).
 * o and lse must then hold a previous result (O_1, LSE_1) of the same queries, LSE_1 = -inf
 * for rows that had no valid key (their O_1 is not read).  This call's result (O_2, LSE_2)
 * is merged into them row by row with the log-sum-exp identity
 *   LSE = ln(e^LSE_1 + e^LSE_2),  O = e^(LSE_1 - LSE) O_1 + e^(LSE_2 - LSE) O_2
 * (fp32, O rounded to bf16 once per call); rows with no valid key in this call keep their
 * stored O and LSE.  Unknown flag bits give FFA_ERR_INVALID_ARGUMENT. */
FFA_API ffa_status ffa_fwd_ex(const ffa_shape* shape, ffa_tensor_in q, ffa_tensor_in k,
                              ffa_tensor_in v, const void* d_meta, ffa_tensor_out o, float* lse,
                              uint32_t flags, void* stream);

/* ffa_bwd_phases with flags; flags = 0 is ffa_bwd_phases.  With FFA_ACCUMULATE the DQ phase
 * adds its result to what dq holds and the DKDV phase to what dk and dv hold (fp32 sum,
 * rounded to bf16 once per call), the backward counterpart of the merge above (blog
 * deep-dive, section "通信与重叠", Fig. 13: partial dKV reduced stage by stage).  When an
 * attention is split into calls with disjoint valid sets, passing every call the merged o and
 * lse of the whole forward makes each call produce exactly its share of dQ, dK and dV, so the
 * accumulated buffers hold the gradients of the whole.  Unknown flag bits give
 * FFA_ERR_INVALID_ARGUMENT. */
FFA_API ffa_status ffa_bwd_ex(const ffa_shape* shape, ffa_tensor_in q, ffa_tensor_in k,
                              ffa_tensor_in v, ffa_tensor_in o, const float* lse,
                              ffa_tensor_in dout, const void* d_meta, ffa_tensor_out dq,
                              ffa_tensor_out dk, ffa_tensor_out dv, void* d_ws, size_t ws_bytes,
                              int32_t phases, uint32_t flags, void* stream);

/* ---------------------------------------------------------------------------
 * Several masks in one launch.
 *
 * The kv heads are cut into num_groups consecutive ranges, group g being kv
 * heads [kv_head_end[g-1], kv_head_end[g]) (kv_head_end[-1] = 0), together with
 * the query heads that read them; each group has its own slice table, i.e. its
 * own metadata buffer d_metas[g], all built for the shape's seqlen_q, seqlen_k
 * and head_dim.  One launch covers every group, so a model whose head groups
 * use different masks (or a layer that reuses the metadata of several masks)
 * needs one call instead of one per mask, and no group waits for another's
 * tail (MagiAttention docs, magi_attn_flex_key / make_flex_key_for_new_mask_after_dispatch:
 * metadata built once per mask and reused).  Results per head are those of a
 * single-mask call with that group's metadata, except that the dK/dV load
 * balancing (see ffa_bwd) weighs every group's work.
 * num_groups in 1..FFA_MAX_MASK_GROUPS; kv_head_end: host int32 [num_groups],
 * strictly increasing, last = num_heads_kv; d_metas: host array of
 * num_groups device pointers (256-byte aligned).  Bad groups give
 * FFA_ERR_INVALID_ARGUMENT.
 * ------------------------------------------------------------------------- */
#define FFA_MAX_MASK_GROUPS 8

FFA_API ffa_status ffa_fwd_grouped(const ffa_shape* shape, ffa_tensor_in q, ffa_tensor_in k,
                                   ffa_tensor_in v, int32_t num_groups, const void* const* d_metas,
                                   const int32_t* kv_head_end, ffa_tensor_out o, float* lse,
                                   uint32_t flags, void* stream);

FFA_API ffa_status ffa_bwd_grouped(const ffa_shape* shape, ffa_tensor_in q, ffa_tensor_in k,
                                   ffa_tensor_in v, ffa_tensor_in o, const float* lse,
                                   ffa_tensor_in dout, int32_t num_groups, const void* const* d_metas,
                                   const int32_t* kv_head_end, ffa_tensor_out dq, ffa_tensor_out dk,
                                   ffa_tensor_out dv, void* d_ws, size_t ws_bytes, int32_t phases,
                                   uint32_t flags, void* stream);

/* ---------------------------------------------------------------------------
 * Context-parallel dispatch (host only: no device memory, no stream).
 *
 * The query sequence is cut into n = ceil(seqlen_q / chunk_size) chunks; chunk c
 * holds queries [c * chunk_size, min((c + 1) * chunk_size, seqlen_q)) and its
 * area is the number of valid (query, key) pairs of those queries.  A dispatch
 * puts the chunks into cp_size buckets (ranks) holding the same number of
 * chunks each, aiming at the smallest largest bucket area, so that attention
 * work is balanced while token-priced layers stay balanced too (MagiAttention
 * blog deep-dive, section "Dispatch Solver": the chunk-count equation, the
 * min-max objective with the equal-count constraint, and the greedy min-heap
 * solution).
 * ------------------------------------------------------------------------- */

/* Area of every chunk.  host_slices: host int32 [num_slices][5], the table as
 * for ffa_build_block_meta (bounds and types are checked here, disjointness is
 * not: overlapping slices are counted once per slice).  areas: host int64
 * [ceil(seqlen_q / chunk_size)].  chunk_size > 0.  A bad table gives
 * FFA_ERR_BAD_SLICES and writes nothing. */
FFA_API ffa_status ffa_chunk_areas(const int32_t* host_slices, int32_t num_slices,
                                   int32_t seqlen_q, int32_t seqlen_k, int32_t chunk_size,
                                   int64_t* areas);

/* Greedy dispatch: the chunks, by decreasing area (equal areas: lower chunk
 * index first), each go to the bucket with the least area so far among those
 * still holding fewer than num_chunks / cp_size chunks (equal areas: lower
 * bucket index).  bucket: host int32 [num_chunks], the bucket of each chunk.
 * num_chunks must be a positive multiple of cp_size and areas >= 0.
 * O(n log n) with a min-heap of buckets. */
FFA_API ffa_status ffa_dispatch_chunks(const int64_t* areas, int32_t num_chunks,
                                       int32_t cp_size, int32_t* bucket);

/* The slice table of one rank's share.  chunks: host int32 [num_chunks],
 * distinct chunk indices; the rank's local queries are these chunks
 * concatenated in the given order.  Outputs (host int32):
 *   local_slices [*][5]: slices over local query rows and receive-buffer key
 *     columns with exactly the valid pairs of the global table on those
 *     queries.  A slice cut to a sub-range [a, b) of its queries keeps its rule
 *     by moving its key range: the end moves back by q_end - b for CAUSAL and
 *     BI-CAUSAL, the start forward by a - q_start for INV-CAUSAL and
 *     BI-CAUSAL; pieces without a valid pair are dropped.  Order: by position
 *     of the chunk in `chunks`, then by slice index.
 *   kv_ranges [*][3] = { global_start, global_end, buffer_start }: the sorted,
 *     disjoint (and non-adjacent) global key ranges the local slices touch,
 *     packed back to back in a receive buffer; the local seqlen_k is the end of
 *     the last one.  These are the keys (and values) the rank has to fetch.
 * max_local / max_kv are the capacities (in rows); num_local / num_kv receive
 * the counts.  A short capacity gives FFA_ERR_WORKSPACE_TOO_SMALL with the
 * needed counts written and the arrays untouched; a bad table
 * FFA_ERR_BAD_SLICES; a chunk index out of range or repeated
 * FFA_ERR_INVALID_ARGUMENT. */
FFA_API ffa_status ffa_rank_slices(const int32_t* host_slices, int32_t num_slices,
                                   int32_t seqlen_q, int32_t seqlen_k, int32_t chunk_size,
                                   const int32_t* chunks, int32_t num_chunks,
                                   int32_t* local_slices, int32_t max_local, int32_t* num_local,
                                   int32_t* kv_ranges, int32_t max_kv, int32_t* num_kv);

/* ---------------------------------------------------------------------------
 * Backward without a workspace argument.
 *
 * For callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid allocation): ffa_bwd
 * with its scratch (the -D / LSE rows, split counters and split partials of
 * ffa_bwd_workspace_size) in a static device array of the library,
 * FFA_STATIC_SCRATCH_BYTES per GPU, which every GPU the library runs on holds
 * until the process ends.  The array's address on the current device is
 * looked up on the first call there.  Results are those of ffa_bwd (same
 * kernels, bitwise).  A shape whose ffa_bwd_workspace_size exceeds
 * FFA_STATIC_SCRATCH_BYTES gives FFA_ERR_TOO_LARGE before anything is
 * enqueued.  Every call on one GPU uses that GPU's one array: calls that may
 * overlap on one GPU (other streams, other host threads) race and must be
 * serialised by the caller.  No device memory is allocated or freed.
 * ------------------------------------------------------------------------- */
#define FFA_STATIC_SCRATCH_BYTES (64u << 20)

FFA_API ffa_status ffa_bwd_static_scratch(const ffa_shape* shape, ffa_tensor_in q,
                                          ffa_tensor_in k, ffa_tensor_in v, ffa_tensor_in o,
                                          const float* lse, ffa_tensor_in dout, const void* d_meta,
                                          ffa_tensor_out dq, ffa_tensor_out dk, ffa_tensor_out dv,
                                          void* stream);

/* Static description of a status code. */
FFA_API const char* ffa_status_string(ffa_status status);

/* FFA_ABI_VERSION of the built library. */
FFA_API int32_t ffa_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* FFA_H_ */
