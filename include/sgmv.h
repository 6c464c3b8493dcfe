/*
 * libsgmv — multi-LoRA segmented gather GEMV (SGMV) delta on AMD Instinct MI355X (gfx950).
 *
 * The library adds, for every token t that carries an adapter id l = ids[t] >= 0,
 *
 *     y[t, :] += (alpha_l / r_l) * B[l, :, :r_l] @ (A[l, :r_l, :] @ x[t, :])
 *
 * to a base output y, for a whole batch in which tokens use different adapters stored in
 * one contiguous pool. Sources (page title and section):
 *   - Fused-LoRA page "09. Triton Fused LoRA" (llm-algo-leetcode), Steps 1-3: pool of all
 *     adapters as A (L, r, in) and B (L, out, r); each token routed by its own index.
 *   - Punica page "III. Punica: Multi-Tenant LoRA Serving", SGMV section (the batched delta
 *     next to the base product), batching-effect section (segment boundary array s), code
 *     section (tokens reordered by adapter, optional fixed-size chunks, weight index per
 *     segment, rows resolved through sorted token ids).
 *   - vLLM-Ascend LoRA operator article, sections 1.1 (delta (alpha/r)(x A^T) B^T), 2.1
 *     (per-adapter rank and alpha), 3.2 (two-stage projection: shrink then expand), 3.3
 *     (decode SGMV with compact per-segment descriptors), 3.4 (prefill grouped GEMM),
 *     4.1 (row-count threshold between vector and matrix units), 4.2 (adapter-major,
 *     rank-second pool with K/N aligned to 16 or 32), 4.3 (keep the M x r intermediate on
 *     chip), 5.3 (skip rows without adapter).
 *
 * Conventions for every call:
 *   - M = 0 is a no-op that returns SGMV_OK; data pointers may then be NULL.
 *   - Pointers are device memory owned by the caller unless a parameter says "host".
 *   - Calls that take a stream are asynchronous and ordered on that stream (a hipStream_t
 *     passed as void*; NULL is the default stream). The library allocates nothing on these
 *     paths and keeps no mutable global state; calls on different streams that write
 *     different outputs may run concurrently.
 *   - Argument errors are reported synchronously by the return value before anything is
 *     launched; SGMV_EHIP reports a failed HIP launch or copy.
 *   - dtype: x, y, A and B share one element type (fp32 or bf16). Accumulation is fp32.
 *     bf16 results are rounded once, to nearest even, when y is stored.
 */
#ifndef SGMV_H
#define SGMV_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  SGMV_OK = 0,
  SGMV_EINVAL = 1,        /* null pointer, negative size, inconsistent descriptor        */
  SGMV_EBADID = 2,        /* an adapter id outside {-1} U [0, L)                          */
  SGMV_EUNSUPPORTED = 3,  /* valid request outside the kernels' limits (see each call)    */
  SGMV_ECAPACITY = 4,     /* a caller-provided array is smaller than the stated bound     */
  SGMV_EHIP = 5           /* a HIP runtime call failed                                    */
} sgmv_status;

typedef enum { SGMV_F32 = 0, SGMV_BF16 = 1 } sgmv_dtype;

/* Rows per work descriptor, and the row count at or below which a descriptor is "small"
 * (decode-like) rather than "large" (prefill-like); Ascend article 3.3 and 4.1. */
#define SGMV_TILE_ROWS 64
#define SGMV_SMALL_ROWS 16
/* int32 entries per work descriptor record (one 128-byte line). */
#define SGMV_TILE_INTS 32
/* Largest adapter rank the kernels take (Ascend article 2.1: a maximum LoRA rank). */
#define SGMV_MAX_RANK 64
/* Largest pool the on-device segment builder takes (its tables live in LDS). */
#define SGMV_DEVICE_BUILDER_MAX_L 1024
/* Most output slices one call writes (e.g. 3 for a fused q/k/v projection). */
#define SGMV_MAX_SLICES 4
/* Largest batch for which sgmv_lora_delta_ids builds the segments inside the delta launch. */
#define SGMV_FUSED_BUILD_MAX_M 512
/* Largest batch on which fused bf16 calls run every large piece as parts of SGMV_SMALL_ROWS
 * rows (part j: rows 16j .. 16j + 15 of the piece), each with the small pieces' column
 * split, so that batches of a few adapters spread over as many workgroups as batches of
 * many. The descriptor records are the same either way. */
#define SGMV_PART_SPLIT_MAX_M 1024

/* ------------------------------------------------------------------------------------ *
 * Adapter pool (Fused-LoRA page Step 1; Ascend article 2.1 and 4.2).
 *
 * Library layout, all device memory, elements of `dtype`:
 *   a     [L][R_pad][K_pad]        A[l][j][k]
 *   b     [L][R_pad/8][N_pad][8]   B[l][n][j] at ((l*(R_pad/8) + j/8)*N_pad + n)*8 + j%8
 *   rank  [L] int32                r_l in [1, R_max]
 *   scale [L] fp32                 alpha_l / r_l
 * Adapter-major, rank second; K and N innermost and padded to multiples of 32; R_pad is R_max
 * rounded up to 16. B is stored in rank octets so that one 16-byte load holds 8 ranks of one
 * output column. The first r_l ranks of an adapter are a contiguous prefix of both blocks.
 * Padding is zero-filled by sgmv_pool_pack; kernels never read ranks at or past r_l.
 * ------------------------------------------------------------------------------------ */
typedef struct {
  void* a;
  void* b;
  int32_t* rank;
  float* scale;
  int32_t L, R_max, R_pad, K, N, K_pad, N_pad;
  int32_t dtype;    /* sgmv_dtype */
  int32_t rank_min; /* smallest r_l, set by sgmv_pool_pack (0 before): when it equals R_pad,
                       no adapter has padding and loads may start before r_l is read */
  int32_t scale_folded; /* 1 if sgmv_pool_pack_ex folded scale_l into b (scale is then 1) */
} sgmv_pool;

/* Fill the dimensions of `pool` for L adapters of rank at most R_max, K inputs and N
 * outputs, and report the byte sizes the caller must allocate for pool->a and pool->b
 * (pool->rank and pool->scale take 4*L bytes each). Pointers in `pool` are cleared.
 * Errors: EINVAL (null pool/outputs, L < 1, R_max < 1, K < 1, N < 1, bad dtype);
 * EUNSUPPORTED (R_max > SGMV_MAX_RANK). */
sgmv_status sgmv_pool_init(int32_t L, int32_t R_max, int32_t K, int32_t N, int32_t dtype,
                           sgmv_pool* pool, size_t* a_bytes, size_t* b_bytes);

/* Pack user-layout adapters into the pool (load time, not on the hot path).
 *   a_user   device, [L][R_max][K] contiguous, pool dtype   (Fused-LoRA page: A (L, r, in))
 *   b_user   device, [L][N][R_max] contiguous, pool dtype   (Fused-LoRA page: B (L, out, r))
 *   rank     host, [L] int32, each in [1, R_max]
 *   alpha    host, [L] fp32; scale_l = alpha_l / rank_l     (Ascend article 2.1, 3.2)
 * Entries of a_user/b_user at ranks >= rank[l] are ignored. pool->a, b, rank, scale must
 * point to allocations of the sizes sgmv_pool_init reported. Sets pool->rank_min.
 * Errors: EINVAL (null pointers, rank out of range, non-finite alpha); EHIP. */
sgmv_status sgmv_pool_pack(const void* a_user, const void* b_user, const int32_t* rank,
                           const float* alpha, sgmv_pool* pool, void* stream);

/* As sgmv_pool_pack, with flags (0 = sgmv_pool_pack):
 *   SGMV_PACK_FOLD_SCALE  fold the scale into B at load time (Ascend article 2.1, 3.2: the
 *     alpha/r factor may sit on either side of the expand, or be folded into B once when the
 *     weights are loaded). Each stored B[l][n][j], j < r_l, becomes scale_l * B[l][n][j],
 *     the product formed in fp32 (scale_l the fp32 quotient alpha_l / r_l) and rounded once
 *     to the pool dtype (bf16: to nearest, ties to even); scale[l] is set to 1 and
 *     pool->scale_folded to 1. For power-of-two scales (and no overflow or underflow) every
 *     delta is bit-identical to the unfolded pool's; otherwise it differs by B's rounding.
 * Errors: as sgmv_pool_pack, plus EINVAL for unknown flags. */
#define SGMV_PACK_FOLD_SCALE 1
sgmv_status sgmv_pool_pack_ex(const void* a_user, const void* b_user, const int32_t* rank,
                              const float* alpha, int32_t flags, sgmv_pool* pool, void* stream);

/* ------------------------------------------------------------------------------------ *
 * Segments (Punica page, batching-effect and code sections; Ascend article 3.3, 4.2).
 *
 * Tokens are grouped by adapter: buckets in the order in which adapters first appear among
 * the tokens, tokens ascending inside a bucket; tokens with id -1 carry no adapter, belong
 * to no segment and are placed last in sorted_token_ids (ascending). With chunk_size C > 0
 * every bucket is cut into ceil(c/C) segments of C rows (the last one shorter); chunks never
 * cross buckets. For the worked example of the Punica page, ids 2,2,2,5,5,1,1 give
 * sorted_token_ids 0..6, seg_indptr [0,3,5,7], seg_lora_ids [2,5,1].
 *
 * Work descriptors ("tiles"): every segment is cut, from its first sorted row, into pieces
 * of SGMV_TILE_ROWS rows, the last one shorter; records follow segment order within each
 * class. A piece of at most SGMV_SMALL_ROWS rows is small, otherwise large.
 * Each descriptor is a record of SGMV_TILE_INTS int32 at tiles + i * SGMV_TILE_INTS:
 *   [0] adapter, [1] first row in sorted order, [2] rows, [3] segment, [4..15] 0,
 *   [16..31] for a small piece its token ids (sorted_token_ids[first .. first + rows)), then
 *            -1; for a large piece all -1.
 * Large pieces occupy records [0, large_cap), small ones [large_cap, large_cap + small_cap).
 * info[4] = {num_segments, num_large_tiles, num_small_tiles, status}.
 *
 * Capacities: seg_cap = min(M, L) without chunking, min(M, min(M, L) + M / C) with;
 * large_cap = M / (SGMV_SMALL_ROWS + 1); small_cap = seg_cap.
 * Array sizes: sorted_token_ids [M], seg_indptr [seg_cap + 1], seg_lora_ids [seg_cap],
 * tiles [(large_cap + small_cap) * SGMV_TILE_INTS] (16-byte aligned), info [4].
 *
 * exchange (optional, may be NULL): device workspace of exchange_bytes for the fused call.
 * With it, a piece whose output columns are split over P workgroups (2 <= P <=
 * SGMV_EXCHANGE_MAX_SPLITS for small pieces, <= SGMV_EXCHANGE_MAX_SPLITS_LARGE for large
 * ones) also splits its shrink over K among them: each workgroup sums its K range, publishes
 * that fp32 partial rows x r tile here, and adds all P partials in split order, so A and x
 * are read once per piece instead of once per workgroup (Ascend article 3.3: weight traffic
 * of the decode kernel; the full intermediate still never leaves the chip, only K-range
 * partial sums pass through this buffer). Results do not depend on timing: a workgroup that
 * waits too long for its partners computes their partials itself, bit-identically.
 * Layout: [large_cap + small_cap][16] int32 control words indexed like the descriptor records
 * (word 0: the piece's arrival counter, which every call advances by exactly 64; when large
 * pieces run as parts, word j of a large record is part j's counter; the rest reserved),
 * padded to 256 bytes; then [small_cap][SGMV_EXCHANGE_MAX_SPLITS][16][64] fp32
 * small-piece partials; then [large_cap][SGMV_EXCHANGE_MAX_SPLITS_LARGE][64][64] fp32
 * large-piece partials (a part j of a large piece keeps its split q partial, 16 rows of ncol
 * floats, at q * 64 * ncol + j * 16 * ncol floats into the piece's slots; ncol is 32 for
 * adapter ranks up to 32, else 64). Zero-fill it when it is allocated; the device builder clears the
 * control words on every build. Fused calls that share one segments object with an exchange
 * workspace must be ordered on one stream.
 * ------------------------------------------------------------------------------------ */
#define SGMV_EXCHANGE_MAX_SPLITS 8
#define SGMV_EXCHANGE_MAX_SPLITS_LARGE 4

typedef struct {
  int32_t* sorted_token_ids;
  int32_t* seg_indptr;
  int32_t* seg_lora_ids;
  int32_t* tiles;
  int32_t* info;
  int32_t M, L, chunk_size;
  int32_t seg_cap, large_cap, small_cap;
  void* exchange;
  int64_t exchange_bytes;
} sgmv_segments;

/* Fill seg->M, L, chunk_size, the three capacities and exchange_bytes; pointers (including
 * exchange) are left untouched.
 * Errors: EINVAL (null seg, M < 0, L < 1, chunk_size < 0). */
sgmv_status sgmv_segments_init(int32_t M, int32_t L, int32_t chunk_size, sgmv_segments* seg);

/* Build the segment arrays and work descriptors from per-token adapter ids.
 *   lora_indices  [M] int32 (Fused-LoRA page Step 1; -1 = no adapter, Ascend article 5.3)
 *   on_device = 0: lora_indices and every array of `seg` are HOST memory; runs on the
 *                  calling thread and returns SGMV_EBADID (outputs unspecified) if any id
 *                  is outside {-1} U [0, L). `stream` is ignored.
 *   on_device = 1: DEVICE memory; one launch on `stream`, never synchronises with the host
 *                  (Ascend article 4.2). A bad id is treated as -1 and info[3] is set to
 *                  SGMV_EBADID; otherwise info[3] = SGMV_OK. Requires L <=
 *                  SGMV_DEVICE_BUILDER_MAX_L (else EUNSUPPORTED).
 * Both paths produce identical arrays. M = 0 gives zero segments and zero tiles.
 * Errors: EINVAL (null pointers, seg not initialised for this M/L/chunk_size); EBADID (host);
 * EUNSUPPORTED; EHIP. */
sgmv_status sgmv_build_segments(const int32_t* lora_indices, int32_t M, int32_t L,
                                int32_t chunk_size, int32_t on_device, const sgmv_segments* seg,
                                void* stream);

/* Grouping cache across steps (Ascend article 4.2 and 5.3: a sequence keeps its adapter, so
 * the grouping only changes when sequences join or leave the batch).
 *   cache  [SGMV_CACHE_HEADER + M] int32, in the same memory as lora_indices (host for
 *          on_device = 0, device for 1), owned by the caller; zero-fill it when it is
 *          allocated (an all-zero cache is empty). It must not overlap lora_indices or seg.
 * The cache holds the ids, M, L and chunk_size of the last build made into `seg` through this
 * call with this cache. If all of them equal this call's, seg already holds the result and
 * nothing is written (the device path still reads both id arrays, in one launch); otherwise
 * seg is built exactly as sgmv_build_segments builds it and the cache is refreshed. Both
 * give arrays identical to a fresh build. Anything else that writes seg (sgmv_build_segments,
 * sgmv_lora_delta_ids) leaves the cache stale: zero cache[0] after such a write.
 * Errors: as sgmv_build_segments, plus EINVAL for a null cache with M > 0. */
#define SGMV_CACHE_HEADER 4
sgmv_status sgmv_build_segments_cached(const int32_t* lora_indices, int32_t M, int32_t L,
                                       int32_t chunk_size, int32_t on_device,
                                       const sgmv_segments* seg, int32_t* cache, void* stream);

/* Chunk size for a batch (Punica page, code section: the reordered tokens are cut into
 * fixed-size chunks, each one segment; the page leaves the rule that picks the size open).
 *   M           tokens in the batch
 *   n_adapters  distinct adapters among them if the caller knows it (a scheduler that
 *               collects each step's adapter set does), else 0
 * Returns the chunk size to pass to sgmv_segments_init / sgmv_build_segments, measured on
 * MI355X over 256..8192 tokens, 1..64 adapters and ranks 16..64 (d = 4096): 0 (no chunks)
 * when 1 <= M <= 512 and M <= 8 * n_adapters, where buckets are already small pieces and the
 * single launch of sgmv_lora_delta_ids groups them itself; 16 for any other M <= 1024 (a few
 * adapters' rows then spread over many more workgroups than 64-row pieces give); 0 above,
 * where sequence-ordered prefill batches measured fastest without chunks. M <= 0 gives 0.
 * Never fails. */
int32_t sgmv_chunk_size_for_batch(int32_t M, int32_t n_adapters);

/* ------------------------------------------------------------------------------------
 * sgmv_exchange_placement: checks, on the current device, the workgroup placement that the
 * K-split exchange of the fused call relies on (the exchange workspace described at
 * sgmv_segments): the workgroups that share a piece have equal launch indices modulo 8 and
 * must run on one XCD, whose L2 performs their arrival counter's atomics. It launches a grid of
 * 2048 workgroups that read their XCD id (hardware register XCC_ID) on `stream`, waits for
 * it, and returns SGMV_OK when every workgroup index b ran on the XCD of index b mod 8 (true
 * when the dispatcher deals workgroups round-robin over 1, 2, 4 or 8 XCDs), with the number
 * of XCDs seen in *n_xcd (may be NULL). SGMV_EUNSUPPORTED: the placement does not hold;
 * callers must then pass segments without an exchange workspace. Allocates a small device
 * buffer; not for use under graph capture. Errors: EHIP.
 * ------------------------------------------------------------------------------------ */
sgmv_status sgmv_exchange_placement(int32_t* n_xcd, void* stream);

/* One output slice: pool columns [n_begin, n_begin + n_len) land in columns [0, n_len) of
 * y, a device array [M][ldy] of the pool dtype (e.g. q, k and v of a fused projection). */
typedef struct {
  void* y;
  int64_t ldy;
  int32_t n_begin, n_len;
} sgmv_slice;

/* Shrink (Ascend article 3.2, first stage): for every token t with an adapter l of rank r,
 *   h[t, j] = sum_k x[t, k] * A[l, j, k]   for j < r,    h[t, j] = 0 for r <= j < R_max.
 * Unscaled, fp32. Rows of tokens without adapter are not written.
 *   x  [M][ldx] pool dtype, ldx >= K;   h [M][ldh] fp32, ldh >= R_max.
 * `seg` must hold device arrays built for (M, pool->L). Rows of x are gathered through
 * sorted_token_ids (Punica page, code section).
 * Errors: EINVAL; EUNSUPPORTED; EHIP. */
sgmv_status sgmv_shrink(const void* x, int64_t ldx, int32_t M, const sgmv_pool* pool,
                        const sgmv_segments* seg, float* h, int64_t ldh, void* stream);

/* Expand (Ascend article 3.2, second stage, and 3.3 scatter-add): for every token t with an
 * adapter l of rank r and every output column n of every slice,
 *   y[t, n] = round(y[t, n] + scale_l * sum_{j < r} h[t, j] * B[l, n, j]).
 * Rows of tokens without adapter are left bit-identical. Slices must be disjoint ranges of
 * [0, N); n_slices in [1, SGMV_MAX_SLICES]; `out` is a HOST array. y must not alias h.
 * Errors: EINVAL; EUNSUPPORTED; EHIP. */
sgmv_status sgmv_expand(const float* h, int64_t ldh, int32_t M, const sgmv_pool* pool,
                        const sgmv_segments* seg, const sgmv_slice* out, int32_t n_slices,
                        void* stream);

/* Fused delta (Ascend article 4.3): shrink and expand in one launch; the M x r intermediate
 * stays in registers and LDS and is never written to memory (with an exchange workspace in
 * `seg`, K-range partial sums of it pass through that workspace; see sgmv_segments):
 *   y[t, n] = round(y[t, n] + scale_l * sum_{j < r} B[l, n, j] * sum_k A[l, j, k] x[t, k]).
 * Same arguments and rules as sgmv_shrink and sgmv_expand. y must not alias x or the pool.
 * Errors: EINVAL; EUNSUPPORTED; EHIP. */
sgmv_status sgmv_lora_delta(const void* x, int64_t ldx, int32_t M, const sgmv_pool* pool,
                            const sgmv_segments* seg, const sgmv_slice* out, int32_t n_slices,
                            void* stream);

/* Segment build and fused delta in one call (Fused-LoRA page Step 1 and Ascend article 4.2
 * for the grouping, Ascend article 4.3 for the delta): the same results, in `seg` and in y,
 * as sgmv_build_segments(lora_indices, M, pool->L, seg->chunk_size, 1, seg, stream)
 * followed by sgmv_lora_delta(x, ldx, M, pool, seg, out, n_slices, stream).
 *   lora_indices  [M] int32 DEVICE array; a bad id counts as -1 and sets info[3] to
 *                 SGMV_EBADID, as in the device builder.
 * For a bf16 pool with R_pad == 16 (every rank <= 16), 1 <= M <= SGMV_FUSED_BUILD_MAX_M and
 * pool->L <= SGMV_DEVICE_BUILDER_MAX_L this is ONE launch: every workgroup groups the batch's
 * tokens itself in LDS, and one of them also writes the arrays of `seg`, which no other
 * workgroup of the launch reads. Without chunking and with pool->L <= seg->small_cap, a small
 * piece's exchange control word and partial tiles are those of slot large_cap + its adapter
 * id rather than of its descriptor; the launch leaves the control words consistent, as every
 * completed fused call does. Otherwise (wider ranks, where two launches measured faster,
 * larger batches, fp32) it issues the two launches. Never synchronises with the host.
 * Errors: EINVAL; EUNSUPPORTED; EHIP. */
sgmv_status sgmv_lora_delta_ids(const int32_t* lora_indices, const void* x, int64_t ldx,
                                int32_t M, const sgmv_pool* pool, const sgmv_segments* seg,
                                const sgmv_slice* out, int32_t n_slices, void* stream);

/* ------------------------------------------------------------------------------------ *
 * Launch options (optional; NULL means library defaults). Shared by the _ex variants below,
 * which behave exactly like the calls without the suffix otherwise.
 *   start_event, stop_event: hipEvent_t (as void*) or NULL. When given, the kernel's own
 *     dispatch records them as it starts and as it ends (no extra stream packets), so
 *     hipEventElapsedTime(start, stop) is the kernel's execution time. The caller creates,
 *     owns and destroys them.
 *   n_split_small, n_split_large: workgroups across the output columns for each small /
 *     large work descriptor in expand and fused calls (for each part of a large piece when
 *     large pieces run as parts); 0 = the library's choice, else 1..64.
 *   exchange: fused calls only; 0 = the library's choice, 1 = split a piece class's shrink
 *     over K whenever seg->exchange is set and its split count is in range (small: 2..8,
 *     large: 2..4; parts of large pieces: 2..8 when R_pad <= 32, else 2..4), -1 = never.
 *   exchange_wait: bound on a small piece's wait for its partners' partial sums, in units of
 *     10 ns (large pieces wait up to 10 times as long); 0 = default (20 us), -1 = no wait
 *     (every partial not yet published is computed locally; same results, for testing that
 *     path).
 * Errors: EINVAL (a split outside 0..64, exchange outside -1..1, exchange_wait < -1).
 * ------------------------------------------------------------------------------------ */
typedef struct {
  void* start_event;
  void* stop_event;
  int32_t n_split_small;
  int32_t n_split_large;
  int32_t exchange;
  int32_t exchange_wait;
} sgmv_launch_opts;

sgmv_status sgmv_build_segments_ex(const int32_t* lora_indices, int32_t M, int32_t L,
                                   int32_t chunk_size, int32_t on_device,
                                   const sgmv_segments* seg, const sgmv_launch_opts* opts,
                                   void* stream);
sgmv_status sgmv_build_segments_cached_ex(const int32_t* lora_indices, int32_t M, int32_t L,
                                          int32_t chunk_size, int32_t on_device,
                                          const sgmv_segments* seg, int32_t* cache,
                                          const sgmv_launch_opts* opts, void* stream);
sgmv_status sgmv_shrink_ex(const void* x, int64_t ldx, int32_t M, const sgmv_pool* pool,
                           const sgmv_segments* seg, float* h, int64_t ldh,
                           const sgmv_launch_opts* opts, void* stream);
sgmv_status sgmv_expand_ex(const float* h, int64_t ldh, int32_t M, const sgmv_pool* pool,
                           const sgmv_segments* seg, const sgmv_slice* out, int32_t n_slices,
                           const sgmv_launch_opts* opts, void* stream);
sgmv_status sgmv_lora_delta_ex(const void* x, int64_t ldx, int32_t M, const sgmv_pool* pool,
                               const sgmv_segments* seg, const sgmv_slice* out,
                               int32_t n_slices, const sgmv_launch_opts* opts, void* stream);
/* With two launches, start_event is recorded by the build and stop_event by the delta. */
sgmv_status sgmv_lora_delta_ids_ex(const int32_t* lora_indices, const void* x, int64_t ldx,
                                   int32_t M, const sgmv_pool* pool, const sgmv_segments* seg,
                                   const sgmv_slice* out, int32_t n_slices,
                                   const sgmv_launch_opts* opts, void* stream);

/* ------------------------------------------------------------------------------------ *
 * For callers that cannot allocate device memory (code under HIP graph capture, tight
 * serving loops, harnesses that forbid allocation): sgmv_lora_delta_ids with the K-split
 * exchange workspace in a static device array of SGMV_NOALLOC_SCRATCH_BYTES that the library
 * holds on every GPU it runs on until the process ends, instead of in seg->exchange (which
 * is ignored). Same arguments, launches and results, bit for bit, as sgmv_lora_delta_ids on
 * segments with a workspace. The call allocates nothing: no hipMalloc or hipFree, no
 * allocating library routine; its first call on a device looks up that device's copy of the
 * array. The caller still provides the inputs and the outputs (ids, x, the pool, the
 * segment arrays of seg, y).
 * Limit: the exchange layout of seg (sgmv_segments_init's exchange_bytes) must fit in
 * SGMV_NOALLOC_SCRATCH_BYTES, e.g. a 256-token batch over a pool of up to 1024 adapters, or a
 * 512-token batch over up to 440; larger ones return SGMV_EUNSUPPORTED before anything runs.
 * Every call on one GPU shares that GPU's array, which keeps the last call's contents (its
 * counters stay consistent across completed calls): calls that overlap on one GPU race, so
 * order them on one stream.
 * Errors: as sgmv_lora_delta_ids; EUNSUPPORTED beyond the limit; EHIP if the array's device
 * address cannot be looked up.
 * ------------------------------------------------------------------------------------ */
#define SGMV_NOALLOC_SCRATCH_BYTES (16 << 20)
sgmv_status sgmv_lora_delta_ids_noalloc(const int32_t* lora_indices, const void* x, int64_t ldx,
                                        int32_t M, const sgmv_pool* pool,
                                        const sgmv_segments* seg, const sgmv_slice* out,
                                        int32_t n_slices, void* stream);

/* ------------------------------------------------------------------------------------ *
 * Merged weight of one adapter (Ascend article 1.1 and 4.4: for a batch that holds only one
 * or two long-lived adapters, merging each into a copy of the base weight and running the
 * plain GEMM can beat the unmerged delta; Punica page, SGMV section: merged and unmerged
 * forms give the same product).
 *   w       device [N][ldw] of the pool dtype: the base weight of y = x W^T (row n = output n,
 *           column k = input k), N = pool->N, K = pool->K, ldw >= K
 *   w_out   device [N][ldo], ldo >= K; may be w itself (in place), must not overlap it
 *           otherwise
 *   adapter l in [0, pool->L)
 * w_out[n][k] = w[n][k] + scale_l * sum_{j < r_l} B[l][n][j] * A[l][j][k], the product summed
 * in fp32 (exact bf16 products) and the result rounded once to the pool dtype (bf16: to
 * nearest even). Ranks at or past r_l are never read. To go back to the unmerged weight keep
 * w (merge out of place): in bf16, merging -scale does not undo a merge exactly.
 * Errors: EINVAL (null pointers, ld < K, adapter out of range, an invalid pool); EHIP. */
sgmv_status sgmv_merge_adapter(const void* w, int64_t ldw, void* w_out, int64_t ldo,
                               const sgmv_pool* pool, int32_t adapter, void* stream);
sgmv_status sgmv_merge_adapter_ex(const void* w, int64_t ldw, void* w_out, int64_t ldo,
                                  const sgmv_pool* pool, int32_t adapter,
                                  const sgmv_launch_opts* opts, void* stream);

/* Human-readable name of a status code (static string). */
const char* sgmv_status_string(sgmv_status s);

/* Library version as major*10000 + minor*100 + patch. */
int32_t sgmv_version(void);

#ifdef __cplusplus
}
#endif

#endif /* SGMV_H */
