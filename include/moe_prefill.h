/*
 * moe_prefill.h -- C ABI of libmoe_prefill.so, the MI355X (gfx950) prompt-path MoE expert layer.
 *
 * The layer is the one the Strata prompt-path pages tune:
 *   [G1] "#439 prefill: a group's expert gathers in one launch (bit-identical, long prompts +4%)"
 *   [G2] "Prompt path: an MMQ group's experts gathered in one launch, after one wait, released by
 *         one event (-9% on a 32K prompt, same output)"
 *   [QS] "#1368 prefill: quantize each token's MoE input once and scatter it to its k rows
 *         (the same bytes)"
 *   [CS] "#1282 prefill: STRATA_PREFILL_CPU_SHARE=auto hands a small chunk's least-routed experts
 *         to the idle CPU pool (opt-in)"
 *
 * Conventions for every entry point
 *   - Pointers are DEVICE pointers unless marked [host].  The caller owns every buffer; the
 *     library allocates nothing on any compute path and keeps no state between calls, apart
 *     from the optional stage profiler and a streamed walk's own object (moe_walk_create, whose
 *     ring bookkeeping and events carry from one call to the next by design).
 *   - `stream` is a hipStream_t passed as void* (NULL = the null stream).  Work is enqueued on it
 *     and the call returns at once; nothing synchronises with the host.
 *   - Return value: MOE_OK (0) or a negative moe_status.  Argument checks run on the host before
 *     anything is enqueued (MOE_EINVAL, MOE_EUNSUPPORTED, MOE_EWORKSPACE); a failed launch returns
 *     MOE_EHIP.  Device-side data is not checked on the host.  A routed expert id outside [0, E)
 *     is a caller error that the kernels detect: the maps give such a route slot = -1 and a row
 *     past offsets[E] with src = -1, it contributes nothing to the output, and its count is
 *     stored in device memory (moe_build_maps: the first int32 of ws; the layer: the first of
 *     the workspace's MOE_WS_STATUS words), 0 when every id is in range; nothing is read or
 *     written out of bounds.  Finite inputs (x, logits, the experts' scales) are the caller's duty: with
 *     non-finite ones the results are unspecified, but the kernels stay in bounds.
 *   - Calls are reentrant; calls that share output or workspace buffers must not overlap.
 *
 * Byte formats (little endian)
 *   Q8_0 weight block, 34 B : fp16 d | int8 q[32]                          w_j = d*q_j
 *   Q4_1 weight block, 20 B : fp16 d | fp16 m | u8 qs[16]                  w_j = d*q_j + m
 *                             qs[j]: element j in the low nibble, element j+16 in the high nibble
 *   expert, expert_bytes    : gate [F rows x H/32 blocks] | up [F x H/32] | down [H x F/32],
 *                             each matrix row-major with its blocks along the reduction dimension
 *   MMQ layout of an expert : what moe_gather_group_mmq writes and moe_mmq_grouped reads (this
 *                             library's choice; the pages only require the gathered experts to
 *                             feed the matmul).  Same order gate | up | down and the same size;
 *                             each matrix of n_rows rows and nblk blocks per row is stored as tiles
 *                             of 64 rows by 4 blocks: for tile j, stage t, row i < 64 (row 64j+i),
 *                             the row's blocks 4t..4t+3 take G = 4 * block bytes at byte
 *                             ((j * nblk/4 + t) * 64 + i) * G, headers first:
 *                               Q4_1 (G = 80) : (d, m) of the 4 blocks, then each block's 16
 *                                               packed bytes in two halves: byte 8h + i holds
 *                                               element 16h + i in its low nibble and element
 *                                               16h + 8 + i in its high nibble
 *                               Q8_0 (G = 136): d of the 4 blocks, then their q[32]
 *   q8_1 row of n values    : n/128 groups of 144 B: (fp16 d, fp16 s) of its 4 blocks of 32, then
 *                             the 4 blocks' int8 q.  d = amax/127 (fp32), q = roundf(v/d), s = d*sum q
 *                             ([QS] opening section and "Identity": the DS4 layout, which carries the
 *                             s that Q4_1's min term needs).
 */
#ifndef MOE_PREFILL_H
#define MOE_PREFILL_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define MOE_ABI_VERSION 7
#define MOE_MAX_GROUP 16     /* experts per group buffer ([G1] "What": MMQ_GROUP = 16) */
#define MOE_MAX_E 2048       /* largest expert count the kernels accept */
#define MOE_MAX_K 64         /* largest routes per token */

typedef enum {
    MOE_OK = 0,
    MOE_EINVAL = -1,        /* a null pointer, a size out of range, inconsistent arguments */
    MOE_EUNSUPPORTED = -2,  /* a valid request the library does not implement (H or F not a
                               multiple of 128, E > MOE_MAX_E, K > MOE_MAX_K, unknown type) */
    MOE_EWORKSPACE = -3,    /* the workspace is smaller than the matching *_workspace_size() */
    MOE_EHIP = -4,          /* a HIP launch or runtime call failed */
    MOE_ENOMEM = -5         /* host memory or host threads could not be obtained (the streamed walk,
                               its CPU share, the host planner and the stage profiler allocate on
                               the host); the call stopped and its outputs are unspecified */
} moe_status;

/* Weight type, and with it the q8_1 layout of the activations the MMQ reads: Q8_0 and Q4_1 take
 * DS4 rows; MOE_Q8_0_D4 is Q8_0 weights taking D4 rows (the layout [QS] "Identity" names for Q8_0:
 * per 128 values the 4 blocks' fp32 d, then their q, no s).  In the MMQ a D4 d enters the scale
 * product as fp16(d) + fp16(d - fp16(d)), which carries d to within max(2^-22 d, 2^-25) while
 * fp16(d) is finite (d <= 65504, a block's largest magnitude <= 8.3e6); beyond that the product
 * overflows, as DS4's fp16 d does. */
typedef enum { MOE_Q8_0 = 0, MOE_Q4_1 = 1, MOE_Q8_0_D4 = 2 } moe_wtype;

/* moe_quantize_scatter_q8_1 mode bits */
#define MOE_QUANT_PER_ROW 1   /* the per-row form (else: scatter) */
#define MOE_QUANT_D4 2        /* D4 rows (else: DS4) */

typedef enum {
    MOE_EPI_F32 = 0,           /* out = fp32 [rows x n_out] products (the down projection) */
    MOE_EPI_SWIGLU_Q8_1 = 1,   /* out = q8_1 rows of h = silu(gate)*up, [rows x n_out/128*144] */
    MOE_EPI_I32_BLOCKDOTS = 2  /* out = int32 [rows x n_out x k_in/32] raw block dots (checking) */
} moe_epilogue;

int moe_abi_version(void);
const char *moe_strerror(int status);

/* Sizes (bytes). */
size_t moe_block_bytes(int wtype);                      /* 34 or 20; 0 if unknown */
size_t moe_expert_bytes(int H, int F, int wtype);       /* 3*H*F/32 blocks */
size_t moe_q8_1_row_bytes(int n);                       /* n/128*144 */
/* The two workspace queries return 0 for shapes the matching entry point would refuse
 * (non-positive sizes, T*K above 2^30, H or F not a positive multiple of 128, unknown type,
 * group_size outside 1..MOE_MAX_GROUP). */
size_t moe_build_maps_workspace_size(int T, int K, int E);
size_t moe_workspace_size(int T, int H, int F, int E, int K, int wtype, int group_size);

/* a0  Top-K routing ([QS] "Identity": routing built as Prefill builds it, 10 of 512 experts).
 * logits fp32 [T x E] -> idx int32 [T x K] (the K largest logits, equal logits: lower id first),
 * w fp32 [T x K] (softmax over the K chosen logits = softmax, top-K, renormalise).  E <= 2048.
 * The logits must be finite (the kernel marks picked entries -inf). */
int moe_route_topk(const float *logits, int T, int E, int K, int32_t *idx, float *w,
                   void *stream);

/* a1  Token -> row maps ([QS] opening section: src_dev names each row's source; token t's k-th row
 * is slot[t*K+k], the inverse of src_dev).  From idx int32 [T x K]:
 *   counts [E]; offsets [E+1] (exclusive prefix of counts); src [T*K]: row r -> t*K+k, rows grouped
 *   by expert id ascending, ascending t*K+k inside an expert (stable); slot [T*K] = src^-1;
 *   order [E]: the experts with rows, in ring order from ring_start ([G2] "What changes": skipped
 *   ring entries hold no rows); n_active [1]: how many.  Group g of size gs is order[gs*g ...].
 * An id outside [0, E) counts as one more expert after the last: its entries take rows
 * offsets[E] .. T*K-1 (index order) with src = -1, and their slot is -1.
 * ws: at least moe_build_maps_workspace_size(T, K, E) bytes of device scratch; after the call its
 * first int32 holds the number of ids outside [0, E). */
int moe_build_maps(const int32_t *topk_idx, int T, int K, int E, int ring_start,
                   int32_t *counts, int32_t *offsets, int32_t *src, int32_t *slot,
                   int32_t *order, int32_t *n_active, void *ws, size_t ws_bytes, void *stream);

/* a1  moe_build_maps for callers that cannot allocate (code under HIP graph capture, tight
 * serving loops, harnesses that forbid hipMalloc): the same maps, bit for bit, with no workspace
 * argument.  Its scratch is a static device array of MOE_NOALLOC_SCRATCH_BYTES that each GPU the
 * library runs on holds until the process ends; nothing is allocated, on the device or the host,
 * by this call (its first call on a device looks the array's address up).  n_invalid: NULL, or
 * a device int32 [1] that receives the number of ids outside [0, E) (else that count lands in
 * the scratch).  T*K above MOE_NOALLOC_MAX_ROUTES or E above MOE_MAX_E: MOE_EUNSUPPORTED.  Every
 * call on one GPU shares that GPU's array (each call rewrites all of it that it reads), so calls
 * that overlap on one GPU, on any streams, race: serialise them. */
#define MOE_NOALLOC_MAX_ROUTES (1 << 19)
#define MOE_NOALLOC_SCRATCH_BYTES ((size_t)4196608)   /* 256 + 512 chunks x 2049 bins x 4 B */
int moe_build_maps_noalloc(const int32_t *topk_idx, int T, int K, int E, int ring_start,
                           int32_t *counts, int32_t *offsets, int32_t *src, int32_t *slot,
                           int32_t *order, int32_t *n_active, int32_t *n_invalid, void *stream);

/* a2  q8_1 quantisation of the layer input ([QS] opening section).
 * x fp32 [T x H] row-major; q8 [T*K x moe_q8_1_row_bytes(H)].
 * mode without MOE_QUANT_PER_ROW (scatter): each token row is read once and written to rows
 * slot[t*K+k], k < K.  With it (per-row gather, the form the page replaces): row r quantises
 * token src[r]/K.  Both write the same bytes.  MOE_QUANT_D4: rows in the D4 layout.  A slot
 * (scatter) or src (per-row) of -1 writes nothing. */
int moe_quantize_scatter_q8_1(const float *x, int T, int H, int K, const int32_t *slot,
                              const int32_t *src, int mode, void *q8, void *stream);

/* a3  One group's gather in one launch ([G1] "What", [G2] "What changes"; blockIdx.y = expert).
 * src_ptrs [host]: n (1..16) device pointers to experts of expert_bytes each.  Expert j lands at
 * group_buf + (first_pos + j) * pos_stride, first_pos + n <= 16 (a batch may start mid-group).
 * The bytes are exactly those of one copy per expert; pointers or sizes that are not 16-byte
 * multiples take a byte-wise path instead of 16-byte copies. */
int moe_gather_group(const void *const *src_ptrs, int n, size_t expert_bytes, void *group_buf,
                     int first_pos, size_t pos_stride, void *stream);

/* a3  The same gather writing each expert in the MMQ layout, the form moe_mmq_grouped reads and
 * the layer uses.  src_ptrs [host]: n (1..16) device pointers to raw experts of
 * moe_expert_bytes(H, F, wtype) bytes; positions as in moe_gather_group, pos_stride >= that size
 * when n > 1.  H and F: multiples of 128.  Experts at 16-byte (Q4_1) or 8-byte (Q8_0) aligned
 * addresses, with a group_buf position of the same alignment, move in whole words; others take a
 * byte-wise path with the same result. */
int moe_gather_group_mmq(const void *const *src_ptrs, int n, int wtype, int H, int F,
                         void *group_buf, int first_pos, size_t pos_stride, void *stream);

/* a4..a6  Grouped quantised matmul (MMQ) over one group buffer ([G2] "What changes", [QS] opening
 * section).  Position j < n_group of group_buf (at j*pos_stride) holds expert group_experts[j] in the
 * MMQ layout (moe_gather_group_mmq)
 * ([host] array, each in [0, E)); its rows are offsets[e] .. offsets[e+1]-1 (offsets: int32 [E+1],
 * device) of act_q8 (q8_1 rows of k_in values,
 * grouped by expert as moe_build_maps orders them).  The weight matrix starts mat_offset bytes into
 * each expert and has n_out rows of k_in/32 blocks (for MOE_EPI_SWIGLU_Q8_1 that matrix is gate and
 * up is the next matrix, n_out*k_in/32 blocks further).  Per block b: I_b = integer dot of the 32 int8 (Q8_0) or 4-bit (Q4_1)
 * weights with the 32 int8 activations; y_b = dw*dx*I_b (+ mw*sx for Q4_1); a row's result is the
 * sum over b.  Output row r is written at row r of `out` (rows of other experts untouched):
 *   MOE_EPI_F32:           fp32 [* x n_out]
 *   MOE_EPI_SWIGLU_Q8_1:   q8_1 rows of h = silu(g)*u (n_out values); debug_h, if not NULL, gets the
 *                          fp32 h [* x n_out] that was quantised
 *   MOE_EPI_I32_BLOCKDOTS: int32 [* x n_out x k_in/32], the raw I_b
 * n_out and k_in: multiples of 128, the matrix (both matrices for MOE_EPI_SWIGLU_Q8_1) below
 * 4 GiB, else MOE_EUNSUPPORTED.  group_buf, pos_stride and mat_offset: multiples of 16 bytes;
 * act_q8: 16-byte aligned.  The matrix must lie inside each position's bytes (caller's duty). */
int moe_mmq_grouped(int wtype, const void *group_buf, size_t pos_stride, size_t mat_offset,
                    int n_out, int k_in, const int32_t *group_experts, int n_group,
                    const int32_t *offsets, int E, const void *act_q8, int epilogue, void *out,
                    float *debug_h, void *stream);

/* a7  Combine ([CS] "What it does": Dm holds the expert rows without their routing weights, which
 * the combine applies).
 * out[t,i] = sum_{k<K} w[t,k] * Dm[slot[t*K+k], i], k ascending, a route with slot -1 left out;
 * Dm fp32 [T*K x H]. */
int moe_combine(const float *Dm, const int32_t *slot, const float *topk_w, int T, int K, int H,
                float *out, void *stream);

/* a1..a7  The whole layer: maps, quantise-scatter, every group's gather, MMQ gate/up with SwiGLU and
 * q8_1 requantisation, MMQ down into Dm, combine.
 * x fp32 [T x H]; topk_idx int32 / topk_w fp32 [T x K]; pool: the experts, expert e at byte
 * expert_off[e] (int64 [E], device) of expert_bytes = moe_expert_bytes(H, F, wtype).  The pool's
 * size is not an argument: every routed expert's bytes lying inside it is the caller's duty.
 * group_size (1..16) and ring_start (0..E-1) set which experts share a group buffer; the output is
 * bit-identical for every choice ([G1] "What": every byte reaches the position one copy per expert
 * gives it; [G2] "What changes": neither the products nor their order change).  ws: moe_workspace_size(...) bytes.
 * out fp32 [T x H].  H, F multiples of 128 (gate and up together, and down, each below 4 GiB);
 * E <= 2048; K <= min(E, 64). */
int moe_prefill_layer(const float *x, int T, int H, int F, int E, int K,
                      const int32_t *topk_idx, const float *topk_w, int wtype,
                      const void *pool, const int64_t *expert_off, size_t expert_bytes,
                      int group_size, int ring_start, void *ws, size_t ws_bytes, float *out,
                      void *stream);

/* a1, a2, a4..a7  The layer over experts that stay resident in the MMQ layout, with no gather
 * (the pages' gather exists to assemble a group buffer from expert slots, [G1] "What"; an expert
 * pool that never leaves device memory can be put in the matmul's layout once, with
 * moe_gather_group_mmq, and read in place).  packed_pool: expert e in the MMQ layout at byte
 * expert_off[e] (int64 [E], device; multiples of 16: an expert at an offset that is not is
 * skipped, its rows are unspecified and the second MOE_WS_STATUS word is set non-zero; inside the
 * pool: the caller's duty, as for moe_prefill_layer).  The matmul sees the bytes moe_prefill_layer gathers, so the output is
 * that call's with the same arguments, bit for bit; ws as there
 * (moe_workspace_size with any group size; the group region is not used). */
int moe_prefill_layer_packed(const float *x, int T, int H, int F, int E, int K,
                             const int32_t *topk_idx, const float *topk_w, int wtype,
                             const void *packed_pool, const int64_t *expert_off,
                             size_t expert_bytes, int ring_start, void *ws, size_t ws_bytes,
                             float *out, void *stream);

/* Where moe_prefill_layer keeps its intermediate results inside ws, for checking them:
 * the byte offset of region `which` (MOE_WS_*) for these arguments, or (size_t)-1. */
enum {
    MOE_WS_COUNTS = 0,   /* int32 [E] */
    MOE_WS_OFFSETS = 1,  /* int32 [E+1] */
    MOE_WS_SRC = 2,      /* int32 [T*K] */
    MOE_WS_SLOT = 3,     /* int32 [T*K] */
    MOE_WS_ORDER = 4,    /* int32 [E], then n_active at MOE_WS_NACTIVE */
    MOE_WS_NACTIVE = 5,  /* int32 [1] */
    MOE_WS_Q8X = 6,      /* q8_1 rows of x [T*K x moe_q8_1_row_bytes(H)] */
    MOE_WS_GROUPS = 7,   /* group buffers: active expert i (ring order) at i * stride */
    MOE_WS_HQ8 = 8,      /* q8_1 rows of h [T*K x moe_q8_1_row_bytes(F)] */
    MOE_WS_DM = 9,       /* fp32 [T*K x H] */
    MOE_WS_GROUP_STRIDE = 10, /* not an offset: the byte stride between group positions */
    MOE_WS_STATUS = 11        /* int32 [2], rewritten by every layer call: [0] the routed ids
                                 outside [0, E); [1] non-zero when moe_prefill_layer_packed met an
                                 expert whose bytes are not 16-byte aligned (its rows are then
                                 unspecified); 0 and 0 for a clean call */
};
size_t moe_workspace_offset(int which, int T, int H, int F, int E, int K, int wtype,
                            int group_size);

/* ---- Streamed walk ([G2] "What changes"; the per-expert form it replaces: the opening section) ----
 *
 * Experts that are not resident in device memory are copied from a host arena into a ring of
 * device slots on a copy stream, while the compute stream walks the routed experts in ring order.
 * Per gather batch (at most one group of group_size positions):
 *   - one wait: the compute stream waits on an event recorded after the batch's last copy (the
 *     copy stream is in order, so that covers every copy of the batch);
 *   - one launch: moe_gather_group_mmq's kernel moves the batch's experts (ring slots or resident
 *     experts) to their group buffer positions;
 *   - one event: recorded after that launch, it gives every ring slot the batch read back to the
 *     copies: before a slot is refilled the copy stream waits on used[used_of[slot]], used_of
 *     mapping each slot to the event recorded by the last batch that read it (events are reused
 *     round-robin from a pool of MOE_WALK_EVENTS: an event recorded again by a later batch can
 *     only delay such a copy, never let it start early).
 * A batch is launched when its group is complete, when the walk meets a ring entry the routing
 * skipped while the group is open ([G2] "What changes": the entries waiting in an open batch
 * never exceed one group), or when the next copy needs a ring slot that the open batch itself holds (a ring
 * smaller than a group).  After a group's last batch its MMQ gate/up and down launch on that
 * group's m-tiles, so a group's products overlap later groups' copies; the MMQs of consecutive
 * groups whose later batches need no copy wait (resident experts, copies already covered) go out
 * as one launch pair over their m-tiles, which fills the GPU where per-group launches would not
 * (MOE_WALK_MMQ_PER_GROUP keeps one pair per group).  The output is
 * bit-identical to moe_prefill_layer's for the same arguments: every expert's bytes reach the
 * position the layer gives them, and the matmuls are the same launches' arithmetic. */
#define MOE_WALK_EVENTS 64
#define MOE_WALK_GATHER_ONE 1      /* one expert per batch: one wait, launch and event per expert
                                      ([G2] "What changes", the opt-out) */
#define MOE_WALK_NO_SKIP_FLUSH 2   /* a skipped ring entry does not launch the open batch */
#define MOE_WALK_MMQ_PER_GROUP 4   /* one MMQ launch pair per group, never merged (the pages' form) */

typedef struct moe_walk moe_walk;

/* Creates the walk's state for a caller-owned device ring of n_slots (>= 1) slots, slot_stride
 * bytes apart (a multiple of 256): a copy stream (default priority), MOE_WALK_EVENTS + 2 events,
 * a pinned host buffer for the routing read-back, and the slot map (every slot free).  The ring
 * must stay allocated until moe_walk_destroy has returned.  *walk is set on MOE_OK; MOE_ENOMEM if
 * the host memory for the walk's state could not be obtained, MOE_EHIP if a HIP resource (the
 * stream, an event, the pinned buffer) could not be made.  A walk serves one call at a time: its
 * host-side plan, read-back buffer and slot map are not guarded, so two threads must not call
 * moe_prefill_layer_streamed on the same walk at once.  For calls in sequence, even on different
 * streams, the walk's events order the reuse of its ring slots; a workspace or output shared
 * between such calls follows the general rule above. */
int moe_walk_create(void *ring, int n_slots, size_t slot_stride, moe_walk **walk);

/* Waits for the walk's copies and for every gather that read its ring (the slots' events), then
 * frees what moe_walk_create made; the ring may be freed after this returns.  NULL is a no-op. */
int moe_walk_destroy(moe_walk *walk);

/* The whole layer as moe_prefill_layer computes it, with the experts streamed as described above.
 *   host_arena [host, pinned]: arena_bytes bytes; host_off [host] int64 [E]: expert e's raw bytes
 *     start at host_arena + host_off[e];
 *   resident [host] [E]: a device pointer to expert e's raw bytes, or NULL to stream it;
 *   flags: MOE_WALK_* bits.
 * Other arguments as in moe_prefill_layer (same workspace, moe_workspace_size).  The call blocks
 * the host once, until the routing is known on the host (the maps, then a read-back of counts,
 * order and n_active: the routing sync); everything after it is enqueued on `stream` and the
 * walk's copy stream.  The arena must stay unchanged until `stream` has passed this call.
 * Calls on one walk must not overlap; the walk's slot map and events carry over between calls,
 * so a slot read by one call is refilled by the next only after that read. */
/* After a MOE_EHIP or MOE_ENOMEM from this call the walk's slot map may name events that were
 * never recorded: destroy the walk. */
int moe_prefill_layer_streamed(moe_walk *walk, const float *x, int T, int H, int F, int E, int K,
                               const int32_t *topk_idx, const float *topk_w, int wtype,
                               const void *host_arena, size_t arena_bytes,
                               const int64_t *host_off, const void *const *resident,
                               int group_size, int ring_start, int flags, void *ws,
                               size_t ws_bytes, float *out, void *stream);

/* Counters of a walk since it was created [host] int64 [n]:
 *   0 copies, 1 bytes copied, 2 gather batches, 3 compute-stream waits on copies,
 *   4 copy-stream waits on slot events (none is issued for an event already complete),
 *   5 batches launched for a skipped entry,
 *   6 batches launched for a ring slot held by the open batch, 7 MMQ launches, 8 routing syncs,
 *   9 host->device transfers (consecutive copies of one batch whose experts lie slot_stride apart
 *     in the arena and land in consecutive slots go out as one transfer),
 *   the CPU share (moe_walk_cpu_share): 10 experts the host computed, 11 their routed rows,
 *   12 host compute time in microseconds, and of the last call 13 the share used (x 10^6),
 *   14 the GPU's measured time per streamed expert (ns), 15 the host's (ns); 0 = not measured.
 * Writes min(n, MOE_WALK_NSTATS) entries. */
#define MOE_WALK_NSTATS 16
int moe_walk_stats(const moe_walk *walk, int64_t *stats, int n);

/* The CPU share of a walk ("#1282 prefill: STRATA_PREFILL_CPU_SHARE=auto hands a small chunk's
 * least-routed experts to the idle CPU pool", "What it does"), opt-in; off unless this is called.
 * From the next moe_prefill_layer_streamed on, after the routing sync, the streamed (non-resident)
 * routed experts routed by at most max_tokens tokens (0: any count), fewest first, up to
 * share x (the call's streamed routed experts), are computed on the host: a pool of `threads` host
 * threads (0: all the host has) reads them from the arena and the call's x and src (copied to the
 * host before the routing sync) and computes their unweighted rows (q8_1 of x, gate/up, SwiGLU,
 * q8_1 of h, down) while the GPU streams and computes the rest; the GPU neither copies, gathers
 * nor multiplies them.  The rows are staged contiguously, copied to the device once and put into
 * their Dm rows, and the combine weights them as any other row.  The host's integer dots are the
 * GPU's; its fp32 sums run in another order, so the output is within fp32 rounding of the GPU's,
 * not bit-identical.  The call blocks until the host's part is done (besides the routing sync).
 *   share: in (0, 1] a fixed share; < 0 automatic: 0.25 first, then g / (c + g) from the
 *          previous call's measured GPU time per streamed expert (g, events around its expert
 *          work) and host time per expert (c); 0 turns the share off and frees its buffers.
 *   max_T, H: the largest T and the H of the calls (a call outside them returns MOE_EINVAL);
 *   max_rows: at most this many rows per call go to the host (its staging capacity).
 * Allocates pinned host buffers (max_T x H and max_rows x H fp32), device buffers (max_rows x H
 * fp32) and starts the threads; MOE_EHIP if the HIP buffers or events cannot be made, MOE_ENOMEM
 * if the host threads or their scratch cannot (either way the previous setting stays).
 * Not a fallback: the HIP path never hands work to the host unless the caller asks for it here. */
int moe_walk_cpu_share(moe_walk *walk, double share, int max_tokens, int threads, int max_T,
                       int H, int max_rows);

/* The host's computation for one expert, as the CPU share runs it ([CS] "What it does"): the
 * unweighted rows of n_rows inputs through a raw expert.  All pointers [host]: expert
 * moe_expert_bytes(H, F, wtype) bytes, x fp32 [n_rows x H], out fp32 [n_rows x H].  Runs on the
 * calling thread.  H, F multiples of 128. */
int moe_cpu_expert_rows(int wtype, int H, int F, const void *expert, const float *x, int n_rows,
                        float *out);
/* The host instruction set the CPU share's dot products use: "avx512-vnni", "avx2" or "scalar". */
const char *moe_cpu_share_isa(void);

/* The walk's schedule alone, computed on the host as moe_prefill_layer_streamed computes it
 * (nothing is enqueued; no device is needed).  Inputs [host]: counts int32 [E], order int32 [E]
 * and n_active as moe_build_maps returns them; streamed uint8 [E] (1 = copied from the arena,
 * 2 = computed by the host: never copied nor gathered, its position kept);
 * group_size, n_slots, flags as above.  State in/out [host]: used_of int32 [n_slots] (the event
 * of each slot's last reader batch, -1 = never read), cursor (next ring slot, 0..n_slots-1),
 * next_event (the event the next batch records, 0..MOE_WALK_EVENTS-1).  ops [host] int32 [max_ops x 6],
 * one record per step in issue order:
 *   {1, pos, expert, slot, wait_event (-1: none), 0}         copy expert into a ring slot
 *   {2, first_pos, n, waits (0/1), event, why}               gather batch of positions
 *                                                            first_pos .. first_pos+n-1;
 *                                                            why: 0 group complete, 1 skipped
 *                                                            entry, 2 slot held, 3 one expert,
 *                                                            4 a host-computed expert follows
 *   {3, group, first_pos, n, 0, 0}                           MMQ of the group's positions
 * Returns the number of records, MOE_EINVAL (inconsistent inputs) or MOE_EWORKSPACE (max_ops too
 * small; the state is then unspecified). */
int moe_walk_plan(const int32_t *counts, const int32_t *order, int n_active, int E,
                  int ring_start, const uint8_t *streamed, int group_size, int n_slots, int flags,
                  int32_t *used_of, int32_t *cursor, int32_t *next_event, int32_t *ops,
                  int max_ops);

/* Optional stage timing of moe_prefill_layer with HIP events recorded on the call's stream.
 * moe_profile_begin(n) arms it for the next n calls (creates the events); moe_profile_end()
 * waits for the last recorded event, writes ms [n_done x MOE_N_STAGES] (stage order: maps,
 * quantize, gather, gate/up, down, combine) into ms [host] (capacity max_calls rows), returns
 * the number of calls recorded (or a negative status) and disarms it. */
#define MOE_N_STAGES 6
int moe_profile_begin(int n_calls);
int moe_profile_end(float *ms, int max_calls);

#ifdef __cplusplus
}
#endif
#endif
