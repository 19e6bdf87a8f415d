/*
 * bsa.h -- C ABI of the MI355X (gfx950) block-sparse attention forward library.
 *
 * The library computes softmax(Q K^T / sqrt(d)) V over exactly the query/key
 * pairs a logical mask selects, for every (batch, head), on one GPU.
 *
 * Two calls carry the method (Tessera, arXiv 2609.25869, abstract: the
 * logical mask that specifies which interactions to compute is decoupled from
 * the GPU execution that computes them, and preparation cost must stay small
 * next to the execution it saves):
 *
 *   bsa_plan    -- host side: validates the logical mask, maps it onto physical
 *                  tiles (empty tiles dropped, exact masking only on partial
 *                  tiles), selects an execution regime from a lookup table
 *                  built by offline profiling, groups tiles into workgroup
 *                  tasks and uploads the result to the device once.
 *   bsa_forward -- device side: runs a plan on caller-owned Q, K, V, O.
 *
 * bsa_plan_device builds the same plan on the GPU from a BLOCK mask already
 * in device memory, and a request (bsa_request_*) pipelines the planning of
 * one mask with the forwards of the previous ones.
 *
 * Conventions
 *  - All functions are plain C, never throw, and report errors through their
 *    return value; bsa_last_error() gives a thread-local message for the last
 *    failing call of the calling thread.
 *  - Tensors Q, K, V, O are caller-owned DEVICE pointers, contiguous
 *    [B][H][L][d] in the plan's dtype (bf16 or fp32), rows in frame-major token
 *    order (token i = t*Hg*Wg + y*Wg + x), 16-byte aligned. Q, K, V are only
 *    read. O is fully overwritten, including rows with no kept key (zeros).
 *  - Masks given to bsa_plan are HOST memory owned by the caller; bsa_plan
 *    copies what it needs, so the caller may free the mask as soon as it
 *    returns (bsa_plan_device reads a device mask; see there).
 *  - A plan owns its host and device memory and is immutable; it may be used
 *    by any number of bsa_forward calls on any streams of its device, also
 *    concurrently. Destroy it only after the streams that use it are done.
 */
#ifndef BSA_H
#define BSA_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define BSA_ABI_VERSION 7

typedef struct bsa_plan_s *bsa_plan_t;

/* Status codes (returned as int32_t). */
enum {
    BSA_OK = 0,
    BSA_ERR_INVALID_ARGUMENT = 1, /* null pointer, bad shape, bad option          */
    BSA_ERR_INVALID_MASK = 2,     /* mask contents out of range / unsorted / dup   */
    BSA_ERR_UNSUPPORTED = 3,      /* valid request the library does not implement  */
    BSA_ERR_OUT_OF_MEMORY = 4,    /* host or device allocation failed              */
    BSA_ERR_HIP = 5,              /* a HIP runtime call failed (message has it)    */
    BSA_ERR_INTERNAL = 6
};

/* Logical mask kinds. */
enum {
    /* uint8 [B][H][ceil(L/block_q)][ceil(L/block_k)], nonzero = keep the whole
     * block. Block i covers logical positions [i*b, min((i+1)*b, L)).
     * Tessera abstract (blocks selected by a logical mask); FG-Attn
     * (arXiv 2509.16518) abstract (M x M blocks, M = 64 typically). */
    BSA_MASK_BLOCK_U8 = 1,
    /* The same mask as uint64 bit rows [B][H][ceil(L/block_q)][ceil(nkb/64)]:
     * key block j is bit (j % 64) of word j / 64. Bits at j >= nkb must be 0. */
    BSA_MASK_BLOCK_BITS = 2,
    /* M x 1 slices (FG-Attn abstract: each slice is the products of a block of
     * M queries with one key): block_q = M, block_k = 1. row_ptr int64
     * [B*H*ceil(L/M) + 1] (row_ptr[0] = 0, non-decreasing) indexes col_idx
     * int32; each list is strictly increasing and within [0, L). All M
     * queries of a block share the list. */
    BSA_MASK_SLICE_CSR = 3,
    /* Element-exact video patterns on token coordinates, one per head
     * (Sparse VideoGen / Splash Attention summary, "Sparse VideoGen" and
     * "Splash Attention": heads routed to spatial or temporal patterns, exact
     * coordinate masking on boundary tiles). block_q = block_k = 1; needs
     * the video geometry in the options. */
    BSA_MASK_VIDEO = 4
};

/* Per-head video patterns (BSA_MASK_VIDEO). */
enum {
    BSA_PAT_DENSE = 0,    /* every key */
    BSA_PAT_SPATIAL = 1,  /* key in the query's frame, or in the anchor frame     */
    BSA_PAT_TEMPORAL = 2  /* |y_k - y_q| <= radius and |x_k - x_q| <= radius, any frame */
};

/* Per-head token layouts. A temporal-major head (Splash Attention section:
 * token layouts permuted into temporal-major order for the temporal patterns)
 * works on logical position j = p*T + t for the frame-major token
 * i = t*Hg*Wg + p. Its BLOCK and SLICE mask indices are logical positions.
 * The permutation is fused into load and store addressing: tensors stay
 * frame-major in memory. */
enum { BSA_LAYOUT_FRAME_MAJOR = 0, BSA_LAYOUT_TEMPORAL_MAJOR = 1 };

enum { BSA_DTYPE_BF16 = 0, BSA_DTYPE_F32 = 1 };

typedef struct {
    int32_t kind;                  /* BSA_MASK_*                                   */
    const void *data;              /* BLOCK_U8: uint8*, BLOCK_BITS: uint64*        */
    const int64_t *row_ptr;        /* SLICE_CSR                                    */
    const int32_t *col_idx;        /* SLICE_CSR                                    */
    const uint8_t *head_pattern;   /* VIDEO: [H] BSA_PAT_*                         */
    int32_t anchor_frame;          /* VIDEO spatial anchor frame (0 <= a < T)     */
    int32_t radius;                /* VIDEO temporal Chebyshev radius (>= 0)      */
    int64_t nnz;                   /* SLICE_CSR: entries of col_idx; 0 = take
                                      row_ptr's last entry (host masks); required
                                      for device masks (bsa_plan_device)          */
} bsa_mask_desc_t;

typedef struct {
    int32_t dtype;                 /* BSA_DTYPE_*; default bf16                    */
    int32_t T, Hg, Wg;             /* video geometry; T*Hg*Wg must equal L when a
                                      VIDEO mask or a temporal-major head is used;
                                      0 = none                                     */
    const uint8_t *head_layout;    /* [H] BSA_LAYOUT_*; NULL = all frame-major     */
    int32_t force_regime;          /* -1 = choose from the lookup table            */
    const char *lut_path;          /* NULL = the table compiled into the library   */
    int32_t device;                /* HIP device ordinal; -1 = host-only plan for
                                      inspection (bsa_forward rejects it)          */
    int32_t task_order;            /* BSA_ORDER_*; -1 = from the lookup table      */
} bsa_plan_opts_t;

/* Task orders (workgroup i of a launch runs task i). LONGEST_FIRST: tasks by
 * decreasing tile count. XCD_GROUPED: the same, with each run of tasks of
 * similar cost interleaved so that neighbouring query tiles of a head land on
 * one XCD (accelerator die with its own L2; the hardware deals workgroups to
 * the XCDs in turn). */
enum { BSA_ORDER_XCD_GROUPED = 0, BSA_ORDER_LONGEST_FIRST = 1 };

/* Fill *opts with the defaults listed above. */
void bsa_plan_opts_default(bsa_plan_opts_t *opts);

typedef struct {
    int32_t regime;                /* regime id (see bsa_regime_info)              */
    int32_t tile_q, tile_k;        /* physical tile shape                          */
    int32_t gather;                /* 1 if key tiles are gathered row lists        */
    int64_t tasks;                 /* tasks: one per (batch, head, query tile)     */
    int64_t workgroups;            /* launched workgroups (one per task)           */
    int64_t tiles_full;            /* key tiles computed without a mask            */
    int64_t tiles_partial;         /* key tiles with exact masking                 */
    int64_t tiles_empty;           /* (query tile, key tile) pairs skipped         */
    int64_t gather_rows;           /* gathered key rows (gather regimes)           */
    double executed_pairs;         /* tile_q * tile_k per computed tile            */
    int64_t device_bytes;          /* device memory owned by the plan              */
    int64_t plan_ns;               /* wall time of bsa_plan                         */
    int64_t phase_ns[5];           /* of which: ingest/validation, regime lookup,
                                      physical mapping, task organisation, upload */
    int32_t task_order;            /* BSA_ORDER_* the plan uses                    */
    double mask_density;           /* regime-lookup features of the mask: kept
                                      blocks / all blocks (slices: listed keys /
                                      all pairs), and fill = kept pairs / pairs of
                                      the non-empty 128 x 64 tiles (block masks,
                                      from every 4th 128-row query tile); -1 when
                                      the kind has none (video; fill of slices)  */
    double mask_fill;
    double mask_fill2;             /* fill over the non-empty 256 x 64 tiles (the
                                      256-row tiles that start at the sampled
                                      128-row tiles); -1 as mask_fill          */
} bsa_plan_info_t;

typedef struct {
    int32_t family;                /* 0 = contiguous/permuted tiles, 1 = gather    */
    int32_t tile_q, tile_k;
    int32_t waves;                 /* wavefronts per workgroup                     */
    int32_t rows_per_wave;         /* query rows each wavefront owns (32)          */
} bsa_regime_desc_t;

/* One physical tile of a plan, as computed by the device (test hook for
 * checking that a plan covers every kept pair exactly once). Positions are
 * logical positions of the head. A video PARTIAL tile is reported once per
 * wavefront (32 query rows) that computes it, each as FULL or PARTIAL for those
 * rows; wavefronts that keep no pair of the tile skip it and report nothing. */
enum { BSA_TILE_FULL = 0, BSA_TILE_PARTIAL = 1 };
enum { BSA_PRED_NONE = 0, BSA_PRED_SUBBLOCK = 1, BSA_PRED_VIDEO = 2, BSA_PRED_LIST = 3 };
typedef struct {
    int64_t q0, q1;                /* query positions [q0, q1), cropped to L       */
    int32_t kind;                  /* BSA_TILE_*                                   */
    int32_t predicate;             /* what a PARTIAL tile evaluates: BSA_PRED_*    */
    int64_t k0, k1;                /* contiguous keys [k0, k1), cropped to L
                                      (k1 - k0 < tile_k means positions >= L are
                                      masked); unused for lists                  */
    const int32_t *keys;           /* BSA_PRED_LIST: key positions, nkeys of them  */
    int64_t nkeys;
    uint32_t sub_bits;             /* BSA_PRED_SUBBLOCK: keep bit of sub-block
                                      (sq * sub_nk + sk)                           */
    int32_t sub_q, sub_k;          /* sub-block shape; sub_nk = tile_k / sub_k     */
    int64_t task;                  /* the record's task = workgroup index in the
                                      launch                                      */
} bsa_tile_record_t;

/* Return nonzero to stop the walk early. */
typedef int (*bsa_cov_sink_t)(void *user, const bsa_tile_record_t *rec);

int32_t bsa_abi_version(void);

/*
 * Build a plan for `logical_mask` over B x H heads of L tokens, head dim d
 * (64 or 128), logical block shape block_q x block_k (BLOCK kinds: each side a
 * power of two in [32, 1024], else UNSUPPORTED; SLICE: block_q = M in {64, 128}
 * (other M: UNSUPPORTED), block_k = 1; VIDEO: 1 x 1). opts may be NULL
 * (defaults). On success *out_plan receives a new
 * plan; on failure it is set to NULL and nothing is leaked.
 * Errors: INVALID_ARGUMENT (null pointers, shapes, options, geometry),
 * INVALID_MASK (contents), UNSUPPORTED (d, block shape, dtype), OUT_OF_MEMORY,
 * HIP (device selection, allocation or upload failed).
 */
int32_t bsa_plan(const bsa_mask_desc_t *logical_mask, int32_t B, int32_t H, int64_t L, int32_t d,
                 int32_t block_q, int32_t block_k, const bsa_plan_opts_t *opts, bsa_plan_t *out_plan);

/*
 * Build a plan on the device for a BLOCK mask (BLOCK_U8 or BLOCK_BITS) or a
 * SLICE_CSR mask whose arrays are already in DEVICE memory (data, or row_ptr
 * and col_idx, are device pointers of the layouts described above; a SLICE
 * mask needs nnz): the tile mapping and the task order run as kernels on
 * `stream` (a hipStream_t; NULL = the default stream of opts->device), with no
 * copy of the mask to the host (Tessera, arXiv 2609.25869, abstract: dynamic
 * masks, preparation kept cheap; FG-Attn, arXiv 2509.16518, abstract: slices
 * whose keys are gathered). Returns after enqueueing; a bsa_forward on the
 * same stream runs after the planning, one on another stream waits for it.
 * The mask must stay valid until the planning work has run (the plan keeps
 * its own copy of the slice keys). The plan equals the one bsa_plan builds
 * from the same mask, except that BLOCK regimes and orders come from the
 * table's rules that hold for every mask density and fill (the features need
 * the mask on the host), and bits past the last key block of a BLOCK_BITS
 * row are ignored. The host cannot validate a device mask: slice
 * keys outside [0, L) are clamped into it, a list whose row_ptr bounds fall
 * outside [0, nnz] or span more than L keys is taken as empty, and keys that
 * are not strictly increasing are used as given; bsa_plan_info then returns
 * BSA_ERR_INVALID_MASK (after filling its output). Such a plan stays safe to
 * run.
 * Device memory: every task has room for a record per key tile (8 bytes per
 * (task, key tile) pair). bsa_plan_info waits for the planning work and reads
 * back its statistics; bsa_plan_coverage also reads back the task and record
 * arrays. Errors: INVALID_ARGUMENT (as bsa_plan; host-only device -1),
 * UNSUPPORTED (VIDEO masks, 2^31 or more (task, key tile) pairs, 2^24 or
 * more tasks, the longest-first order with more than 8190 key tiles),
 * OUT_OF_MEMORY, HIP.
 */
int32_t bsa_plan_device(const bsa_mask_desc_t *logical_mask, int32_t B, int32_t H, int64_t L, int32_t d,
                        int32_t block_q, int32_t block_k, const bsa_plan_opts_t *opts, void *stream,
                        bsa_plan_t *out_plan);

/*
 * Enqueue the forward pass of `plan` on `stream` (a hipStream_t; NULL = the
 * default stream of the plan's device). Q, K, V, O as described above. Never
 * synchronises and never allocates; returns after the launch. After the
 * launch it records the plan's last-use event on `stream`; a forward on a
 * different stream than the plan's previous forward first makes `stream` wait
 * for that previous forward (so later work on `stream` waits for it too).
 * Launch errors
 * are reported (BSA_ERR_HIP); faults inside the kernel surface at the
 * caller's next synchronisation of the stream.
 * Errors: INVALID_ARGUMENT (null plan or pointer, misaligned pointer, host-only
 * plan), HIP.
 */
int32_t bsa_forward(bsa_plan_t plan, const void *Q, const void *K, const void *V, void *O, void *stream);

/* bsa_forward with clock stamps, for measuring the shader clock the kernel
 * runs at (the rooflines' per-clock rates; it is no step of the method). The
 * output is the same as bsa_forward's. `stamps` is a caller-owned device
 * buffer of 4 * workgroups uint64 (bsa_plan_info: workgroups): thread 0 of
 * workgroup i writes [4i] the shader-clock counter (s_memtime) and [4i+1] the
 * constant 100 MHz counter (s_memrealtime) when its task starts, [4i+2] and
 * [4i+3] the same when it ends; workgroups that run no task (padding of an XCD
 * segment) write nothing. A task's shader clock is 100 MHz x (delta [4i+2] -
 * [4i]) / (delta [4i+3] - [4i+1]). bf16 plans only.
 * Errors: those of bsa_forward; INVALID_ARGUMENT (stamps NULL or not 8-byte
 * aligned), UNSUPPORTED (fp32 plan). */
int32_t bsa_forward_stamped(bsa_plan_t plan, const void *Q, const void *K, const void *V, void *O, uint64_t *stamps,
                            void *stream);

/* Free a plan (NULL is allowed). Blocks until every forward enqueued on the
 * plan has finished (its last-use event), so that no running kernel still
 * reads the plan's device memory when it is handed to the next plan; a plan
 * may therefore be destroyed right after an asynchronous forward. */
void bsa_plan_destroy(bsa_plan_t plan);

/* Statistics of a plan. Errors: INVALID_ARGUMENT. */
int32_t bsa_plan_info(bsa_plan_t plan, bsa_plan_info_t *out);

/* Walk the tiles the device will compute for head (b, h), in task order.
 * Errors: INVALID_ARGUMENT (null plan/sink, b or h out of range). */
int32_t bsa_plan_coverage(bsa_plan_t plan, int32_t b, int32_t h, bsa_cov_sink_t sink, void *user);

/*
 * Requests: a sequence of forward calls over one shape, each with its own
 * mask, pipelined (Tessera, arXiv 2609.25869, abstract: a request runs many
 * dynamic masks, and preparing each must cost little next to running it).
 * bsa_request_submit plans the mask, enqueues its forward on the request's
 * stream and returns, so the planning of the next mask overlaps the forwards
 * already enqueued. At most `depth` plans are alive: a submit that finds
 * `depth` plans in flight first waits for the oldest one's forward and
 * destroys that plan. The request owns its plans. A request is used by one
 * thread at a time.
 */
typedef struct bsa_request_s *bsa_request_t;

typedef struct {
    int32_t B, H;
    int64_t L;
    int32_t d;
    bsa_plan_opts_t opts;   /* for every plan (copied, pointers included); opts.device >= 0 */
    void *stream;           /* forward stream (hipStream_t); NULL = the device's default stream */
    void *plan_stream;      /* stream of device planning (bsa_plan_device); NULL = `stream` */
    int32_t depth;          /* plans alive at most, >= 1 */
} bsa_request_desc_t;

typedef struct {
    int64_t submitted;      /* forwards enqueued */
    int64_t plan_ns;        /* host time spent planning (device planning: enqueueing) */
    int64_t wait_ns;        /* host time spent waiting for a ring slot */
} bsa_request_stats_t;

/* Errors: INVALID_ARGUMENT (null pointers, depth < 1, host-only device,
 * bad shape), OUT_OF_MEMORY, HIP. */
int32_t bsa_request_create(const bsa_request_desc_t *desc, bsa_request_t *out);

/*
 * Plan `mask` (host memory: bsa_plan; mask_on_device = 1: a BLOCK mask in
 * device memory, bsa_plan_device on the request's plan stream, after any work
 * the caller enqueued there) and enqueue the forward on Q, K, V, O (as
 * bsa_forward). Errors: those of bsa_plan / bsa_plan_device / bsa_forward, and
 * HIP; a failed submit leaves the request usable.
 */
int32_t bsa_request_submit(bsa_request_t req, const bsa_mask_desc_t *mask, int32_t block_q, int32_t block_k,
                           int32_t mask_on_device, const void *Q, const void *K, const void *V, void *O);

/* Wait for every forward submitted so far and destroy their plans. Errors: HIP. */
int32_t bsa_request_finish(bsa_request_t req);

/* Errors: INVALID_ARGUMENT. */
int32_t bsa_request_stats(bsa_request_t req, bsa_request_stats_t *out);

/* Finish, then free the request (NULL is allowed). */
void bsa_request_destroy(bsa_request_t req);

/*
 * Head routing (Sparse VideoGen / Splash Attention summary, "Sparse
 * VideoGen": each attention head is routed on the fly to a spatial or a
 * temporal sparse pattern). The pages give no routing rule; this call takes
 * the plain one: for every head, the pattern whose masked attention output is
 * nearer the dense output, measured as the mean squared difference over the
 * batch, the sampled query tokens and the head dimension (ties: spatial). The
 * patterns are those of BSA_MASK_VIDEO (spatial: key in the query's frame or
 * the anchor frame; temporal: key pixel within `radius`, any frame).
 */
typedef struct {
    int32_t T, Hg, Wg;          /* token grid, T*Hg*Wg == L; Hg, Wg < 32768 */
    int32_t anchor_frame;       /* 0 <= anchor_frame < T */
    int32_t radius;             /* 0 .. 256 */
    const int32_t *rows;        /* HOST [n_rows]: sampled query tokens (frame-major), each in [0, L) */
    int32_t n_rows;             /* 1 .. 4096 */
    int32_t device;             /* device of Q, K, V: 0 <= device < device count */
} bsa_route_desc_t;

/*
 * Q, K, V: bf16 DEVICE tensors [B][H][L][d] in frame-major token order, d in
 * {64, 128}. Runs the probe kernels on `stream` (hipStream_t; NULL = the
 * device's default stream) after the work already enqueued there, WAITS for
 * them, and writes head_pattern (HOST [H]: BSA_PAT_SPATIAL or
 * BSA_PAT_TEMPORAL) and, if err is not NULL, err (HOST [H][2]: the spatial and
 * the temporal mean squared difference). Scratch device memory comes from the
 * library's pool. Errors: INVALID_ARGUMENT (null pointers, shapes, geometry,
 * rows out of range, no such device), OUT_OF_MEMORY, HIP.
 */
int32_t bsa_route_heads(const void *Q, const void *K, const void *V, int32_t B, int32_t H, int64_t L, int32_t d,
                        const bsa_route_desc_t *desc, void *stream, uint8_t *head_pattern, double *err);

/*
 * bsa_route_heads for callers that cannot allocate memory: code under graph
 * capture, tight serving loops, harnesses that forbid allocation. Same
 * arguments, checks, errors and results (the per-head sums are formed on the
 * device in the order bsa_route_heads forms them on the host); it allocates
 * nothing and creates no event. Its scratch is a fixed 32 MiB array in each
 * device's memory, held until the process ends and shared by every call on
 * that device: calls on one device are serialized by a host lock, and work
 * that touches the array from calls overlapping on one device by any other
 * means would race. The sampled rows (HOST) are copied to the array and the
 * per-head sums back with stream-ordered copies; the call waits for `stream`
 * before it returns. Limits, each an UNSUPPORTED error: B * H <= 1024, and
 * the rows, the per-row errors (B*H*n_rows*8 bytes) and one key chunk of
 * partial softmax states (B*H*ceil(n_rows/32)*3*(64 + 32 d)*4 bytes) must fit
 * the 32 MiB (at d = 128 and 24 heads: up to 832 sampled rows); within the
 * limit the key range is cut into as many chunks as the array holds.
 */
int32_t bsa_route_heads_noalloc(const void *Q, const void *K, const void *V, int32_t B, int32_t H, int64_t L,
                                int32_t d, const bsa_route_desc_t *desc, void *stream, uint8_t *head_pattern,
                                double *err);

/* Number of execution regimes compiled in, and their shapes. */
int32_t bsa_regime_count(void);
int32_t bsa_regime_info(int32_t regime, bsa_regime_desc_t *out);

const char *bsa_status_str(int32_t status);
const char *bsa_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* BSA_H */
