/*
 * cap.h -- C ABI of libcap: single-step decode attention over a paged
 * radix-tree KV cache on AMD MI355X (gfx950), where every request under a
 * tree node is served by one stream of that node's KV per step.
 *
 * Source of the operation: the Capillary Kernels project page (abstract,
 * first paragraph) states the problem -- a radix-tree KV cache lets decode
 * requests reuse common context prefixes, yet conventional attention kernels
 * load each request's KV tiles independently, so shared prefixes are fetched
 * again and again.  Its second paragraph gives the three ingredients this ABI
 * exposes as separate calls: a per-decoding-step cost model that picks the
 * query grouping (cap_plan_step), an attention kernel in which work that
 * shares a KV prefix reads it once and emits partial attention results
 * (cap_decode_attention), and the combination of those partial results
 * (cap_merge_partials).  The page gives no formula; the attention computed
 * is standard scaled-dot-product softmax attention of each request's one
 * decode query over its whole root-to-leaf context (no mask, no bias).
 *
 * Conventions for every call:
 *  - Plain C; no exceptions cross the boundary.  The return code is the only
 *    error channel; cap_last_error() gives a human-readable message for the
 *    last failure on the calling thread.
 *  - A call that fails validation has no side effects (nothing launched,
 *    nothing copied, no handle created).
 *  - The library never allocates device memory and never synchronises the
 *    device.  The caller owns every device buffer and passes raw device
 *    pointers plus a stream (a hipStream_t; NULL = the null stream).  The
 *    library owns only its host-side handles.
 *  - Launch failures map to CAP_ERR_HIP; device faults surface at the
 *    caller's next synchronisation.
 *
 * Data layouts (all bf16 values are IEEE bfloat16 bit patterns):
 *  - Page size P = 16 tokens.  Every tree node starts on a fresh page and
 *    owns ceil(tokens/16) pages; its last page may be partial.  Slots past a
 *    node's last token are never read into the result (they may hold NaN).
 *  - K pool: bf16 [num_pool_pages][Hkv][D/8][P][8].  Within one
 *    (page, KV head) block, token slot t, dim d is at ((d/8)*P + t)*8 + d%8.
 *  - V pool: bf16 [num_pool_pages][Hkv][D][P].  Within one block, (t, d) is
 *    at d*P + t (tokens contiguous for each dim).
 *  - q:   bf16 [R][Hq][D], request-major, in the tree's request order.
 *  - out: bf16 [R][Hq][D], rounded to nearest-even from fp32.
 *  - Query head h reads KV head h / (Hq/Hkv).
 */
#ifndef CAP_H
#define CAP_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define CAP_ABI_VERSION 5

typedef enum cap_status {
    CAP_OK = 0,
    CAP_ERR_INVALID_ARG = 1,   /* NULL pointer, bad option value, size overflow */
    CAP_ERR_BAD_TREE = 2,      /* tree or request paths are malformed */
    CAP_ERR_WORKSPACE = 3,     /* a caller buffer is smaller than required / misaligned */
    CAP_ERR_UNSUPPORTED = 4,   /* shape outside the supported envelope */
    CAP_ERR_HIP = 5,           /* a HIP runtime call or kernel launch failed */
    CAP_ERR_STATE = 6          /* handle used in the wrong state (e.g. plan not uploaded) */
} cap_status;

/* A hipStream_t, passed through untouched. */
typedef void *cap_stream_t;

/* Attention shape.  Supported: head_dim in {64, 128}; page_size == 16;
 * num_q_heads % num_kv_heads == 0 with G = num_q_heads / num_kv_heads in
 * {1, 2, 4, 8, 16, 32}; sm_scale finite and > 0 (usually 1/sqrt(head_dim)). */
typedef struct cap_attn_desc {
    int32_t num_q_heads;
    int32_t num_kv_heads;
    int32_t head_dim;
    int32_t page_size;
    float sm_scale;
} cap_attn_desc;

/* Paged radix tree and request paths.  All pointers are HOST pointers; the
 * arrays are copied during cap_tree_upload and may be freed after it returns.
 *  parent[N]          parent node id, -1 for a root; parent[i] < i.
 *  num_tokens[N]      tokens held by node i (>= 0; 0 allowed, e.g. a sentinel root).
 *  page_offsets[N+1]  CSR into page_ids; node i owns exactly ceil(num_tokens[i]/16)
 *                     pages page_ids[page_offsets[i] .. page_offsets[i+1]).
 *  page_ids[..]       physical page indices into the K/V pools, each in
 *                     [0, num_pool_pages), no page owned twice.
 *  num_pool_pages     pages in the pools, at most 2^26 (CAP_ERR_UNSUPPORTED
 *                     above: a plan packs page id and token count in 32 bits).
 *  path_offsets[R+1]  CSR into path_nodes; request r's path runs from a root
 *                     down to the node where its context ends; consecutive
 *                     entries are parent and child.  Every request must have
 *                     at least one context token.  Several requests may share
 *                     a path or end at an internal node. */
typedef struct cap_tree_desc {
    int32_t num_nodes;
    const int32_t *parent;
    const int32_t *num_tokens;
    const int64_t *page_offsets;
    const int32_t *page_ids;
    int32_t num_requests;
    const int32_t *path_offsets;
    const int32_t *path_nodes;
    int64_t num_pool_pages;
} cap_tree_desc;

/* Planner options.  Zero-initialise for defaults (then set what you need);
 * cap_plan_opts_default() fills the defaults explicitly. */
typedef struct cap_plan_opts {
    int32_t share_mode;       /* -1 auto (cost model), 0 fold all (unshared baseline:
                                 every request streams its whole context), 1 share
                                 every non-empty node, 2 auto (same as -1) */
    int32_t split_pages;      /* 0 auto; else the most KV pages one work item streams
                                 (shared items hold at most 64, private at most 256) */
    int32_t shared_rows;      /* 0 = 16: request groups with more query rows than this
                                 (requests x G) are served by shared items (KV staged in
                                 LDS for up to 128 rows); the others by private items (up
                                 to 16 rows, pages split over the 4 waves).  G > 16
                                 always uses shared items */
    int32_t num_cus;          /* 0 = 256 (MI355X); used by the cost model */
    float shared_cost;        /* 0 = 1.5; cost of a shared item's page relative to a
                                 private item's page, used to size items */
    float rounds;             /* 0 = 1.5; target work items per CU (two run at once) */
    float share_margin;       /* 0 = 1.0; share a node only if saved bytes exceed
                                 margin x added partial bytes */
    int32_t order;            /* dispatch order of the work items (workgroups start in
                                 item order as CUs free up): 0 = default (2); 1 = the
                                 two item kinds interleaved evenly, each costliest
                                 first; 2 = costliest first over both kinds; 3 = all
                                 shared items first, then private ones costliest first;
                                 4 = one shared and one private workgroup per CU first
                                 (num_cus of each kind), then as 1 */
    float private_rounds;     /* 0 = 1.0; like `rounds`, but sizes the private items only
                                 (splitting a private run adds one request's partial
                                 rows, splitting a shared one adds a whole group's) */
    float tail_factor;        /* 0 = 1.0; with order 2, cut private items so that none
                                 costs more than the work still to be dispatched per
                                 workgroup slot / tail_factor (the last items to start
                                 are short, so the slots finish together); a huge value
                                 (>= 1e30) turns the cuts off */
    int32_t tail_min_pages;   /* 0 = 16; smallest private piece such a cut leaves */
    int32_t item_dispatch;    /* 0 = one workgroup per item, started by the hardware
                                 in item order (each bound to one shader engine, so a
                                 free slot can wait for a busy engine); 1 = work
                                 queues: two resident workgroups per CU take items as
                                 they finish, workgroup b from queue b mod 8 (items
                                 congruent to it mod 8, in item order), through
                                 counters in the plan buffer.  Both read the same
                                 bytes; with the memory system saturated neither is
                                 faster on the measured trees, 0 by a little */
} cap_plan_opts;

/* Plan summary (host-side numbers; bytes are per decode step). */
typedef struct cap_plan_stats {
    int64_t num_items;            /* work items (one 4-wave workgroup each) */
    int64_t num_shared_items;     /* ... of which shared items */
    int64_t num_tasks;            /* (page run, request group) pairs; items = tasks x Hkv */
    int64_t num_groups;           /* request groups after share/fold decisions */
    int64_t partial_rows;         /* partial slots = partial_rows x Hq */
    int64_t workspace_bytes;      /* required partial workspace */
    int64_t plan_device_bytes;    /* required plan device buffer */
    int64_t tree_device_bytes;    /* device page table size */
    int64_t kv_bytes_streamed;    /* K+V bytes the items read (pages x row groups x heads) */
    int64_t kv_bytes_unique;      /* K+V bytes of the tree's tokens (each once) */
    int64_t kv_bytes_unshared;    /* K+V bytes if every request read its own context */
    int64_t partial_bytes;        /* partial bytes written (= read by the merge) */
    int32_t max_partials_per_request;
    int32_t max_pages_per_item;
    double plan_host_us;          /* host time spent in cap_plan_step */
} cap_plan_stats;

typedef struct cap_tree cap_tree;   /* opaque host handles */
typedef struct cap_plan cap_plan;

/* Work item as stored in the plan (exposed for inspection and tests).  Each
 * is run by one 4-wave workgroup: a private item (mode 0) serves up to 16
 * query rows and streams up to 256 pages; a shared item (mode 1) serves up to
 * 128 rows and streams up to 64 pages. */
typedef struct cap_work_item {
    int32_t stream_off;   /* first entry of its page run in the plan's page stream */
    int32_t npages;       /* pages in the run */
    int32_t head;         /* KV head */
    int32_t row_off;      /* first entry of its request list in the plan's row table */
    int32_t nreq;         /* requests served; query rows = nreq x G */
    int32_t slot_base;    /* first entry of its requests' partial rows in the plan's
                             slot-row table (request position q: slot_rows[slot_base + q]) */
    int32_t mode;         /* 0 private, 1 shared */
    int32_t reserved;
} cap_work_item;

/* Read-only host view of a plan (pointers valid until cap_plan_free).
 * Page-stream entry e: physical pool page = e >> 5 (resolved from the tree's
 * page table when the plan is built), valid tokens = (e & 31) + 1.
 * Partial slot of item row i (request position i/G, query head head*G + i%G):
 *   slot_rows[slot_base + i/G] * Hq + head*G + i%G.
 * Request r's partial rows are the block merge_off[r] .. merge_off[r+1] - 1
 * (each row written by exactly one item per KV head). */
typedef struct cap_plan_view {
    int32_t num_items;         const cap_work_item *items;
    int32_t stream_len;        const int32_t *stream;
    int32_t rows_len;          const int32_t *rows;
    int32_t num_requests;      const int32_t *merge_off;
    int32_t slot_rows_len;     const int32_t *slot_rows;
} cap_plan_view;

int32_t cap_abi_version(void);
const char *cap_last_error(void);
void cap_plan_opts_default(cap_plan_opts *opts);

/* Bytes of device memory the tree's page table needs (4 x total pages, >= 256). */
cap_status cap_tree_device_bytes(const cap_attn_desc *attn, const cap_tree_desc *tree,
                                 size_t *bytes);

/* Validate the tree and derive node->requests lists and context lengths.
 * Plans built from the tree carry the physical page ids they stream, so the
 * kernels never read the tree's page table; dev_buf is optional (may be NULL)
 * and, when given (>= cap_tree_device_bytes, 16-byte aligned), receives a
 * device copy of page_ids with one asynchronous copy on `stream` for callers
 * that want the table on the GPU.  The host arrays may be freed on return.
 * On success *out owns a handle the caller releases with cap_tree_free
 * (after the stream has passed the copy, if one was made).
 * Errors: CAP_ERR_INVALID_ARG (NULL desc/out), CAP_ERR_UNSUPPORTED (shape),
 * CAP_ERR_BAD_TREE (parents, page counts, page ids, paths, empty requests),
 * CAP_ERR_WORKSPACE (dev_bytes too small), CAP_ERR_HIP (copy failed). */
cap_status cap_tree_upload(const cap_attn_desc *attn, const cap_tree_desc *tree,
                           void *dev_buf, size_t dev_bytes, cap_stream_t stream,
                           cap_tree **out);
void cap_tree_free(cap_tree *tree);

/* Per-step planner (host only, no device calls): share/fold decisions per
 * node, KV split lengths, request groups, work-item order, partial slots and
 * the per-request merge lists.  opts may be NULL (defaults).  The plan refers
 * to `tree`, which must outlive it.  Errors: CAP_ERR_INVALID_ARG. */
cap_status cap_plan_step(const cap_tree *tree, const cap_plan_opts *opts, cap_plan **out);
cap_status cap_plan_get_stats(const cap_plan *plan, cap_plan_stats *stats);
cap_status cap_plan_get_view(const cap_plan *plan, cap_plan_view *view);

/* Copy the plan into dev_buf (>= stats.plan_device_bytes, 256-byte aligned)
 * with one asynchronous host-to-device copy.  The plan keeps the host copy
 * alive; free the plan only after the stream has passed this copy.  The
 * buffer ends with counters that the decode kernel updates (the fused
 * step's arrival counters, R x Hkv int32, and the work queues' counters;
 * all zero after the upload and again after every completed launch), so it
 * must stay writable device memory, and launches that use one plan buffer
 * must not overlap (on one stream they never do).
 * Errors: CAP_ERR_INVALID_ARG, CAP_ERR_WORKSPACE, CAP_ERR_HIP. */
cap_status cap_plan_upload(cap_plan *plan, void *dev_buf, size_t bytes, cap_stream_t stream);

/* Launch the decode kernel: every work item streams its KV pages once for
 * all its query rows and writes (m, l, o/l) partials into `workspace`
 * (>= stats.workspace_bytes, 256-byte aligned): m the reference maximum of
 * the base-2-scaled logits (fp32), l the sum of 2^(logit - m) (fp32), o/l the
 * normalised weighted sum of V (fp16, |o/l| <= max |v|).  Layout: o/l
 * [slots][D] fp16, then m [slots], then l [slots], each region starting on a
 * 256-byte boundary; slot = partial row x Hq + query head.  q, k_pool, v_pool: device
 * pointers in the layouts above, 16-byte aligned.  Errors:
 * CAP_ERR_INVALID_ARG, CAP_ERR_WORKSPACE, CAP_ERR_STATE (plan not uploaded),
 * CAP_ERR_HIP. */
cap_status cap_decode_attention(const cap_plan *plan, const void *q, const void *k_pool,
                                const void *v_pool, void *workspace, size_t ws_bytes,
                                cap_stream_t stream);

/* Launch the merge kernel: for each (request, query head) combine its
 * partials with log-sum-exp rescaling and write bf16 `out`.  Must follow
 * cap_decode_attention on the same stream with the same workspace.
 * Errors: as cap_decode_attention. */
cap_status cap_merge_partials(const cap_plan *plan, const void *workspace, size_t ws_bytes,
                              void *out, cap_stream_t stream);
/* The whole step in one launch: the decode kernel of cap_decode_attention,
 * with the merge of cap_merge_partials done inside it.  Each work item, once
 * its partials are written, counts itself in on a per-(request, KV head)
 * counter in the plan buffer; the item that brings a request's count to its
 * number of partials merges that request's G query heads with the same
 * log-sum-exp combination (Capillary Kernels project page, second paragraph:
 * partial results of one request are reduced into one output) and writes
 * its rows of bf16 `out` [R][Hq][D] (16-byte aligned), then resets the
 * counter.  workspace: as cap_decode_attention; its contents afterwards are
 * unspecified.  Steps that share a plan buffer must not overlap (counters).
 * Errors: as cap_decode_attention, CAP_ERR_INVALID_ARG for a NULL or
 * misaligned `out`, CAP_ERR_UNSUPPORTED when the partial o region
 * (stats.partial_rows x Hq x D x 2 bytes) reaches 2 GiB (32-bit buffer
 * offsets; the two-call form has no such limit). */
cap_status cap_decode_step(const cap_plan *plan, const void *q, const void *k_pool,
                           const void *v_pool, void *workspace, size_t ws_bytes, void *out,
                           cap_stream_t stream);
void cap_plan_free(cap_plan *plan);

#ifdef __cplusplus
}
#endif
#endif /* CAP_H */
