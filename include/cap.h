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

#define CAP_ABI_VERSION 8

typedef enum cap_status {
    CAP_OK = 0,
    CAP_ERR_INVALID_ARG = 1,   /* NULL pointer, bad option value, size overflow */
    CAP_ERR_BAD_TREE = 2,      /* tree or request paths are malformed */
    CAP_ERR_WORKSPACE = 3,     /* a caller buffer is smaller than required / misaligned */
    CAP_ERR_UNSUPPORTED = 4,   /* shape outside the supported envelope */
    CAP_ERR_HIP = 5,           /* a HIP runtime call or kernel launch failed */
    CAP_ERR_STATE = 6,         /* handle used in the wrong state (e.g. plan not uploaded) */
    CAP_ERR_REPLAN = 7         /* cap_plan_refresh: the plan cannot take the tree's changes in
                                  place; build a new plan with cap_plan_step */
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
                                 (shared items hold at most 128, private at most 256) */
    int32_t shared_rows;      /* 0 = 16: request groups with more query rows than this
                                 (requests x G) are served by shared items (KV staged in
                                 LDS for up to 128 rows); the others by private items (up
                                 to 16 rows, pages split over the 4 waves).  G > 16
                                 always uses shared items */
    int32_t num_cus;          /* 0 = 256 (MI355X); used by the cost model */
    float shared_cost;        /* 0 = 2.0; cost of a shared item's page relative to a
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
    int32_t append_slack;     /* 0 = 8; -1 = none; at most 4096.  Free page-stream entries
                                 reserved after each request's own leaf run, so that
                                 cap_plan_refresh can add that many new leaf pages per
                                 request before a new plan is needed */
    float item_us;            /* 0 = 4.7; < 0 = no item term.  Start cost of one round of
                                 work items (every workgroup slot starting one), in us:
                                 sharing a node adds items, and each is charged this
                                 cost / (2 x num_cus) slots, as bytes of streaming at
                                 7.2 TB/s, against the bytes sharing saves */
    float reread_factor;      /* 0 = 3.0; >= 1.  A folded node's rereads by its sibling
                                 groups cost 1 / reread_factor of fresh HBM bytes: the
                                 siblings run side by side on one XCD and read the node
                                 mostly from its L2 */
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
    double refresh_host_us;       /* host time of the last cap_plan_refresh (0: none yet) */
    int64_t refresh_words;        /* 32-bit words of the plan image it changed */
    int32_t refresh_full_copy;    /* 1 if it sent the whole image instead of a word list */
    int32_t refreshes;            /* cap_plan_refresh calls that changed the plan */
} cap_plan_stats;

typedef struct cap_tree cap_tree;   /* opaque host handles */
typedef struct cap_plan cap_plan;

/* Work item as stored in the plan (exposed for inspection and tests).  Each
 * is run by one 4-wave workgroup: a private item (mode 0) serves up to 16
 * query rows and streams up to 256 pages; a shared item (mode 1) serves up to
 * 128 rows and streams up to 128 pages. */
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
 * that want the table on the GPU (the table as uploaded: cap_tree_append does
 * not update it).  The host arrays may be freed on return.
 * On success *out owns a handle the caller releases with cap_tree_free
 * (after the stream has passed the copy, if one was made).
 * Errors: CAP_ERR_INVALID_ARG (NULL desc/out), CAP_ERR_UNSUPPORTED (shape),
 * CAP_ERR_BAD_TREE (parents, page counts, page ids, paths, empty requests),
 * CAP_ERR_WORKSPACE (dev_bytes too small), CAP_ERR_HIP (copy failed). */
cap_status cap_tree_upload(const cap_attn_desc *attn, const cap_tree_desc *tree,
                           void *dev_buf, size_t dev_bytes, cap_stream_t stream,
                           cap_tree **out);
void cap_tree_free(cap_tree *tree);

/* Host view of the tree as it stands (after any appends), in the form of
 * cap_tree_desc.  The pointers refer to the tree's own arrays and stay valid
 * until the next cap_tree_append or cap_tree_free.  Errors: CAP_ERR_INVALID_ARG. */
cap_status cap_tree_get_desc(const cap_tree *tree, cap_tree_desc *desc);

/* Grow the tree by one decode step: each active request (active[r] != 0;
 * active NULL = every request) gains one context token, the token whose K/V
 * the step produced, at the end of its context.  Where the cache keeps it
 * (the radix-tree KV cache of the Capillary Kernels project page, abstract,
 * first paragraph; the pages give no update rule, so this is the plain one):
 *  - the request's path ends at a leaf that no other request's path passes
 *    through: the leaf grows by one token, into the next slot of its last
 *    page, or into the page new_pages[r] when that page is full or the leaf
 *    has none;
 *  - otherwise (its end node is shared or has children): a new one-token
 *    child of that node holding page new_pages[r] becomes the request's
 *    leaf (node id = the next free id, in request order); the end node and
 *    its pages stay as they are for the other requests.
 * Host-only bookkeeping: no device call.  dest[r] (out, host [R]) receives
 * (physical page << 4) | slot of the new token, or -1 for an inactive
 * request; slot 0 means new_pages[r] was taken, otherwise it is still free.
 * new_pages (host [R]) may be NULL when no request needs a page; each page a
 * request takes must be in [0, num_pool_pages), owned by no node, and not
 * given to two requests.  A new child changes the tree's shape: plans built
 * before it answer cap_plan_refresh with CAP_ERR_REPLAN.  Validation happens
 * before any change.  Errors: CAP_ERR_INVALID_ARG (NULL tree/dest, new_pages
 * needed but NULL), CAP_ERR_BAD_TREE (a new page out of range, owned or given
 * twice), CAP_ERR_UNSUPPORTED (2^26 pages or more). */
cap_status cap_tree_append(cap_tree *tree, const uint8_t *active, const int32_t *new_pages,
                           int32_t *dest);

/* Write the new tokens' K and V into the pools: token i, KV head h goes to
 * page dest[i] >> 4, slot dest[i] & 15 of head h's block (the pool layouts
 * above).  dest: DEVICE int32 [n] (e.g. cap_tree_append's output copied to
 * the GPU); entries < 0 or with a page >= the tree's num_pool_pages are
 * skipped.  k_new, v_new: device bf16 [n][Hkv][D], 16-byte aligned.  One
 * launch on `stream`; n = 0 launches nothing.  Errors: CAP_ERR_INVALID_ARG,
 * CAP_ERR_UNSUPPORTED (n x Hkv x D/8 >= 2^31), CAP_ERR_HIP. */
cap_status cap_append_kv(const cap_tree *tree, const int32_t *dest, int32_t n, const void *k_new,
                         const void *v_new, void *k_pool, void *v_pool, cap_stream_t stream);

/* Per-step planner (host only, no device calls): share/fold decisions per
 * node, KV split lengths, request groups, work-item order, partial slots and
 * the per-request merge lists.  opts may be NULL (defaults).  The plan refers
 * to `tree`, which must outlive it.  Errors: CAP_ERR_INVALID_ARG. */
cap_status cap_plan_step(const cap_tree *tree, const cap_plan_opts *opts, cap_plan **out);

/* Plan again into an existing plan handle: the same plan cap_plan_step would
 * build for `tree` and `opts` (the per-decoding-step cost model of the
 * Capillary Kernels project page, second paragraph, run every step), in the
 * handle's own host memory, so that a loop planning every step allocates
 * nothing once the handle has held a plan of that size.  `tree` may be
 * another tree than the plan's last one.  Host only: the plan afterwards
 * counts as not uploaded (call cap_plan_upload).  Because cap_plan_upload
 * copies from the plan's host memory asynchronously, the stream must have
 * passed the plan's previous upload before this call (e.g. alternate two
 * handles and wait for an event recorded after each one's upload).  Errors:
 * CAP_ERR_INVALID_ARG (NULL plan or tree, bad option; the plan is then
 * unchanged). */
cap_status cap_plan_rebuild(cap_plan *plan, const cap_tree *tree, const cap_plan_opts *opts);
cap_status cap_plan_get_stats(const cap_plan *plan, cap_plan_stats *stats);
cap_status cap_plan_get_view(const cap_plan *plan, cap_plan_view *view);

/* Copy the plan into dev_buf (>= stats.plan_device_bytes, 256-byte aligned)
 * with one asynchronous host-to-device copy.  The plan keeps the host copy
 * alive; free the plan only after the stream has passed this copy.  The
 * buffer ends with counters that the decode kernel updates (the fused
 * step's arrival counters, R x Hkv int32, and the work queues' counters;
 * all zero after the upload and again after every completed launch), so it
 * must stay writable device memory, and launches that use one plan buffer
 * must not overlap (on one stream they never do).  After the counters comes
 * the area cap_plan_refresh stages its patches in.
 * Errors: CAP_ERR_INVALID_ARG, CAP_ERR_WORKSPACE, CAP_ERR_HIP. */
cap_status cap_plan_upload(cap_plan *plan, void *dev_buf, size_t bytes, cap_stream_t stream);

/* Bring the plan up to date with the tree after cap_tree_append, without
 * planning again: each leaf run that serves one request and ends with the
 * pages of that request's own leaf takes the leaf's new token count and new
 * pages (into the free entries reserved after the run, see append_slack);
 * the items of that run stream the longer run, the partial rows stay.  The
 * host plan changes first; if the plan has been uploaded, the changed
 * 32-bit words go to its device buffer on `stream`: one copy of a
 * (word, value) list into the buffer's patch area and one small kernel that
 * applies it (one copy of the whole plan image before the counters, when
 * the list outgrows the area).  Stream-ordered like cap_plan_upload: launches
 * on `stream` after it see the new plan; the list is read from host memory
 * the plan owns, as in cap_plan_upload.  Splits and balance stay those of
 * the plan's own build, so a long-lived plan drifts from what cap_plan_step
 * would choose; callers replan now and then.  Returns CAP_ERR_REPLAN, with
 * nothing changed, when a changed node has no such run (a node shared with
 * other requests, or a leaf folded into a run with others), when a run has
 * no room left (free entries, or the item's page limit: 128 shared, 256
 * private), or when the tree's shape changed (a new node).  Errors:
 * CAP_ERR_INVALID_ARG, CAP_ERR_REPLAN, CAP_ERR_HIP (the device copy is then
 * out of date and the plan counts as not uploaded). */
cap_status cap_plan_refresh(cap_plan *plan, cap_stream_t stream);

/* Launch the decode kernel: every work item streams its KV pages once for
 * all its query rows and writes (m, l, o/l) partials into `workspace`
 * (>= stats.workspace_bytes, 256-byte aligned): m the reference maximum of
 * the base-2-scaled logits (fp32), l the sum of 2^(logit - m) (fp32), o/l the
 * normalised weighted sum of V (|o/l| <= max |v|), kept in fp16.  Layout:
 * o/l [slots][D] fp16, then m [slots], then l [slots], then o/l [slots][D]
 * fp32, each region starting on a 256-byte boundary; slot = partial row x Hq
 * + query head.  The fp32 region is written only for 4-dim groups whose
 * fp16 form is not finite (|o/l| past 65504), so bf16 V of any magnitude in
 * the supported range keeps fp32 range while unit-scale V writes fp16 only.
 * q, k_pool, v_pool: device pointers in the layouts above, 16-byte aligned.
 * Supported values: finite bf16 Q, K, V with sm_scale x |q.k| < 2^120 (fp32
 * logits) and |v| x 2^8 x (context tokens) < 2^127 (fp32 accumulators; e.g.
 * |v| <= 1e30 for contexts of up to 2^20 tokens).  Errors:
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

/* cap_decode_step without a workspace argument, for callers that cannot
 * allocate device memory (code under HIP graph capture, allocation-free
 * serving loops, harnesses that forbid hipMalloc).  The partial workspace is
 * a static device array inside the library, CAP_NOALLOC_WORKSPACE_BYTES
 * (64 MiB) per GPU, held from the library's first use on that GPU until the
 * process ends; this call allocates nothing.  Same kernels, arguments and
 * result as cap_decode_step.  Every call on one GPU shares that GPU's array
 * (whose contents persist between calls; nothing in it needs to start at
 * zero): calls that overlap on one GPU race, so serialise them (one stream,
 * or events).  Errors: as cap_decode_step, and CAP_ERR_UNSUPPORTED when the
 * plan's stats.workspace_bytes exceeds CAP_NOALLOC_WORKSPACE_BYTES (nothing
 * launched). */
#define CAP_NOALLOC_WORKSPACE_BYTES (64u << 20)
cap_status cap_decode_step_noalloc(const cap_plan *plan, const void *q, const void *k_pool,
                                   const void *v_pool, void *out, cap_stream_t stream);

void cap_plan_free(cap_plan *plan);

#ifdef __cplusplus
}
#endif
#endif /* CAP_H */
