// cap_host.cpp -- host side of libcap: tree validation and upload, the
// per-step planner, and the C ABI entry points declared in include/cap.h.
//
// The planner is this library's counterpart of the per-decoding-step cost
// model on the Capillary Kernels project page (abstract, second paragraph),
// which picks query grouping so that saved HBM traffic pays for the cost of
// cooperating.  On CDNA4 the cooperation cost is the (m, l, o) partial
// traffic through global memory, so each tree node is either
//   * shared: its pages (plus any folded ancestors') are streamed once per
//     KV head for all requests below it, split into page runs that each
//     write one partial per query row, or
//   * folded: its pages ride along as a prefix of each child's run, read
//     again by every child group but adding no partials of its own.
// A node is shared when the bytes it saves, (groups below - 1) x its bytes,
// exceed `share_margin` x the partial bytes sharing adds (cf. the CREDIT
// summary, section III.B "Traffic Model": the saving is the removed reread
// bytes, while fixed traffic stays).  Runs are sized so that the work items
// fill the GPU's resident wave slots about `rounds` times (cf. CREDIT
// section III.D "Occupancy": the wave count enters the execution time).
#include <hip/hip_runtime.h>

#include <algorithm>
#include <chrono>
#include <cmath>
#include <cstddef>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <limits>
#include <new>
#include <string>
#include <vector>

#include "../../include/cap_bench.h"
#include "../../include/cap_rows.h"
#include "cap_internal.h"

using cap::WorkItem;

namespace {

thread_local std::string g_err;

cap_status fail(cap_status st, const char *fmt, ...)
{
    char buf[512];
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(buf, sizeof buf, fmt, ap);
    va_end(ap);
    g_err = buf;
    return st;
}

constexpr size_t kAlign = 256;
constexpr int64_t kMaxPoolPages = (int64_t)1 << 26;   // page-stream entry: (page << 5) | (ntok - 1)
size_t align_up(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }

}  // namespace

struct cap_tree {
    cap_attn_desc attn{};
    int32_t N = 0, R = 0, G = 0;
    std::vector<int32_t> parent, ntok;
    std::vector<int64_t> page_off;
    std::vector<int32_t> page_ids;
    std::vector<int32_t> path_off, path_nodes;
    int64_t num_pool_pages = 0;
    // derived
    std::vector<std::vector<int32_t>> children;
    std::vector<int32_t> req_off, req_list;   // requests whose path contains node (sorted)
    std::vector<int32_t> end_off, end_list;   // requests whose path ends at node
    std::vector<int64_t> ctx_len;
    int64_t unique_tokens = 0, sum_ctx = 0;
    const int32_t *dev_pages = nullptr;       // device copy of page_ids as uploaded (may be null)
    // mutation state
    int64_t shape_gen = 0;                    // bumped when nodes or request paths change
    std::vector<uint64_t> owned;              // bitmap of pool pages held by a node (built on first append)
};

struct cap_plan {
    const cap_tree *tree = nullptr;
    cap_plan_stats stats{};
    std::vector<WorkItem> items;          // one workgroup each
    std::vector<int32_t> stream;      // (physical page << 5) | (ntok - 1)
    std::vector<int32_t> rows;        // request ids
    std::vector<int32_t> merge_off;   // request r's partial rows: merge_off[r] .. merge_off[r+1] - 1
    std::vector<int32_t> slot_rows;   // partial row of each (task, request) pair, by task
    // device image
    size_t off_items = 0, off_stream = 0, off_rows = 0, off_moff = 0, off_srows = 0, off_cnt = 0, off_queue = 0,
           dev_bytes = 0;
    bool work_queue = false;          // item_dispatch 1
    std::vector<unsigned char> host_image;
    void *dev = nullptr;
    // growth in place (cap_plan_refresh): per request, the leaf run that
    // ends with the pages of the node its context ends at
    struct Leaf {
        int32_t node = -1;            // -1: no run the plan can extend
        int32_t pages = 0;            // the node's pages as the plan holds them
        int32_t end = 0;              // stream index one past the run's last entry
        int32_t limit = 0;            // one past the free entries reserved after it
        int32_t item0 = 0;            // first of the Hkv items whose page run ends at `end`
    };
    std::vector<Leaf> leaf;
    std::vector<int32_t> node_tokens; // the tree's token counts the plan holds
    int64_t shape_gen = 0;
    size_t off_patch = 0, patch_cap = 0;   // patch area: patch_cap (word, value) pairs
    std::vector<uint32_t> patch;
};

namespace {

cap_status check_attn(const cap_attn_desc *a)
{
    if (!a) return fail(CAP_ERR_INVALID_ARG, "attn desc is NULL");
    if (a->num_q_heads <= 0 || a->num_kv_heads <= 0)
        return fail(CAP_ERR_UNSUPPORTED, "head counts must be positive (Hq=%d, Hkv=%d)",
                    a->num_q_heads, a->num_kv_heads);
    if (a->num_q_heads % a->num_kv_heads != 0)
        return fail(CAP_ERR_UNSUPPORTED, "Hq=%d is not a multiple of Hkv=%d", a->num_q_heads,
                    a->num_kv_heads);
    const int G = a->num_q_heads / a->num_kv_heads;
    if (G > cap::kRowsPerItem || cap::kRowsPerItem % G != 0)
        return fail(CAP_ERR_UNSUPPORTED, "GQA group size %d not in {1,2,4,8,16,32}", G);
    if (a->head_dim != 64 && a->head_dim != 128)
        return fail(CAP_ERR_UNSUPPORTED, "head_dim %d not in {64, 128}", a->head_dim);
    if (a->page_size != cap::kPage)
        return fail(CAP_ERR_UNSUPPORTED, "page_size %d != 16", a->page_size);
    if (!(a->sm_scale > 0.f) || !std::isfinite(a->sm_scale))
        return fail(CAP_ERR_INVALID_ARG, "sm_scale must be finite and > 0");
    return CAP_OK;
}

// Tables derived from parent, ntok and the request paths: children,
// node -> requests (passing through / ending at), context lengths and totals.
void derive(cap_tree &t)
{
    const int N = t.N, R = t.R;
    t.children.assign(N, {});
    for (int i = 0; i < N; ++i)
        if (t.parent[i] >= 0) t.children[t.parent[i]].push_back(i);
    std::vector<std::vector<int32_t>> under(N), ends(N);
    t.ctx_len.assign(R, 0);
    for (int r = 0; r < R; ++r) {
        for (int j = t.path_off[r]; j < t.path_off[r + 1]; ++j) {
            under[t.path_nodes[j]].push_back(r);
            t.ctx_len[r] += t.ntok[t.path_nodes[j]];
        }
        ends[t.path_nodes[t.path_off[r + 1] - 1]].push_back(r);
    }
    t.req_off.assign(N + 1, 0);
    t.end_off.assign(N + 1, 0);
    t.req_list.clear();
    t.end_list.clear();
    t.unique_tokens = 0;
    t.sum_ctx = 0;
    for (int i = 0; i < N; ++i) {
        t.req_off[i + 1] = t.req_off[i] + (int32_t)under[i].size();
        t.end_off[i + 1] = t.end_off[i] + (int32_t)ends[i].size();
        t.req_list.insert(t.req_list.end(), under[i].begin(), under[i].end());
        t.end_list.insert(t.end_list.end(), ends[i].begin(), ends[i].end());
        t.unique_tokens += t.ntok[i];
    }
    for (int r = 0; r < R; ++r) t.sum_ctx += t.ctx_len[r];
}

// Validate and copy the description into a new tree object (host only).
cap_status build_tree(const cap_attn_desc *attn, const cap_tree_desc *d, cap_tree **out)
{
    cap_status st = check_attn(attn);
    if (st != CAP_OK) return st;
    if (!d) return fail(CAP_ERR_INVALID_ARG, "tree desc is NULL");
    const int N = d->num_nodes, R = d->num_requests;
    if (N <= 0) return fail(CAP_ERR_BAD_TREE, "num_nodes must be > 0");
    if (R <= 0) return fail(CAP_ERR_BAD_TREE, "num_requests must be > 0");
    if (!d->parent || !d->num_tokens || !d->page_offsets || !d->path_offsets || !d->path_nodes)
        return fail(CAP_ERR_INVALID_ARG, "a tree array pointer is NULL");
    if (d->num_pool_pages <= 0)
        return fail(CAP_ERR_BAD_TREE, "num_pool_pages %lld out of range",
                    (long long)d->num_pool_pages);
    if (d->num_pool_pages > kMaxPoolPages)
        return fail(CAP_ERR_UNSUPPORTED, "num_pool_pages %lld above the limit of %lld (page ids share an "
                    "int32 with the token count)", (long long)d->num_pool_pages, (long long)kMaxPoolPages);
    if (d->page_offsets[0] != 0) return fail(CAP_ERR_BAD_TREE, "page_offsets[0] != 0");
    for (int i = 0; i < N; ++i) {
        const int p = d->parent[i];
        if (p < -1 || p >= i)
            return fail(CAP_ERR_BAD_TREE, "node %d: parent %d must be -1 or a smaller node id", i, p);
        if (d->num_tokens[i] < 0) return fail(CAP_ERR_BAD_TREE, "node %d: negative token count", i);
        const int64_t want = (d->num_tokens[i] + cap::kPage - 1) / cap::kPage;
        const int64_t have = d->page_offsets[i + 1] - d->page_offsets[i];
        if (have != want)
            return fail(CAP_ERR_BAD_TREE, "node %d: %lld pages for %d tokens (need %lld)", i,
                        (long long)have, d->num_tokens[i], (long long)want);
    }
    const int64_t total_pages = d->page_offsets[N];
    if (total_pages >= (int64_t(1) << 26))
        return fail(CAP_ERR_UNSUPPORTED, "tree has %lld pages (limit 2^26)", (long long)total_pages);
    if (total_pages > 0 && !d->page_ids) return fail(CAP_ERR_INVALID_ARG, "page_ids is NULL");
    {
        std::vector<int32_t> ids(d->page_ids, d->page_ids + total_pages);
        for (int64_t i = 0; i < total_pages; ++i)
            if (ids[i] < 0 || ids[i] >= d->num_pool_pages)
                return fail(CAP_ERR_BAD_TREE, "page_ids[%lld] = %d outside the pool of %lld pages",
                            (long long)i, ids[i], (long long)d->num_pool_pages);
        std::sort(ids.begin(), ids.end());
        for (int64_t i = 1; i < total_pages; ++i)
            if (ids[i] == ids[i - 1])
                return fail(CAP_ERR_BAD_TREE, "physical page %d is owned twice", ids[i]);
    }
    if (d->path_offsets[0] != 0) return fail(CAP_ERR_BAD_TREE, "path_offsets[0] != 0");
    std::vector<int64_t> ctx(R, 0);
    for (int r = 0; r < R; ++r) {
        const int b = d->path_offsets[r], e = d->path_offsets[r + 1];
        if (e <= b) return fail(CAP_ERR_BAD_TREE, "request %d has an empty path", r);
        for (int j = b; j < e; ++j) {
            const int nd = d->path_nodes[j];
            if (nd < 0 || nd >= N) return fail(CAP_ERR_BAD_TREE, "request %d: node %d out of range", r, nd);
            if (j == b && d->parent[nd] != -1)
                return fail(CAP_ERR_BAD_TREE, "request %d: path starts at node %d, not a root", r, nd);
            if (j > b && d->parent[nd] != d->path_nodes[j - 1])
                return fail(CAP_ERR_BAD_TREE, "request %d: node %d does not follow its parent", r, nd);
            ctx[r] += d->num_tokens[nd];
        }
        if (ctx[r] == 0) return fail(CAP_ERR_BAD_TREE, "request %d has no context tokens", r);
    }

    cap_tree *t = new (std::nothrow) cap_tree();
    if (!t) return fail(CAP_ERR_INVALID_ARG, "out of host memory");
    t->attn = *attn;
    t->N = N;
    t->R = R;
    t->G = attn->num_q_heads / attn->num_kv_heads;
    t->parent.assign(d->parent, d->parent + N);
    t->ntok.assign(d->num_tokens, d->num_tokens + N);
    t->page_off.assign(d->page_offsets, d->page_offsets + N + 1);
    t->page_ids.assign(d->page_ids, d->page_ids + total_pages);
    t->path_off.assign(d->path_offsets, d->path_offsets + R + 1);
    t->path_nodes.assign(d->path_nodes + 0, d->path_nodes + d->path_offsets[R]);
    t->num_pool_pages = d->num_pool_pages;
    derive(*t);
    *out = t;
    return CAP_OK;
}

// ------------------------------------------------------------------ planner

// Device form of a work item: the item, its requests' first id when they are
// consecutive, and the stream entries of its first pages, split over the
// waves as the decode kernel splits a private item's steps.
cap::DevItem dev_item(const cap_plan &p, const WorkItem &w)
{
    cap::DevItem d{};
    d.stream_off = w.stream_off;
    d.npages = w.npages;
    d.head = w.head;
    d.row_off = w.row_off;
    d.nreq = w.nreq;
    d.slot_base = w.slot_base;
    d.mode = w.mode;
    bool consecutive = true;
    for (int q = 1; q < w.nreq; ++q) consecutive &= p.rows[w.row_off + q] == p.rows[w.row_off] + q;
    d.req0 = consecutive ? p.rows[w.row_off] : -1;
    const int32_t *e = p.stream.data() + w.stream_off;
    if (w.mode == cap::kModeShared) {
        for (int j = 0; j < cap::kInlineEntries && j < w.npages; ++j) d.ent[j] = e[j];
    } else {
        const int nsteps = (w.npages + 1) >> 1;
        for (int wv = 0; wv < cap::kWaves; ++wv) {
            const int first = 2 * (nsteps * wv / cap::kWaves);
            const int count = std::min(w.npages, 2 * (nsteps * (wv + 1) / cap::kWaves)) - first;
            for (int j = 0; j < cap::kInlinePerWave && j < count; ++j)
                d.ent[cap::kInlinePerWave * wv + j] = e[first + j];
        }
    }
    return d;
}

struct Group {
    std::vector<int32_t> reqs;     // sorted request ids
    std::vector<int32_t> entries;  // page-stream entries
    int32_t at = -1;               // node whose pages end the entries (the walk emitted it there)
};

struct Planner {
    const cap_tree &t;
    cap_plan_opts o;
    int D, Hkv, G;
    int64_t head_tok_bytes;        // K+V bytes per token per KV head
    int64_t partial_row_bytes;     // partial bytes per query row (o, m, l)
    double unit = 0;               // target cost of one shared work item (cost units)
    double unit_private = 0;       // ... of one private work item
    int max_pages = 0;             // largest page run of any item
    std::vector<Group> groups;

    Planner(const cap_tree &tree, const cap_plan_opts &opts) : t(tree), o(opts)
    {
        D = t.attn.head_dim;
        Hkv = t.attn.num_kv_heads;
        G = t.G;
        head_tok_bytes = 4LL * D;
        partial_row_bytes = 2LL * D + 8;
    }

    void node_entries(int n, std::vector<int32_t> &out) const
    {
        const int64_t np = t.page_off[n + 1] - t.page_off[n];
        for (int64_t p = 0; p < np; ++p) {
            const int64_t left = t.ntok[n] - p * cap::kPage;
            const int nt = (int)std::min<int64_t>(cap::kPage, left);
            out.push_back((int32_t)(((int64_t)t.page_ids[t.page_off[n] + p] << 5) | (nt - 1)));
        }
    }

    // Groups wider than the threshold run as shared workgroup items (up to
    // 256 rows each), the rest as private one-wave items (up to 16 rows).
    bool is_shared(int64_t nreq) const
    {
        return G > cap::kPrivateRows || nreq * G > o.shared_rows;
    }
    int reqs_per_item(int64_t nreq) const
    {
        return is_shared(nreq) ? cap::kSharedRows / G : cap::kPrivateRows / G;
    }

    // Cost of streaming `pages` pages for one item, in private-page units: a
    // shared item also runs the MFMA/softmax work of up to 256 rows, which
    // makes its pages dearer (o.shared_cost).
    double page_cost(bool shared) const { return shared ? (double)o.shared_cost : 1.0; }

    // Page runs of `pages` pages for a group, split so each item costs about
    // `unit` and fits the kernel's page-table limits.
    int64_t chunks(int64_t pages, bool shared) const
    {
        const int64_t cap = shared ? cap::kMaxSharedPages : cap::kMaxPrivatePages;
        int64_t k = (pages + cap - 1) / cap;
        if (o.split_pages > 0) {
            k = std::max<int64_t>(k, (pages + o.split_pages - 1) / o.split_pages);
        } else if (unit > 0) {
            const double u = shared ? unit : unit_private;
            k = std::max<int64_t>(k, (int64_t)std::ceil(pages * page_cost(shared) / u));
        }
        return std::max<int64_t>(1, std::min<int64_t>(k, pages));
    }

    int64_t estimate_chunks(int64_t pages) const { return chunks(pages, true); }

    bool decide_share(int n, int64_t prefix_tokens) const
    {
        if (o.share_mode == 1) return t.ntok[n] > 0 || prefix_tokens > 0;
        if (o.share_mode == 0) return false;
        const int64_t below = (int64_t)t.children[n].size() + (t.end_off[n + 1] > t.end_off[n] ? 1 : 0);
        if (below <= 1) return false;                 // a chain: folding costs nothing
        const int64_t tok = t.ntok[n] + prefix_tokens;
        if (tok == 0) return false;
        const int64_t nreq = t.req_off[n + 1] - t.req_off[n];
        const int64_t saved = (below - 1) * tok * head_tok_bytes;
        const int64_t pages = (tok + cap::kPage - 1) / cap::kPage;
        const int64_t added = 2 * nreq * G * partial_row_bytes * estimate_chunks(pages);
        return (double)saved > (double)o.share_margin * (double)added;
    }

    void emit(const int32_t *reqs, int nreq, const std::vector<int32_t> &entries, int at)
    {
        if (entries.empty() || nreq == 0) return;
        Group g;
        g.reqs.assign(reqs, reqs + nreq);
        g.entries = entries;
        g.at = at;
        groups.push_back(std::move(g));
    }

    void walk(int n, std::vector<int32_t> prefix, int64_t prefix_tokens)
    {
        std::vector<int32_t> entries = std::move(prefix);
        node_entries(n, entries);
        const int64_t tok = prefix_tokens + t.ntok[n];
        if (decide_share(n, prefix_tokens)) {
            emit(&t.req_list[t.req_off[n]], t.req_off[n + 1] - t.req_off[n], entries, n);
            for (int c : t.children[n]) walk(c, {}, 0);
        } else {
            emit(t.end_list.data() + t.end_off[n], t.end_off[n + 1] - t.end_off[n], entries, n);
            for (int c : t.children[n]) walk(c, entries, tok);
        }
    }

    void build_groups()
    {
        // first pass with a provisional item size, then size items so that
        // the total cost fills every CU about `rounds` times, and plan again
        // (the share/fold test depends on the split)
        for (int pass = 0; pass < 2; ++pass) {
            groups.clear();
            for (int n = 0; n < t.N; ++n)
                if (t.parent[n] == -1) walk(n, {}, 0);
            double W = 0;   // total cost if nothing were split
            for (const Group &g : groups) {
                const int64_t nreq = (int64_t)g.reqs.size();
                const int64_t rg = (nreq + reqs_per_item(nreq) - 1) / reqs_per_item(nreq);
                W += (double)g.entries.size() * rg * Hkv * page_cost(is_shared(nreq));
            }
            unit = std::max(4.0, W / ((double)o.num_cus * o.rounds));
            unit_private = std::max(4.0, W / ((double)o.num_cus * o.private_rounds));
        }
    }
};

void fill_defaults(cap_plan_opts &o)
{
    if (o.share_mode == 2) o.share_mode = -1;
    if (o.shared_rows == 0) o.shared_rows = cap::kPrivateRows;
    if (o.num_cus == 0) o.num_cus = 256;
    if (o.shared_cost == 0.f) o.shared_cost = 2.0f;
    if (o.rounds == 0.f) o.rounds = 1.5f;
    if (o.share_margin == 0.f) o.share_margin = 1.0f;
    if (o.order == 0) o.order = 2;
    if (o.private_rounds == 0.f) o.private_rounds = 1.0f;
    if (o.tail_factor == 0.f) o.tail_factor = 1.0f;
    if (o.tail_min_pages == 0) o.tail_min_pages = 16;
    if (o.append_slack == 0) o.append_slack = 8;
}

}  // namespace

extern "C" {

int32_t cap_abi_version(void) { return CAP_ABI_VERSION; }

const char *cap_last_error(void) { return g_err.c_str(); }

void cap_plan_opts_default(cap_plan_opts *opts)
{
    if (!opts) return;
    std::memset(opts, 0, sizeof *opts);
    opts->share_mode = -1;
    fill_defaults(*opts);
}

cap_status cap_tree_device_bytes(const cap_attn_desc *attn, const cap_tree_desc *tree, size_t *bytes)
{
    if (!tree || !bytes) return fail(CAP_ERR_INVALID_ARG, "NULL argument");
    cap_status st = check_attn(attn);
    if (st != CAP_OK) return st;
    if (tree->num_nodes <= 0 || !tree->page_offsets) return fail(CAP_ERR_BAD_TREE, "empty tree");
    const int64_t pages = tree->page_offsets[tree->num_nodes];
    if (pages < 0) return fail(CAP_ERR_BAD_TREE, "negative page count");
    *bytes = align_up((size_t)std::max<int64_t>(pages, 1) * 4);
    return CAP_OK;
}

cap_status cap_tree_upload(const cap_attn_desc *attn, const cap_tree_desc *desc, void *dev_buf,
                           size_t dev_bytes, cap_stream_t stream, cap_tree **out)
{
    if (!out) return fail(CAP_ERR_INVALID_ARG, "out is NULL");
    *out = nullptr;
    cap_tree *t = nullptr;
    cap_status st = build_tree(attn, desc, &t);
    if (st != CAP_OK) return st;
    if (dev_buf) {
        const size_t need = t->page_ids.size() * 4;
        if (dev_bytes < need || (reinterpret_cast<uintptr_t>(dev_buf) & 15)) {
            delete t;
            return fail(CAP_ERR_WORKSPACE, "tree device buffer: %zu bytes given, %zu needed (16-byte aligned)",
                        dev_bytes, need);
        }
        if (need) {
            hipError_t e = hipMemcpyAsync(dev_buf, t->page_ids.data(), need, hipMemcpyHostToDevice,
                                          reinterpret_cast<hipStream_t>(stream));
            if (e != hipSuccess) {
                delete t;
                return fail(CAP_ERR_HIP, "tree upload copy failed: %s", hipGetErrorString(e));
            }
        }
        t->dev_pages = static_cast<const int32_t *>(dev_buf);
    }
    *out = t;
    return CAP_OK;
}

void cap_tree_free(cap_tree *tree) { delete tree; }

cap_status cap_tree_get_desc(const cap_tree *t, cap_tree_desc *d)
{
    if (!t || !d) return fail(CAP_ERR_INVALID_ARG, "NULL argument");
    d->num_nodes = t->N;
    d->parent = t->parent.data();
    d->num_tokens = t->ntok.data();
    d->page_offsets = t->page_off.data();
    d->page_ids = t->page_ids.data();
    d->num_requests = t->R;
    d->path_offsets = t->path_off.data();
    d->path_nodes = t->path_nodes.data();
    d->num_pool_pages = t->num_pool_pages;
    return CAP_OK;
}

// One decode step's token for each active request.  A request whose path
// ends at a leaf that no other request passes through extends that leaf
// (into the free slot of its last page, or a new page when the last page is
// full or the leaf has none); any other request gets a new one-token child
// under its end node (a radix-tree branch: the end node stays shared).
cap_status cap_tree_append(cap_tree *t, const uint8_t *active, const int32_t *new_pages, int32_t *dest)
{
    if (!t || !dest) return fail(CAP_ERR_INVALID_ARG, "NULL argument");
    const int R = t->R;
    if (t->owned.empty()) {
        t->owned.assign((size_t)(t->num_pool_pages + 63) / 64, 0);
        for (int32_t pg : t->page_ids) t->owned[pg >> 6] |= uint64_t(1) << (pg & 63);
    }
    enum { kSkip, kSlot, kPage, kBranch };
    std::vector<uint8_t> kind(R, kSkip);
    std::vector<int32_t> taken;
    int32_t branches = 0;
    for (int r = 0; r < R; ++r) {
        if (active && !active[r]) continue;
        const int n = t->path_nodes[t->path_off[r + 1] - 1];
        const bool exclusive = t->children[n].empty() && t->req_off[n + 1] - t->req_off[n] == 1;
        if (exclusive && t->ntok[n] == std::numeric_limits<int32_t>::max())
            return fail(CAP_ERR_UNSUPPORTED, "request %d: node %d holds 2^31 - 1 tokens", r, n);
        kind[r] = !exclusive ? kBranch : (t->ntok[n] % cap::kPage ? kSlot : kPage);
        if (kind[r] == kSlot) continue;
        if (!new_pages) return fail(CAP_ERR_INVALID_ARG, "request %d needs a new page but new_pages is NULL", r);
        const int32_t pg = new_pages[r];
        if (pg < 0 || pg >= t->num_pool_pages)
            return fail(CAP_ERR_BAD_TREE, "new_pages[%d] = %d outside the pool of %lld pages", r, pg,
                        (long long)t->num_pool_pages);
        if (t->owned[pg >> 6] >> (pg & 63) & 1)
            return fail(CAP_ERR_BAD_TREE, "new_pages[%d] = %d is already owned by a node", r, pg);
        taken.push_back(pg);
        branches += kind[r] == kBranch;
    }
    std::vector<int32_t> sorted = taken;
    std::sort(sorted.begin(), sorted.end());
    for (size_t i = 1; i < sorted.size(); ++i)
        if (sorted[i] == sorted[i - 1])
            return fail(CAP_ERR_BAD_TREE, "new page %d is given to two requests", sorted[i]);
    if ((int64_t)t->page_ids.size() + (int64_t)taken.size() >= (int64_t(1) << 26))
        return fail(CAP_ERR_UNSUPPORTED, "tree would hold 2^26 pages or more");
    if ((int64_t)t->N + branches > std::numeric_limits<int32_t>::max() / 2)
        return fail(CAP_ERR_UNSUPPORTED, "tree would hold too many nodes");

    // apply: token counts, then one rebuild of the page lists (and of the
    // paths and derived tables when a branch was made)
    const int N0 = t->N;
    std::vector<std::vector<int32_t>> extra(N0);   // pages appended to existing nodes
    std::vector<int32_t> new_parent, new_page, new_req;
    for (int r = 0; r < R; ++r) {
        if (kind[r] == kSkip) {
            dest[r] = -1;
            continue;
        }
        const int n = t->path_nodes[t->path_off[r + 1] - 1];
        if (kind[r] == kBranch) {
            new_parent.push_back(n);
            new_page.push_back(new_pages[r]);
            new_req.push_back(r);
            dest[r] = new_pages[r] << 4;
            continue;
        }
        const int32_t slot = t->ntok[n] % cap::kPage;
        int32_t pg;
        if (kind[r] == kSlot) {
            pg = t->page_ids[t->page_off[n] + t->ntok[n] / cap::kPage];
        } else {
            pg = new_pages[r];
            extra[n].push_back(pg);
        }
        ++t->ntok[n];
        ++t->ctx_len[r];
        ++t->sum_ctx;
        ++t->unique_tokens;
        dest[r] = pg << 4 | slot;
    }
    for (int32_t pg : taken) t->owned[pg >> 6] |= uint64_t(1) << (pg & 63);
    if (taken.empty()) return CAP_OK;
    std::vector<int64_t> off(N0 + new_parent.size() + 1, 0);
    std::vector<int32_t> ids;
    ids.reserve(t->page_ids.size() + taken.size());
    for (int n = 0; n < N0; ++n) {
        ids.insert(ids.end(), t->page_ids.begin() + t->page_off[n], t->page_ids.begin() + t->page_off[n + 1]);
        ids.insert(ids.end(), extra[n].begin(), extra[n].end());
        off[n + 1] = (int64_t)ids.size();
    }
    for (size_t b = 0; b < new_parent.size(); ++b) {
        ids.push_back(new_page[b]);
        off[N0 + b + 1] = (int64_t)ids.size();
    }
    t->page_ids.swap(ids);
    t->page_off.swap(off);
    if (new_parent.empty()) return CAP_OK;
    std::vector<int32_t> poff(R + 1, 0), pnodes;
    pnodes.reserve(t->path_nodes.size() + new_parent.size());
    size_t b = 0;
    for (int r = 0; r < R; ++r) {
        pnodes.insert(pnodes.end(), t->path_nodes.begin() + t->path_off[r],
                      t->path_nodes.begin() + t->path_off[r + 1]);
        if (b < new_req.size() && new_req[b] == r) pnodes.push_back(N0 + (int32_t)b++);
        poff[r + 1] = (int32_t)pnodes.size();
    }
    t->path_off.swap(poff);
    t->path_nodes.swap(pnodes);
    for (size_t i = 0; i < new_parent.size(); ++i) {
        t->parent.push_back(new_parent[i]);
        t->ntok.push_back(1);
    }
    t->N = N0 + (int32_t)new_parent.size();
    derive(*t);
    ++t->shape_gen;
    return CAP_OK;
}

cap_status cap_plan_step(const cap_tree *tree, const cap_plan_opts *opts_in, cap_plan **out)
{
    if (!tree || !out) return fail(CAP_ERR_INVALID_ARG, "NULL argument");
    *out = nullptr;
    const auto t0 = std::chrono::steady_clock::now();
    cap_plan_opts o;
    if (opts_in) o = *opts_in; else cap_plan_opts_default(&o);
    fill_defaults(o);
    if (o.share_mode < -1 || o.share_mode > 1)
        return fail(CAP_ERR_INVALID_ARG, "share_mode %d not in {-1, 0, 1, 2}", o.share_mode);
    if (o.shared_rows < 0)
        return fail(CAP_ERR_INVALID_ARG, "shared_rows %d is negative", o.shared_rows);
    if (o.split_pages < 0 || o.num_cus < 0 || !(o.shared_cost > 0.f) || !(o.rounds > 0.f) ||
        !(o.share_margin > 0.f) || !(o.private_rounds > 0.f) || o.tail_factor < 0.f || o.tail_min_pages < 1)
        return fail(CAP_ERR_INVALID_ARG, "negative planner option");
    if (o.item_dispatch < 0 || o.item_dispatch > 1)
        return fail(CAP_ERR_INVALID_ARG, "item_dispatch %d not in {0, 1}", o.item_dispatch);
    if (o.append_slack < -1 || o.append_slack > 4096)
        return fail(CAP_ERR_INVALID_ARG, "append_slack %d not in [-1, 4096]", o.append_slack);
    if (o.append_slack == -1) o.append_slack = 0;
    if (o.order < 1 || o.order > 4) return fail(CAP_ERR_INVALID_ARG, "order %d not in {0, .., 4}", o.order);

    cap_plan *p = new (std::nothrow) cap_plan();
    if (!p) return fail(CAP_ERR_INVALID_ARG, "out of host memory");
    p->tree = tree;
    p->work_queue = o.item_dispatch == 1;
    const int Hkv = tree->attn.num_kv_heads, Hq = tree->attn.num_q_heads, D = tree->attn.head_dim;
    Planner pl(*tree, o);
    pl.build_groups();

    // tasks: (page run, request subgroup); balanced splits of both.  Partial
    // slots are assigned once the dispatch sequence is fixed.
    struct Task { int32_t so, np, ro, nr, sb; bool shared; double cost; int32_t idx, grp; };
    std::vector<Task> tasks;
    p->leaf.assign(tree->R, cap_plan::Leaf{});
    std::vector<int32_t> grp_leaf(pl.groups.size(), -1);   // request whose leaf run the group is
    for (size_t gi = 0; gi < pl.groups.size(); ++gi) {
        const Group &g = pl.groups[gi];
        const int64_t npg = (int64_t)g.entries.size();
        const int nreq = (int)g.reqs.size();
        const bool shared = pl.is_shared(nreq);
        const int64_t k = pl.chunks(npg, shared);
        const int rg = (nreq + pl.reqs_per_item(nreq) - 1) / pl.reqs_per_item(nreq);
        const int32_t so0 = (int32_t)p->stream.size();
        p->stream.insert(p->stream.end(), g.entries.begin(), g.entries.end());
        // a run serving one request, ending with the pages of the leaf where
        // that request's context ends and no other request's path passes,
        // can take the leaf's new pages in place: free entries follow it
        if (nreq == 1) {
            const int r = g.reqs[0], n = g.at;
            if (tree->path_nodes[tree->path_off[r + 1] - 1] == n && tree->children[n].empty() &&
                tree->req_off[n + 1] - tree->req_off[n] == 1) {
                cap_plan::Leaf &lf = p->leaf[r];
                lf.node = n;
                lf.pages = (int32_t)(tree->page_off[n + 1] - tree->page_off[n]);
                lf.end = (int32_t)p->stream.size();
                lf.limit = lf.end + o.append_slack;
                p->stream.insert(p->stream.end(), (size_t)o.append_slack, 0);
                grp_leaf[gi] = r;
            }
        }
        const int32_t ro0 = (int32_t)p->rows.size();
        p->rows.insert(p->rows.end(), g.reqs.begin(), g.reqs.end());
        for (int64_t ci = 0; ci < k; ++ci) {
            const int64_t pb = npg * ci / k, pe = npg * (ci + 1) / k;
            for (int ri = 0; ri < rg; ++ri) {
                const int rb = (int)((int64_t)nreq * ri / rg), re = (int)((int64_t)nreq * (ri + 1) / rg);
                tasks.push_back(Task{(int32_t)(so0 + pb), (int32_t)(pe - pb), ro0 + rb, re - rb, -1, shared,
                                     (double)(pe - pb) * pl.page_cost(shared), (int32_t)tasks.size(),
                                     (int32_t)gi});
            }
        }
    }
    // The hardware starts workgroups in item order as CUs free up, so a list
    // sorted costliest first is greedy longest-processing-time scheduling.
    // order 1 interleaves the two kinds evenly (each costliest first), 2 sorts
    // both kinds together, 3 puts every shared item first, 4 starts with one
    // shared and one private workgroup per CU.  One item per task and KV head,
    // the heads of a task back to back.
    std::stable_sort(tasks.begin(), tasks.end(), [&](const Task &a, const Task &b) {
        if (o.order == 3 && a.shared != b.shared) return a.shared;
        return a.cost > b.cost;
    });
    std::vector<Task> seq;
    seq.reserve(tasks.size() * 2);
    if (o.order == 1 || o.order == 4) {
        std::vector<const Task *> sh, pr;
        for (const Task &tk : tasks) (tk.shared ? sh : pr).push_back(&tk);
        size_t i_sh = 0, i_pr = 0;
        if (o.order == 4) {
            // first wave: one shared and one private workgroup on every CU (the
            // hardware gives each CU of an XCD one workgroup before any second)
            const size_t per = std::max<size_t>(1, (size_t)o.num_cus / std::max(1, Hkv));
            for (; i_sh < std::min(per, sh.size()); ++i_sh) seq.push_back(*sh[i_sh]);
            for (; i_pr < std::min(per, pr.size()); ++i_pr) seq.push_back(*pr[i_pr]);
        }
        const size_t sh0 = i_sh, pr0 = i_pr;
        while (i_sh < sh.size() || i_pr < pr.size()) {
            // take the kind that is further behind its share of the rest
            const double a = (double)(i_sh - sh0) * (pr.size() - pr0), b = (double)(i_pr - pr0) * (sh.size() - sh0);
            const bool take_sh = i_pr >= pr.size() || (i_sh < sh.size() && a <= b);
            seq.push_back(take_sh ? *sh[i_sh++] : *pr[i_pr++]);
        }
    } else if (o.tail_factor < 1e30f) {
        // Costliest first with a shrinking cap on private items (guided
        // self-scheduling): an item may cost at most the remaining work per
        // workgroup slot / tail_factor, so the last items to start are short
        // and the slots finish together.  Only private runs are cut (a cut
        // adds one request group's partial rows; cutting a shared run would add
        // a whole group's).  Ties keep creation order, which puts the request
        // subgroups of one page run next to each other: with the heads of a
        // task back to back, their items for one KV head start Hkv apart, on
        // the same XCD when Hkv = 8, and the later ones read the run from its L2.
        auto less = [](const Task &a, const Task &b) {
            return a.cost < b.cost || (a.cost == b.cost && a.idx > b.idx);
        };
        std::vector<Task> heap(tasks.begin(), tasks.end());
        std::make_heap(heap.begin(), heap.end(), less);
        double remaining = 0;
        for (const Task &tk : tasks) remaining += tk.cost;
        const double slots = 2.0 * o.num_cus / std::max(1, Hkv);   // task slots: Hkv items each
        while (!heap.empty()) {
            std::pop_heap(heap.begin(), heap.end(), less);
            Task tk = heap.back();
            heap.pop_back();
            const double cap_cost = remaining / (slots * o.tail_factor);
            const int32_t cap_pages = std::max<int32_t>(o.tail_min_pages, (int32_t)(cap_cost / pl.page_cost(false)));
            if (!tk.shared && tk.np > cap_pages + o.tail_min_pages) {
                Task rest = tk;
                tk.np = cap_pages;
                tk.cost = tk.np * pl.page_cost(false);
                rest.so += cap_pages;
                rest.np -= cap_pages;
                rest.cost = rest.np * pl.page_cost(false);
                heap.push_back(rest);
                std::push_heap(heap.begin(), heap.end(), less);
            }
            remaining -= tk.cost;
            seq.push_back(tk);
        }
    } else {
        seq.assign(tasks.begin(), tasks.end());
    }
    // Partial rows: each request's are one contiguous block (merge_off), so a
    // merge finds them without a table; a task reaches the row of each of its
    // requests through slot_rows[sb + q], filled in dispatch order.
    p->merge_off.assign(tree->R + 1, 0);
    for (const Task &tk : seq)
        for (int q = 0; q < tk.nr; ++q) ++p->merge_off[p->rows[tk.ro + q] + 1];
    int32_t maxp = 0;
    for (int r = 0; r < tree->R; ++r) {
        maxp = std::max<int32_t>(maxp, p->merge_off[r + 1]);
        p->merge_off[r + 1] += p->merge_off[r];
    }
    const int32_t slot_rows = p->merge_off[tree->R];
    std::vector<int32_t> fill(p->merge_off.begin(), p->merge_off.end() - 1);
    p->slot_rows.reserve(slot_rows);
    for (Task &tk : seq) {
        tk.sb = (int32_t)p->slot_rows.size();
        for (int q = 0; q < tk.nr; ++q) p->slot_rows.push_back(fill[p->rows[tk.ro + q]]++);
        pl.max_pages = std::max<int>(pl.max_pages, tk.np);
    }
    p->items.reserve(seq.size() * Hkv);
    for (const Task &tk : seq) {
        const int32_t r = grp_leaf[tk.grp];
        if (r >= 0 && tk.so + tk.np == p->leaf[r].end) p->leaf[r].item0 = (int32_t)p->items.size();
        for (int h = 0; h < Hkv; ++h)
            p->items.push_back(WorkItem{tk.so, tk.np, h, tk.ro, tk.nr, tk.sb,
                                        tk.shared ? cap::kModeShared : cap::kModePrivate, 0});
    }
    p->node_tokens = tree->ntok;
    p->shape_gen = tree->shape_gen;

    // device image: items | stream | rows | slot_rows | merge_off | counters |
    // queue | patch (the fused step's arrival counters, one per request and
    // KV head, and the work queues' counters, all zero; then the area that
    // cap_plan_refresh stages its word patches in)
    std::vector<cap::DevItem> dev_items(p->items.size());
    for (size_t i = 0; i < p->items.size(); ++i) dev_items[i] = dev_item(*p, p->items[i]);
    p->off_items = 0;
    p->off_stream = align_up(dev_items.size() * sizeof(cap::DevItem));
    p->off_rows = p->off_stream + align_up(p->stream.size() * 4);
    p->off_srows = p->off_rows + align_up(p->rows.size() * 4);
    p->off_moff = p->off_srows + align_up(p->slot_rows.size() * 4);
    p->off_cnt = p->off_moff + align_up(p->merge_off.size() * 4);
    p->off_queue = p->off_cnt + align_up((size_t)tree->R * Hkv * 4);
    p->off_patch = p->off_queue + align_up(cap::kQueueInts * 4);
    p->patch_cap = (size_t)4 * tree->R * (Hkv + 1) + 256;
    p->dev_bytes = p->off_patch + align_up(p->patch_cap * 8);
    p->host_image.assign(p->dev_bytes, 0);
    std::memcpy(p->host_image.data() + p->off_items, dev_items.data(), dev_items.size() * sizeof(cap::DevItem));
    std::memcpy(p->host_image.data() + p->off_stream, p->stream.data(), p->stream.size() * 4);
    std::memcpy(p->host_image.data() + p->off_rows, p->rows.data(), p->rows.size() * 4);
    std::memcpy(p->host_image.data() + p->off_srows, p->slot_rows.data(), p->slot_rows.size() * 4);
    std::memcpy(p->host_image.data() + p->off_moff, p->merge_off.data(), p->merge_off.size() * 4);

    cap_plan_stats &s = p->stats;
    s.num_items = (int64_t)p->items.size();
    s.num_shared_items = 0;
    for (const WorkItem &w : p->items) s.num_shared_items += w.mode == cap::kModeShared;
    s.num_tasks = (int64_t)seq.size();
    s.num_groups = (int64_t)pl.groups.size();
    s.partial_rows = slot_rows;
    const size_t slots = (size_t)slot_rows * Hq;
    s.workspace_bytes = (int64_t)(align_up(slots * D * 2) + 2 * align_up(slots * 4));
    s.plan_device_bytes = (int64_t)p->dev_bytes;
    s.tree_device_bytes = (int64_t)align_up(std::max<size_t>(tree->page_ids.size(), 1) * 4);
    const int64_t page_bytes = 2LL * cap::kPage * D * 2;   // K+V of one page, one head
    int64_t streamed = 0;
    for (const Task &tk : seq) streamed += (int64_t)tk.np * page_bytes * Hkv;
    s.kv_bytes_streamed = streamed;
    s.kv_bytes_unique = tree->unique_tokens * 4LL * D * Hkv;
    s.kv_bytes_unshared = tree->sum_ctx * 4LL * D * Hkv;
    s.partial_bytes = (int64_t)slots * (2LL * D + 8);
    s.max_partials_per_request = maxp;
    s.max_pages_per_item = pl.max_pages;
    s.plan_host_us = std::chrono::duration<double, std::micro>(std::chrono::steady_clock::now() - t0).count();
    *out = p;
    return CAP_OK;
}

cap_status cap_plan_get_stats(const cap_plan *plan, cap_plan_stats *stats)
{
    if (!plan || !stats) return fail(CAP_ERR_INVALID_ARG, "NULL argument");
    *stats = plan->stats;
    return CAP_OK;
}

cap_status cap_plan_get_view(const cap_plan *plan, cap_plan_view *v)
{
    if (!plan || !v) return fail(CAP_ERR_INVALID_ARG, "NULL argument");
    v->num_items = (int32_t)plan->items.size();
    v->items = reinterpret_cast<const cap_work_item *>(plan->items.data());
    v->stream_len = (int32_t)plan->stream.size();
    v->stream = plan->stream.data();
    v->rows_len = (int32_t)plan->rows.size();
    v->rows = plan->rows.data();
    v->num_requests = plan->tree->R;
    v->merge_off = plan->merge_off.data();
    v->slot_rows_len = (int32_t)plan->slot_rows.size();
    v->slot_rows = plan->slot_rows.data();
    return CAP_OK;
}

cap_status cap_plan_upload(cap_plan *plan, void *dev_buf, size_t bytes, cap_stream_t stream)
{
    if (!plan || !dev_buf) return fail(CAP_ERR_INVALID_ARG, "NULL argument");
    if (bytes < plan->dev_bytes || (reinterpret_cast<uintptr_t>(dev_buf) & (kAlign - 1)))
        return fail(CAP_ERR_WORKSPACE, "plan buffer: %zu bytes given, %zu needed (256-byte aligned)",
                    bytes, plan->dev_bytes);
    hipError_t e = hipMemcpyAsync(dev_buf, plan->host_image.data(), plan->dev_bytes,
                                  hipMemcpyHostToDevice, reinterpret_cast<hipStream_t>(stream));
    if (e != hipSuccess) return fail(CAP_ERR_HIP, "plan upload copy failed: %s", hipGetErrorString(e));
    plan->dev = dev_buf;
    return CAP_OK;
}

cap_status cap_plan_refresh(cap_plan *p, cap_stream_t stream)
{
    if (!p) return fail(CAP_ERR_INVALID_ARG, "NULL argument");
    const auto t0 = std::chrono::steady_clock::now();
    const cap_tree &t = *p->tree;
    if (t.shape_gen != p->shape_gen)
        return fail(CAP_ERR_REPLAN, "the tree's nodes or request paths changed since the plan was built");
    // every node whose token count changed must end a leaf run with room
    std::vector<int32_t> grow;
    for (int n = 0; n < t.N; ++n) {
        if (t.ntok[n] == p->node_tokens[n]) continue;
        const int r = t.end_off[n + 1] - t.end_off[n] == 1 ? t.end_list[t.end_off[n]] : -1;
        if (t.ntok[n] < p->node_tokens[n] || r < 0 || p->leaf[r].node != n)
            return fail(CAP_ERR_REPLAN, "node %d changed and the plan has no run of its own for it", n);
        const cap_plan::Leaf &lf = p->leaf[r];
        const int32_t add = (int32_t)(t.page_off[n + 1] - t.page_off[n]) - lf.pages;
        const WorkItem &w = p->items[lf.item0];
        const int32_t cap = w.mode == cap::kModeShared ? cap::kMaxSharedPages : cap::kMaxPrivatePages;
        if (lf.end + add > lf.limit || w.npages + add > cap)
            return fail(CAP_ERR_REPLAN, "request %d: %d new pages exceed the room after its run", r, add);
        grow.push_back(r);
    }
    p->patch.clear();
    bool overflow = false;
    int64_t words = 0;
    auto set = [&](size_t byte_off, uint32_t v) {
        uint32_t *word = reinterpret_cast<uint32_t *>(p->host_image.data() + byte_off);
        if (*word == v) return;
        *word = v;
        ++words;
        if (p->patch.size() / 2 < p->patch_cap) {
            p->patch.push_back((uint32_t)(byte_off / 4));
            p->patch.push_back(v);
        } else {
            overflow = true;
        }
    };
    const int Hkv = t.attn.num_kv_heads;
    int64_t added = 0;
    for (int r : grow) {
        cap_plan::Leaf &lf = p->leaf[r];
        const int n = lf.node;
        const int32_t pages = (int32_t)(t.page_off[n + 1] - t.page_off[n]);
        const int32_t first = lf.end - lf.pages;   // stream index of the node's first page
        for (int32_t k = std::max(0, lf.pages - 1); k < pages; ++k) {
            const int64_t left = t.ntok[n] - (int64_t)k * cap::kPage;
            const int32_t e = (int32_t)(((int64_t)t.page_ids[t.page_off[n] + k] << 5) |
                                        (std::min<int64_t>(cap::kPage, left) - 1));
            p->stream[first + k] = e;
            set(p->off_stream + 4 * (size_t)(first + k), (uint32_t)e);
        }
        // the run's Hkv items differ only in their head; of a device item
        // only the page count and the inline entries can change
        const int32_t add = pages - lf.pages;
        for (int h = 0; h < Hkv; ++h) p->items[lf.item0 + h].npages += add;
        const cap::DevItem d = dev_item(*p, p->items[lf.item0]);
        p->stats.max_pages_per_item = std::max<int32_t>(p->stats.max_pages_per_item, d.npages);
        const size_t base = p->off_items + (size_t)lf.item0 * sizeof(cap::DevItem);
        auto put = [&](size_t field, uint32_t v) {   // same word of all Hkv items
            if (*reinterpret_cast<const uint32_t *>(p->host_image.data() + base + field) == v) return;
            for (int h = 0; h < Hkv; ++h) set(base + h * sizeof(cap::DevItem) + field, v);
        };
        put(offsetof(cap::DevItem, npages), (uint32_t)d.npages);
        for (int j = 0; j < cap::kInlineEntries; ++j) put(offsetof(cap::DevItem, ent) + 4 * j, (uint32_t)d.ent[j]);
        lf.end += add;
        lf.pages = pages;
        added += add;
    }
    p->node_tokens = t.ntok;
    const int64_t D = t.attn.head_dim;
    p->stats.kv_bytes_streamed += added * 2LL * cap::kPage * D * 2 * Hkv;
    p->stats.kv_bytes_unique = t.unique_tokens * 4LL * D * Hkv;
    p->stats.kv_bytes_unshared = t.sum_ctx * 4LL * D * Hkv;
    if (words == 0) return CAP_OK;
    p->stats.refresh_words = words;
    p->stats.refresh_full_copy = overflow ? 1 : 0;
    ++p->stats.refreshes;
    auto done = [&] {
        p->stats.refresh_host_us =
            std::chrono::duration<double, std::micro>(std::chrono::steady_clock::now() - t0).count();
        return CAP_OK;
    };
    if (!p->dev) return done();
    hipStream_t s = reinterpret_cast<hipStream_t>(stream);
    char *dev = static_cast<char *>(p->dev);
    hipError_t e;
    if (overflow) {
        // everything before the counters (they read zero between launches)
        e = hipMemcpyAsync(dev, p->host_image.data(), p->off_cnt, hipMemcpyHostToDevice, s);
    } else {
        e = hipMemcpyAsync(dev + p->off_patch, p->patch.data(), p->patch.size() * 4, hipMemcpyHostToDevice, s);
        if (e == hipSuccess) {
            const int le = cap::launch_patch(dev, reinterpret_cast<const uint32_t *>(dev + p->off_patch),
                                             (int)(p->patch.size() / 2), stream);
            e = static_cast<hipError_t>(le);
        }
    }
    if (e != hipSuccess) {
        p->dev = nullptr;   // device copy out of date: upload again
        return fail(CAP_ERR_HIP, "plan patch upload failed: %s", hipGetErrorString(e));
    }
    return done();
}

cap_status cap_append_kv(const cap_tree *tree, const int32_t *dest, int32_t n, const void *k_new,
                         const void *v_new, void *k_pool, void *v_pool, cap_stream_t stream)
{
    if (!tree || n < 0) return fail(CAP_ERR_INVALID_ARG, "NULL tree or negative count");
    if (n == 0) return CAP_OK;
    if (!dest || !k_new || !v_new || !k_pool || !v_pool) return fail(CAP_ERR_INVALID_ARG, "NULL argument");
    if (((uintptr_t)k_new | (uintptr_t)v_new | (uintptr_t)k_pool | (uintptr_t)v_pool) & 15)
        return fail(CAP_ERR_INVALID_ARG, "k_new, v_new, k_pool and v_pool must be 16-byte aligned");
    if ((int64_t)n * tree->attn.num_kv_heads * (tree->attn.head_dim / 8) >= ((int64_t)1 << 31))
        return fail(CAP_ERR_UNSUPPORTED, "%d tokens: too many for one launch", n);
    cap::AppendArgs a{};
    a.dest = dest;
    a.n = n;
    a.k_new = static_cast<const uint16_t *>(k_new);
    a.v_new = static_cast<const uint16_t *>(v_new);
    a.k_pool = static_cast<uint16_t *>(k_pool);
    a.v_pool = static_cast<uint16_t *>(v_pool);
    a.Hkv = tree->attn.num_kv_heads;
    a.D = tree->attn.head_dim;
    a.pool_pages = tree->num_pool_pages;
    const int e = cap::launch_append(a, stream);
    if (e != 0) return fail(CAP_ERR_HIP, "append launch failed: %s", cap::hip_error_string(e));
    return CAP_OK;
}

static cap_status split_workspace(const cap_plan *p, const void *ws, size_t ws_bytes, uint16_t **o,
                                  float **m, float **l)
{
    if ((size_t)p->stats.workspace_bytes > ws_bytes || (reinterpret_cast<uintptr_t>(ws) & (kAlign - 1)))
        return fail(CAP_ERR_WORKSPACE, "workspace: %zu bytes given, %lld needed (256-byte aligned)",
                    ws_bytes, (long long)p->stats.workspace_bytes);
    const size_t slots = (size_t)p->stats.partial_rows * p->tree->attn.num_q_heads;
    const size_t o_bytes = align_up(slots * p->tree->attn.head_dim * 2);
    char *b = (char *)ws;
    *o = (uint16_t *)b;
    *m = (float *)(b + o_bytes);
    *l = (float *)(b + o_bytes + align_up(slots * 4));
    return CAP_OK;
}

static cap_status decode_args(const cap_plan *plan, const void *q, const void *k_pool, const void *v_pool,
                              void *workspace, size_t ws_bytes, cap::DecodeArgs &a)
{
    if (!plan || !q || !k_pool || !v_pool || !workspace) return fail(CAP_ERR_INVALID_ARG, "NULL argument");
    if (!plan->dev) return fail(CAP_ERR_STATE, "plan not uploaded (call cap_plan_upload first)");
    if (((uintptr_t)q | (uintptr_t)k_pool | (uintptr_t)v_pool) & 15)
        return fail(CAP_ERR_INVALID_ARG, "q, k_pool and v_pool must be 16-byte aligned");
    a = cap::DecodeArgs{};
    cap_status st = split_workspace(plan, workspace, ws_bytes, &a.part_o, &a.part_m, &a.part_l);
    if (st != CAP_OK) return st;
    const char *d = static_cast<const char *>(plan->dev);
    a.items = reinterpret_cast<const cap::DevItem *>(d + plan->off_items);
    a.stream = reinterpret_cast<const int32_t *>(d + plan->off_stream);
    a.rows = reinterpret_cast<const int32_t *>(d + plan->off_rows);
    a.slot_rows = reinterpret_cast<const int32_t *>(d + plan->off_srows);
    a.q = static_cast<const uint16_t *>(q);
    a.k_pool = static_cast<const uint16_t *>(k_pool);
    a.v_pool = static_cast<const uint16_t *>(v_pool);
    a.n_items = (int32_t)plan->items.size();
    a.Hq = plan->tree->attn.num_q_heads;
    a.Hkv = plan->tree->attn.num_kv_heads;
    a.G = plan->tree->G;
    a.log2G = __builtin_ctz((unsigned)a.G);   // G is a power of two (checked with the shape)
    a.scale_log2 = (float)((double)plan->tree->attn.sm_scale * 1.4426950408889634);
    if (plan->work_queue) a.queue = reinterpret_cast<int32_t *>(static_cast<char *>(plan->dev) + plan->off_queue);
    return CAP_OK;
}

cap_status cap_decode_attention(const cap_plan *plan, const void *q, const void *k_pool,
                                const void *v_pool, void *workspace, size_t ws_bytes,
                                cap_stream_t stream)
{
    cap::DecodeArgs a;
    cap_status st = decode_args(plan, q, k_pool, v_pool, workspace, ws_bytes, a);
    if (st != CAP_OK) return st;
    const int e = cap::launch_decode(a, plan->tree->attn.head_dim, stream);
    if (e != 0) return fail(CAP_ERR_HIP, "decode launch failed: %s", cap::hip_error_string(e));
    return CAP_OK;
}

cap_status cap_decode_step(const cap_plan *plan, const void *q, const void *k_pool, const void *v_pool,
                           void *workspace, size_t ws_bytes, void *out, cap_stream_t stream)
{
    if (!out) return fail(CAP_ERR_INVALID_ARG, "NULL argument");
    if ((uintptr_t)out & 15) return fail(CAP_ERR_INVALID_ARG, "out must be 16-byte aligned");
    cap::DecodeArgs a;
    cap_status st = decode_args(plan, q, k_pool, v_pool, workspace, ws_bytes, a);
    if (st != CAP_OK) return st;
    const int64_t slots = plan->stats.partial_rows * (int64_t)a.Hq;
    if (slots * plan->tree->attn.head_dim * 2 >= (int64_t)1 << 31)
        return fail(CAP_ERR_UNSUPPORTED, "fused step: %lld partial slots exceed the 2 GiB partial-o limit "
                    "(use cap_decode_attention + cap_merge_partials)", (long long)slots);
    a.slots = (int32_t)slots;
    char *d = static_cast<char *>(plan->dev);
    a.counters = reinterpret_cast<int32_t *>(d + plan->off_cnt);
    a.merge_off = reinterpret_cast<const int32_t *>(d + plan->off_moff);
    a.out = static_cast<uint16_t *>(out);
    const int e = cap::launch_decode(a, plan->tree->attn.head_dim, stream);
    if (e != 0) return fail(CAP_ERR_HIP, "decode launch failed: %s", cap::hip_error_string(e));
    return CAP_OK;
}

cap_status cap_merge_partials(const cap_plan *plan, const void *workspace, size_t ws_bytes, void *out,
                              cap_stream_t stream)
{
    if (!plan || !workspace || !out) return fail(CAP_ERR_INVALID_ARG, "NULL argument");
    if (!plan->dev) return fail(CAP_ERR_STATE, "plan not uploaded (call cap_plan_upload first)");
    if ((uintptr_t)out & 15) return fail(CAP_ERR_INVALID_ARG, "out must be 16-byte aligned");
    cap::MergeArgs a{};
    uint16_t *o;
    float *m, *l;
    cap_status st = split_workspace(plan, workspace, ws_bytes, &o, &m, &l);
    if (st != CAP_OK) return st;
    const char *d = static_cast<const char *>(plan->dev);
    a.merge_off = reinterpret_cast<const int32_t *>(d + plan->off_moff);
    a.part_o = o;
    a.part_m = m;
    a.part_l = l;
    a.out = static_cast<uint16_t *>(out);
    a.R = plan->tree->R;
    a.Hq = plan->tree->attn.num_q_heads;
    const int e = cap::launch_merge(a, plan->tree->attn.head_dim, stream);
    if (e != 0) return fail(CAP_ERR_HIP, "merge launch failed: %s", cap::hip_error_string(e));
    return CAP_OK;
}

void cap_plan_free(cap_plan *plan) { delete plan; }

// ------------------------------------------------------- wide-row workloads

static cap_status rows_launch(cap::RowArgs &a, int32_t mode, cap_stream_t stream)
{
    if (!a.x || !a.y) return fail(CAP_ERR_INVALID_ARG, "NULL argument");
    if (a.rows < 0 || a.width < 1) return fail(CAP_ERR_INVALID_ARG, "rows %lld / width %lld out of range",
                                             (long long)a.rows, (long long)a.width);
    if (mode < 0 || mode > 2) return fail(CAP_ERR_INVALID_ARG, "mode %d not in {0, 1, 2}", mode);
    if (a.rows > std::numeric_limits<int32_t>::max())
        return fail(CAP_ERR_UNSUPPORTED, "%lld rows: at most 2^31 - 1", (long long)a.rows);
    if (a.width > ((int64_t)1 << 24))
        return fail(CAP_ERR_UNSUPPORTED, "width %lld above 2^24", (long long)a.width);
    if (mode == 1 && a.width > cap::kMaxRetainedWidth)
        return fail(CAP_ERR_UNSUPPORTED, "width %lld: a retained row holds at most %lld values",
                    (long long)a.width, (long long)cap::kMaxRetainedWidth);
    const size_t bytes = (size_t)a.rows * a.width * 4;
    const uintptr_t x0 = (uintptr_t)a.x, y0 = (uintptr_t)a.y;
    if (x0 != y0 && x0 < y0 + bytes && y0 < x0 + bytes)
        return fail(CAP_ERR_INVALID_ARG, "x and y overlap without being the same buffer");
    if (a.rows == 0) return CAP_OK;
    uintptr_t align = x0 | y0;
    if (a.kind == cap::kRowLayerNorm) align |= (uintptr_t)a.gamma | (uintptr_t)a.beta;
    const bool vec4 = (a.width % 4 == 0) && (align & 15) == 0;
    // auto: retained up to 64K values with 16-byte accesses; with 4-byte
    // accesses only up to 16K (a wider retained row spills registers)
    const bool retained = mode == 1 || (mode == 0 && a.width <= (vec4 ? cap::kMaxRetainedWidth : 16384));
    const int e = cap::launch_rows(a, vec4, retained, stream);
    if (e != 0) return fail(CAP_ERR_HIP, "row kernel launch failed: %s", cap::hip_error_string(e));
    return CAP_OK;
}

cap_status cap_rows_softmax(const float *x, float *y, int64_t rows, int64_t width, int32_t mode,
                            cap_stream_t stream)
{
    cap::RowArgs a{};
    a.x = x;
    a.y = y;
    a.rows = rows;
    a.width = width;
    a.kind = cap::kRowSoftmax;
    return rows_launch(a, mode, stream);
}

cap_status cap_rows_layernorm(const float *x, const float *gamma, const float *beta, float *y, int64_t rows,
                              int64_t width, float eps, int32_t mode, cap_stream_t stream)
{
    if (!gamma || !beta) return fail(CAP_ERR_INVALID_ARG, "NULL gamma or beta");
    if (!(eps >= 0.f) || !std::isfinite(eps)) return fail(CAP_ERR_INVALID_ARG, "eps must be finite and >= 0");
    cap::RowArgs a{};
    a.x = x;
    a.gamma = gamma;
    a.beta = beta;
    a.y = y;
    a.rows = rows;
    a.width = width;
    a.eps = eps;
    a.kind = cap::kRowLayerNorm;
    return rows_launch(a, mode, stream);
}

// ------------------------------------------------------------ bench helpers

cap_status cap_bench_fill(void *buf, size_t bytes, uint32_t value, cap_stream_t stream)
{
    if (!buf || bytes == 0 || (bytes & 15) || ((uintptr_t)buf & 15))
        return fail(CAP_ERR_INVALID_ARG, "fill: bad buffer or size");
    const int e = cap::launch_fill(buf, bytes / 4, value, stream);
    return e ? fail(CAP_ERR_HIP, "fill launch failed: %s", cap::hip_error_string(e)) : CAP_OK;
}

cap_status cap_bench_read(const void *buf, size_t bytes, void *sink, cap_stream_t stream)
{
    if (!buf || !sink || bytes == 0 || (bytes & 15) || ((uintptr_t)buf & 15))
        return fail(CAP_ERR_INVALID_ARG, "read: bad buffer or size");
    const int e = cap::launch_read(buf, bytes / 16, sink, stream);
    return e ? fail(CAP_ERR_HIP, "read launch failed: %s", cap::hip_error_string(e)) : CAP_OK;
}

cap_status cap_bench_read_stream(const void *buf, size_t bytes, void *sink, cap_stream_t stream)
{
    if (!buf || !sink || bytes == 0 || (bytes & 15) || ((uintptr_t)buf & 15))
        return fail(CAP_ERR_INVALID_ARG, "read: bad buffer or size");
    const int e = cap::launch_read_stream(buf, bytes / 16, sink, stream);
    return e ? fail(CAP_ERR_HIP, "read launch failed: %s", cap::hip_error_string(e)) : CAP_OK;
}

cap_status cap_bench_copy(void *dst, const void *src, size_t bytes, cap_stream_t stream)
{
    if (!dst || !src || bytes == 0 || (bytes & 15) || (((uintptr_t)dst | (uintptr_t)src) & 15))
        return fail(CAP_ERR_INVALID_ARG, "copy: bad buffer or size");
    const int e = cap::launch_copy(dst, src, bytes / 16, stream);
    return e ? fail(CAP_ERR_HIP, "copy launch failed: %s", cap::hip_error_string(e)) : CAP_OK;
}

}  // extern "C"
