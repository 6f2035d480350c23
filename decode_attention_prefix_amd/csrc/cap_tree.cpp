// cap_tree.cpp -- host side of libcap: the tree handle (validation, the
// derived node -> request tables, the optional device copy of the page
// table, growth by one token per request and step) and the error channel.
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

#include "cap_host_internal.h"

namespace cap {
namespace host {

namespace {
thread_local std::string g_err;
}  // namespace

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

const char *last_error() { return g_err.c_str(); }

static cap_status check_attn(const cap_attn_desc *a)
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
static cap_status build_tree(const cap_attn_desc *attn, const cap_tree_desc *d, cap_tree **out)
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

}  // namespace host
}  // namespace cap

using namespace cap::host;

extern "C" {

int32_t cap_abi_version(void) { return CAP_ABI_VERSION; }

const char *cap_last_error(void) { return last_error(); }

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

}  // extern "C"
