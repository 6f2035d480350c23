// cap_plan.cpp -- host side of libcap: the per-step planner, the plan's
// device image and its upload, and growth of an uploaded plan in place.
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
// discounted for the rereads that hit the L2, exceed `share_margin` x the
// partial bytes sharing adds plus the start cost of the items it adds (cf.
// the CREDIT summary, section III.B "Traffic Model": the saving is the
// removed reread bytes, while fixed traffic stays; section III.D: each
// candidate's overhead enters its profitability).  Runs are sized so that the work items
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

#include "cap_host_internal.h"

using cap::WorkItem;

namespace cap {
namespace host {

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

}  // namespace host
}  // namespace cap

using namespace cap::host;

namespace {

using cap::host::ChainLink;
using cap::host::PlanGroup;
using cap::host::PlanScratch;
using cap::host::PlanTask;

struct Planner {
    const cap_tree &t;
    cap_plan_opts o;
    PlanScratch &sc;
    int D, Hkv, G;
    int64_t head_tok_bytes;        // K+V bytes per token per KV head
    int64_t partial_row_bytes;     // partial bytes per query row (o, m, l)
    double unit = 0;               // target cost of one shared work item (cost units)
    double unit_private = 0;       // ... of one private work item
    double item_bytes = 0;         // start cost of one item, as bytes streamed meanwhile (per KV head)

    Planner(const cap_tree &tree, const cap_plan_opts &opts, PlanScratch &scratch) : t(tree), o(opts), sc(scratch)
    {
        D = t.attn.head_dim;
        Hkv = t.attn.num_kv_heads;
        G = t.G;
        head_tok_bytes = 4LL * D;
        partial_row_bytes = 2LL * D + 8;
        // a round of items (every workgroup slot starting one) costs item_us;
        // one item's share of it, over 2 x num_cus slots, while the GPU
        // streams at the HBM rate (7.2 TB/s measured on MI355X = 7.2e6 B/us)
        item_bytes = o.item_us > 0.f ? (double)o.item_us * kHbmBytesPerUs / (2.0 * o.num_cus) : 0.0;
    }

    static constexpr double kHbmBytesPerUs = 7.2e6;

    int32_t node_pages(int n) const { return (int32_t)(t.page_off[n + 1] - t.page_off[n]); }

    // Page-stream entries of node n appended at out: (physical page << 5) |
    // (tokens in the page - 1); every page is full except the last.
    int32_t *node_entries(int n, int32_t *out) const
    {
        const int32_t np = node_pages(n);
        const int32_t *ids = t.page_ids.data() + t.page_off[n];
        for (int32_t p = 0; p < np; ++p) out[p] = (ids[p] << 5) | (cap::kPage - 1);
        if (np > 0) out[np - 1] = (ids[np - 1] << 5) | ((t.ntok[n] - 1) % cap::kPage);
        return out + np;
    }

    // Groups wider than the threshold run as shared workgroup items (up to
    // 128 rows each), the rest as private items (up to 16 rows).
    bool is_shared(int64_t nreq) const
    {
        return G > cap::kPrivateRows || nreq * G > o.shared_rows;
    }
    int reqs_per_item(int64_t nreq) const
    {
        return is_shared(nreq) ? cap::kSharedRows / G : cap::kPrivateRows / G;
    }

    // Cost of streaming `pages` pages for one item, in private-page units: a
    // shared item also runs the MFMA/softmax work of up to 128 rows, which
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

    // Share node n (with the folded nodes above it, prefix_tokens) or fold
    // it into its children's runs.  Per KV head, in bytes of streaming:
    //   saved = (groups below - 1) x its K+V bytes / reread_factor -- what
    //           folding would reread (mostly from the XCD's L2: the sibling
    //           groups' items run side by side);
    //   added = share_margin x the partial bytes sharing adds (written and
    //           merged) + its new items x one item's start cost, i.e. the
    //           measured start cost of a round of items spread over the
    //           workgroup slots, as bytes streamed at the HBM rate meanwhile.
    // Share when saved > added.  A node's shared items are small when the
    // node is, and the scheduler starts the smallest items last, so their
    // start latency lands in the step's tail; this is the occupancy side of
    // the trade (cf. the CREDIT summary, section III.D, "Profitability and
    // Candidate Selection": the wave count enters the execution time), next
    // to its traffic side (section III.B, "Traffic Model").
    bool decide_share(int n, int64_t prefix_tokens) const
    {
        if (o.share_mode == 1) return t.ntok[n] > 0 || prefix_tokens > 0;
        if (o.share_mode == 0) return false;
        const int64_t below = (int64_t)t.children[n].size() + (t.end_off[n + 1] > t.end_off[n] ? 1 : 0);
        if (below <= 1) return false;                 // a chain: folding costs nothing
        const int64_t tok = t.ntok[n] + prefix_tokens;
        if (tok == 0) return false;
        const int64_t nreq = t.req_off[n + 1] - t.req_off[n];
        const double saved = (double)((below - 1) * tok * head_tok_bytes) / o.reread_factor;
        const int64_t pages = (tok + cap::kPage - 1) / cap::kPage;
        const int64_t chunks = estimate_chunks(pages);
        const double added_partial = (double)(2 * nreq * G * partial_row_bytes * chunks);
        const int64_t row_groups = (nreq + reqs_per_item(nreq) - 1) / reqs_per_item(nreq);
        const double added_items = (double)(chunks * row_groups) * item_bytes;
        return saved > (double)o.share_margin * added_partial + added_items;
    }

    // Depth-first walk in node order (preorder, children in order): each node
    // either is shared -- one group of every request below it streams its
    // pages and those of the folded nodes above it -- or folds, and its pages
    // ride along as a prefix of its children's runs (the requests that end at
    // it form a group of their own).  A group keeps its node chain as links,
    // not a copy of its pages.
    void build_groups_once()
    {
        sc.groups.clear();
        sc.links.clear();
        sc.frames.clear();
        for (int n = t.N - 1; n >= 0; --n)
            if (t.parent[n] == -1) sc.frames.push_back({n, -1, 0});
        while (!sc.frames.empty()) {
            const PlanScratch::Frame f = sc.frames.back();
            sc.frames.pop_back();
            const int n = f.node;
            const int32_t link = (int32_t)sc.links.size();
            sc.links.push_back({n, f.chain});
            const int32_t prefix_pages = f.chain >= 0 ? chain_pages(f.chain) : 0;
            const int32_t npages = prefix_pages + node_pages(n);
            const int64_t tok = f.prefix_tokens + t.ntok[n];
            const bool share = decide_share(n, f.prefix_tokens);
            const int32_t *reqs = share ? &t.req_list[t.req_off[n]] : t.end_list.data() + t.end_off[n];
            const int32_t nreq = share ? t.req_off[n + 1] - t.req_off[n] : t.end_off[n + 1] - t.end_off[n];
            if (npages > 0 && nreq > 0) sc.groups.push_back({reqs, nreq, link, npages, n});
            const std::vector<int32_t> &ch = t.children[n];
            for (size_t i = ch.size(); i-- > 0;)
                sc.frames.push_back(share ? PlanScratch::Frame{ch[i], -1, 0} : PlanScratch::Frame{ch[i], link, tok});
        }
    }

    int32_t chain_pages(int32_t link) const
    {
        int32_t np = 0;
        for (; link >= 0; link = sc.links[link].prev) np += node_pages(sc.links[link].node);
        return np;
    }

    // Page-stream entries of a group's run, root-first, appended at out.
    int32_t *group_entries(const PlanGroup &g, int32_t *out)
    {
        sc.nodes.clear();
        for (int32_t link = g.chain; link >= 0; link = sc.links[link].prev) sc.nodes.push_back(sc.links[link].node);
        for (size_t i = sc.nodes.size(); i-- > 0;) out = node_entries(sc.nodes[i], out);
        return out;
    }

    void build_groups()
    {
        // first pass with a provisional item size, then size items so that
        // the total cost fills every CU about `rounds` times, and plan again
        // (the share/fold test depends on the split)
        for (int pass = 0; pass < 2; ++pass) {
            build_groups_once();
            double W = 0;   // total cost if nothing were split
            for (const PlanGroup &g : sc.groups) {
                const int64_t rg = (g.nreq + reqs_per_item(g.nreq) - 1) / reqs_per_item(g.nreq);
                W += (double)g.npages * rg * Hkv * page_cost(is_shared(g.nreq));
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
    if (o.item_us == 0.f) o.item_us = 4.7f;
    if (o.reread_factor == 0.f) o.reread_factor = 3.0f;
}

cap_status check_opts(const cap_plan_opts *opts_in, cap_plan_opts &o)
{
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
    if (!std::isfinite(o.item_us) || !(o.reread_factor >= 1.f) || !std::isfinite(o.reread_factor))
        return fail(CAP_ERR_INVALID_ARG, "item_us must be finite and reread_factor finite and >= 1");
    return CAP_OK;
}

// Copy `bytes` bytes into the image at `off` and zero the rest of the region
// up to `end` (the alignment gap before the next region).
void put(std::vector<unsigned char> &img, size_t off, const void *src, size_t bytes, size_t end)
{
    if (bytes) std::memcpy(img.data() + off, src, bytes);
    std::memset(img.data() + off + bytes, 0, end - off - bytes);
}

// The whole plan for `tree` into `p`, whose vectors keep their capacity from
// earlier plans (nothing is allocated once they are large enough).
void build_plan(cap_plan *p, const cap_tree *tree, const cap_plan_opts &o)
{
    const auto t0 = std::chrono::steady_clock::now();
    PlanScratch &sc = p->scratch;
    p->tree = tree;
    p->dev = nullptr;
    p->stats = cap_plan_stats{};
    p->work_queue = o.item_dispatch == 1;
    p->items.clear();
    p->stream.clear();
    p->rows.clear();
    p->merge_off.clear();
    p->slot_rows.clear();
    p->patch.clear();
    const int Hkv = tree->attn.num_kv_heads, Hq = tree->attn.num_q_heads, D = tree->attn.head_dim;
    Planner pl(*tree, o, sc);
    pl.build_groups();

    // tasks: (page run, request subgroup); balanced splits of both.  Partial
    // slots are assigned once the dispatch sequence is fixed.
    std::vector<PlanTask> &tasks = sc.tasks;
    tasks.clear();
    p->leaf.assign(tree->R, cap_plan::Leaf{});
    sc.grp_leaf.assign(sc.groups.size(), -1);   // request whose leaf run the group is
    size_t stream_len = 0, rows_len = 0;
    for (const PlanGroup &g : sc.groups) {
        stream_len += g.npages + (g.nreq == 1 ? o.append_slack : 0);
        rows_len += g.nreq;
    }
    p->stream.resize(stream_len);
    p->rows.resize(rows_len);
    int32_t so = 0, ro = 0;
    for (size_t gi = 0; gi < sc.groups.size(); ++gi) {
        const PlanGroup &g = sc.groups[gi];
        const int64_t npg = g.npages;
        const int nreq = g.nreq;
        const bool shared = pl.is_shared(nreq);
        const int64_t k = pl.chunks(npg, shared);
        const int rg = (nreq + pl.reqs_per_item(nreq) - 1) / pl.reqs_per_item(nreq);
        const int32_t so0 = so;
        so = (int32_t)(pl.group_entries(g, p->stream.data() + so) - p->stream.data());
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
                lf.end = so;
                lf.limit = lf.end + o.append_slack;
                std::fill(p->stream.begin() + so, p->stream.begin() + so + o.append_slack, 0);
                so += o.append_slack;
                sc.grp_leaf[gi] = r;
            }
        }
        const int32_t ro0 = ro;
        std::copy(g.reqs, g.reqs + nreq, p->rows.begin() + ro);
        ro += nreq;
        for (int64_t ci = 0; ci < k; ++ci) {
            const int64_t pb = npg * ci / k, pe = npg * (ci + 1) / k;
            for (int ri = 0; ri < rg; ++ri) {
                const int rb = (int)((int64_t)nreq * ri / rg), re = (int)((int64_t)nreq * (ri + 1) / rg);
                tasks.push_back(PlanTask{(int32_t)(so0 + pb), (int32_t)(pe - pb), ro0 + rb, re - rb, -1, shared,
                                         (double)(pe - pb) * pl.page_cost(shared), (int32_t)tasks.size(),
                                         (int32_t)gi});
            }
        }
    }
    p->stream.resize(so);
    // The hardware starts workgroups in item order as CUs free up, so a list
    // sorted costliest first is greedy longest-processing-time scheduling.
    // order 1 interleaves the two kinds evenly (each costliest first), 2 sorts
    // both kinds together, 3 puts every shared item first, 4 starts with one
    // shared and one private workgroup per CU.  One item per task and KV head,
    // the heads of a task back to back.
    std::stable_sort(tasks.begin(), tasks.end(), [&](const PlanTask &a, const PlanTask &b) {
        if (o.order == 3 && a.shared != b.shared) return a.shared;
        return a.cost > b.cost;
    });
    std::vector<PlanTask> &seq = sc.seq;
    seq.clear();
    if (o.order == 1 || o.order == 4) {
        std::vector<const PlanTask *> sh, pr;
        for (const PlanTask &tk : tasks) (tk.shared ? sh : pr).push_back(&tk);
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
        auto less = [](const PlanTask &a, const PlanTask &b) {
            return a.cost < b.cost || (a.cost == b.cost && a.idx > b.idx);
        };
        std::vector<PlanTask> &heap = sc.heap;
        heap.assign(tasks.begin(), tasks.end());
        std::make_heap(heap.begin(), heap.end(), less);
        double remaining = 0;
        for (const PlanTask &tk : tasks) remaining += tk.cost;
        const double slots = 2.0 * o.num_cus / std::max(1, Hkv);   // task slots: Hkv items each
        // when every task already starts in the first round, a cut cannot
        // shorten the step: it only adds an item and a partial row
        const bool cut = (double)tasks.size() > slots;
        while (!heap.empty()) {
            std::pop_heap(heap.begin(), heap.end(), less);
            PlanTask tk = heap.back();
            heap.pop_back();
            const double cap_cost = remaining / (slots * o.tail_factor);
            const int32_t cap_pages = std::max<int32_t>(o.tail_min_pages, (int32_t)(cap_cost / pl.page_cost(false)));
            if (cut && !tk.shared && tk.np > cap_pages + o.tail_min_pages) {
                PlanTask rest = tk;
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
    for (const PlanTask &tk : seq)
        for (int q = 0; q < tk.nr; ++q) ++p->merge_off[p->rows[tk.ro + q] + 1];
    int32_t maxp = 0;
    for (int r = 0; r < tree->R; ++r) {
        maxp = std::max<int32_t>(maxp, p->merge_off[r + 1]);
        p->merge_off[r + 1] += p->merge_off[r];
    }
    const int32_t slot_rows = p->merge_off[tree->R];
    sc.fill.assign(p->merge_off.begin(), p->merge_off.end() - 1);
    int32_t max_pages = 0;
    for (PlanTask &tk : seq) {
        tk.sb = (int32_t)p->slot_rows.size();
        for (int q = 0; q < tk.nr; ++q) p->slot_rows.push_back(sc.fill[p->rows[tk.ro + q]]++);
        max_pages = std::max<int32_t>(max_pages, tk.np);
    }
    for (const PlanTask &tk : seq) {
        const int32_t r = sc.grp_leaf[tk.grp];
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
    // cap_plan_refresh stages its word patches in, which is not uploaded)
    p->off_items = 0;
    p->off_stream = align_up(p->items.size() * sizeof(cap::DevItem));
    p->off_rows = p->off_stream + align_up(p->stream.size() * 4);
    p->off_srows = p->off_rows + align_up(p->rows.size() * 4);
    p->off_moff = p->off_srows + align_up(p->slot_rows.size() * 4);
    p->off_cnt = p->off_moff + align_up(p->merge_off.size() * 4);
    p->off_queue = p->off_cnt + align_up((size_t)tree->R * Hkv * 4);
    p->off_patch = p->off_queue + align_up(cap::kQueueInts * 4);
    p->patch_cap = (size_t)4 * tree->R * (Hkv + 1) + 256;
    p->dev_bytes = p->off_patch + align_up(p->patch_cap * 8);
    p->host_image.resize(p->dev_bytes);
    {
        // the Hkv items of a task differ only in their KV head
        cap::DevItem *di = reinterpret_cast<cap::DevItem *>(p->host_image.data() + p->off_items);
        for (size_t i = 0; i < p->items.size(); i += Hkv) {
            cap::DevItem d = dev_item(*p, p->items[i]);
            for (int h = 0; h < Hkv; ++h) {
                d.head = h;
                di[i + h] = d;
            }
        }
        const size_t ib = p->items.size() * sizeof(cap::DevItem);
        std::memset(p->host_image.data() + ib, 0, p->off_stream - ib);
    }
    put(p->host_image, p->off_stream, p->stream.data(), p->stream.size() * 4, p->off_rows);
    put(p->host_image, p->off_rows, p->rows.data(), p->rows.size() * 4, p->off_srows);
    put(p->host_image, p->off_srows, p->slot_rows.data(), p->slot_rows.size() * 4, p->off_moff);
    put(p->host_image, p->off_moff, p->merge_off.data(), p->merge_off.size() * 4, p->off_cnt);
    std::memset(p->host_image.data() + p->off_cnt, 0, p->off_patch - p->off_cnt);

    cap_plan_stats &s = p->stats;
    s.num_items = (int64_t)p->items.size();
    s.num_shared_items = 0;
    for (const WorkItem &w : p->items) s.num_shared_items += w.mode == cap::kModeShared;
    s.num_tasks = (int64_t)seq.size();
    s.num_groups = (int64_t)sc.groups.size();
    s.partial_rows = slot_rows;
    const size_t slots = (size_t)slot_rows * Hq;
    s.workspace_bytes = (int64_t)(align_up(slots * D * 2) + 2 * align_up(slots * 4) + align_up(slots * D * 4));
    s.plan_device_bytes = (int64_t)p->dev_bytes;
    s.tree_device_bytes = (int64_t)align_up(std::max<size_t>(tree->page_ids.size(), 1) * 4);
    const int64_t page_bytes = 2LL * cap::kPage * D * 2;   // K+V of one page, one head
    int64_t streamed = 0;
    for (const PlanTask &tk : seq) streamed += (int64_t)tk.np * page_bytes * Hkv;
    s.kv_bytes_streamed = streamed;
    s.kv_bytes_unique = tree->unique_tokens * 4LL * D * Hkv;
    s.kv_bytes_unshared = tree->sum_ctx * 4LL * D * Hkv;
    s.partial_bytes = (int64_t)slots * (2LL * D + 8);
    s.max_partials_per_request = maxp;
    s.max_pages_per_item = max_pages;
    s.plan_host_us = std::chrono::duration<double, std::micro>(std::chrono::steady_clock::now() - t0).count();
}

}  // namespace

extern "C" {

void cap_plan_opts_default(cap_plan_opts *opts)
{
    if (!opts) return;
    std::memset(opts, 0, sizeof *opts);
    opts->share_mode = -1;
    fill_defaults(*opts);
}

cap_status cap_plan_step(const cap_tree *tree, const cap_plan_opts *opts_in, cap_plan **out)
{
    if (!tree || !out) return fail(CAP_ERR_INVALID_ARG, "NULL argument");
    *out = nullptr;
    const auto t0 = std::chrono::steady_clock::now();
    cap_plan_opts o;
    cap_status st = check_opts(opts_in, o);
    if (st != CAP_OK) return st;
    cap_plan *p = new (std::nothrow) cap_plan();
    if (!p) return fail(CAP_ERR_INVALID_ARG, "out of host memory");
    build_plan(p, tree, o);
    p->stats.plan_host_us = std::chrono::duration<double, std::micro>(std::chrono::steady_clock::now() - t0).count();
    *out = p;
    return CAP_OK;
}

cap_status cap_plan_rebuild(cap_plan *plan, const cap_tree *tree, const cap_plan_opts *opts_in)
{
    if (!plan || !tree) return fail(CAP_ERR_INVALID_ARG, "NULL argument");
    const auto t0 = std::chrono::steady_clock::now();
    cap_plan_opts o;
    cap_status st = check_opts(opts_in, o);
    if (st != CAP_OK) return st;
    build_plan(plan, tree, o);
    plan->stats.plan_host_us =
        std::chrono::duration<double, std::micro>(std::chrono::steady_clock::now() - t0).count();
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
    hipError_t e = hipMemcpyAsync(dev_buf, plan->host_image.data(), plan->off_patch,
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

void cap_plan_free(cap_plan *plan) { delete plan; }

}  // extern "C"
