// cap_host_internal.h -- host-side state of libcap shared by its host
// sources (cap_tree.cpp, cap_plan.cpp, cap_launch.cpp).  Not part of the
// public ABI.
#pragma once

#include <stddef.h>
#include <stdint.h>

#include <string>
#include <vector>

#include "cap_internal.h"

namespace cap {
namespace host {

// Record a formatted message for cap_last_error() and return `st`.
cap_status fail(cap_status st, const char *fmt, ...);

constexpr size_t kAlign = 256;
constexpr int64_t kMaxPoolPages = (int64_t)1 << 26;   // page-stream entry: (page << 5) | (ntok - 1)
inline size_t align_up(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }

}  // namespace host
}  // namespace cap

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

namespace cap {
namespace host {

// The planner's working memory, kept with a plan so that planning again into
// the same handle (cap_plan_rebuild) reuses it instead of allocating.
struct PlanGroup {
    const int32_t *reqs;           // its requests (sorted ids, in the tree's node -> request tables)
    int32_t nreq;
    int32_t chain;                 // last entry of its node chain (links, root-first by following prev)
    int32_t npages;
    int32_t at;                    // node whose pages end the run
};
struct ChainLink {
    int32_t node, prev;            // prev: the link of the folded node above (-1: none)
};
struct PlanTask {
    int32_t so, np, ro, nr, sb;
    bool shared;
    double cost;
    int32_t idx, grp;
};
struct PlanScratch {
    std::vector<PlanGroup> groups;
    std::vector<ChainLink> links;
    std::vector<PlanTask> tasks, seq, heap;
    std::vector<int32_t> grp_leaf, fill, nodes;
    struct Frame {
        int32_t node, chain;
        int64_t prefix_tokens;
    };
    std::vector<Frame> frames;
};

}  // namespace host
}  // namespace cap

struct cap_plan {
    const cap_tree *tree = nullptr;
    cap::host::PlanScratch scratch;
    cap_plan_stats stats{};
    std::vector<cap::WorkItem> items;          // one workgroup each
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

namespace cap {
namespace host {

// Tables derived from parent, ntok and the request paths (cap_tree.cpp).
void derive(cap_tree &t);

// Device form of a work item (cap_plan.cpp).
DevItem dev_item(const cap_plan &p, const WorkItem &w);

}  // namespace host
}  // namespace cap
