// cap_internal.h -- structures shared by the host side of libcap and its
// HIP kernels.  Not part of the public ABI.
#pragma once

#include <stdint.h>

#include "../../include/cap.h"

namespace cap {

// Layout constants of the paged KV cache.
constexpr int kPage = 16;            // tokens per page
constexpr int kWaveSize = 64;        // CDNA wavefront
constexpr int kWaves = 4;            // waves per decode workgroup
constexpr int kSharedThreads = kWaves * kWaveSize;
constexpr int kPrivateRows = 16;     // query rows of a private (one-wave) item
constexpr int kSharedRows = 32 * kWaves;  // query rows of a shared item: 32 per wave
constexpr int kRowsPerItem = 32;     // the GQA group must divide this
constexpr int kMaxSharedPages = 128;  // a shared item's waves keep its page table in two registers, one page per lane each
constexpr int kMaxPrivatePages = 64 * kWaves; // a private item: 64 pages per wave
constexpr int kModePrivate = 0, kModeShared = 1;

// A run of KV pages of one KV head applied to nreq requests x G query heads,
// run by one workgroup: up to 16 rows and kMaxPrivatePages pages for a
// private item, up to kSharedRows rows and 64 pages for a shared item.  Same
// layout as cap_work_item.
struct WorkItem {
    int32_t stream_off;
    int32_t npages;
    int32_t head;
    int32_t row_off;
    int32_t nreq;
    int32_t slot_base;
    int32_t mode;                // kModePrivate / kModeShared
    int32_t reserved;
};
static_assert(sizeof(WorkItem) == sizeof(cap_work_item), "work item layout");

// Device form of a work item: the fields above plus what lets a workgroup
// issue its first K/V and Q loads right after reading the item, without
// first reading the page stream and the row table (each a dependent trip to
// memory).
constexpr int kInlineEntries = 16;
constexpr int kInlinePerWave = kInlineEntries / kWaves;   // private items: per wave
struct DevItem {
    int32_t stream_off;
    int32_t npages;
    int32_t head;
    int32_t row_off;
    int32_t nreq;
    int32_t slot_base;
    int32_t mode;
    int32_t req0;               // first request id when the item's requests are consecutive ids, else -1
    // page-stream entries of the first pages: private items, pages
    // 0 .. kInlinePerWave - 1 of wave w's sub-stream at [kInlinePerWave * w ..];
    // shared items, pages 0 .. kInlineEntries - 1 (0 past the end)
    int32_t ent[kInlineEntries];
};

constexpr int kQueues = 8;            // one per XCD (workgroup b runs on XCD b mod 8)
constexpr int kQueueStride = 64;      // ints: one 256-byte line per counter
constexpr int kQueueInts = (kQueues + 1) * kQueueStride;

struct DecodeArgs {
    const DevItem *items;          // one workgroup each
    const int32_t *stream;       // page-stream entries: (physical page << 5) | (ntok - 1)
    const int32_t *rows;         // request ids of each item's request list
    const int32_t *slot_rows;    // partial row of each item request: slot_rows[slot_base + q]
    const uint16_t *q;           // [R][Hq][D] bf16
    const uint16_t *k_pool;      // [pages][Hkv][D/8][16][8] bf16
    const uint16_t *v_pool;      // [pages][Hkv][D][16] bf16
    uint16_t *part_o;            // [slots][D] fp16: o / l (the normalised partial output)
    float *part_m;               // [slots]
    float *part_l;               // [slots]
    float *part_w;               // [slots][D] fp32: o / l of each 4-dim group whose fp16 form is not
                                 // finite (written only for those groups)
    int32_t n_items;             // the grid never exceeds it
    int32_t Hq, Hkv, G;
    int32_t log2G;               // G is a power of two: row / G = row >> log2G
    float scale_log2;            // sm_scale * log2(e)
    // work queues (nullptr: one workgroup per item): kQueues counters of items
    // handed out, then the count of finished workgroups, each kQueueStride
    // ints apart; zero between launches
    int32_t *queue;
    // fused step only (counters == nullptr: partials are left for merge_kernel)
    int32_t *counters;           // [R][Hkv] arrival counts, zero between steps
    const int32_t *merge_off;    // [R+1]: request r's partial rows are merge_off[r] .. merge_off[r+1] - 1
    uint16_t *out;               // [R][Hq][D] bf16
    int32_t slots;               // partial slots (fused: slots * D * 2 < 2^31)
};

struct MergeArgs {
    const int32_t *merge_off;    // [R+1]: request r's partial rows are merge_off[r] .. merge_off[r+1] - 1
    const uint16_t *part_o;      // fp16 o / l
    const float *part_m;
    const float *part_l;
    const float *part_w;         // fp32 o / l of the groups whose fp16 form is not finite
    uint16_t *out;               // [R][Hq][D] bf16
    int32_t R, Hq;
};

// New tokens' K/V written into their pool slots.
struct AppendArgs {
    const int32_t *dest;         // [n]: (physical page << 4) | slot; negative = skip
    int32_t n;
    const uint16_t *k_new;       // [n][Hkv][D] bf16
    const uint16_t *v_new;       // [n][Hkv][D] bf16
    uint16_t *k_pool;            // [pages][Hkv][D/8][16][8]
    uint16_t *v_pool;            // [pages][Hkv][D][16]
    int32_t Hkv, D;
    int64_t pool_pages;          // entries with a page at or past this are skipped
};

// Wide-row reduction-reuse workloads (cap_rows.hip).
constexpr int kRowSoftmax = 0, kRowLayerNorm = 1;
constexpr int64_t kMaxRetainedWidth = 65536;   // one row in one workgroup's registers
struct RowArgs {
    const float *x;              // [rows][width]
    const float *gamma, *beta;   // [width] (LayerNorm)
    float *y;                    // [rows][width]
    int64_t rows, width;
    float eps;
    int32_t kind;
    int32_t pipelined;           // retained schedule: 1 = several rows per workgroup, the next one in flight
};

// Kernel launchers (cap_kernels.hip, cap_aux.hip, cap_rows.hip); return the
// hipError_t as int.
// ev_start / ev_stop (hipEvent_t, or null): events bound to the launch's own
// dispatch (hipExtLaunchKernel), which time the kernel's execution alone
int launch_decode(const DecodeArgs &a, int head_dim, void *stream, void *ev_start = nullptr,
                  void *ev_stop = nullptr);
int launch_merge(const MergeArgs &a, int head_dim, void *stream);
// The static partial workspace of cap_decode_step_noalloc (cap_kernels.hip):
// its device address on the current device (looked up on the first call per
// device).
constexpr size_t kScratchBytes = (size_t)64 << 20;
int scratch_address(void **ptr);
int launch_fill(void *buf, size_t words, uint32_t value, void *stream);
int launch_patch(void *base, const uint32_t *patch, int n, void *stream);
int launch_append(const AppendArgs &a, void *stream);
int launch_rows(const RowArgs &a, bool vec4, bool retained, void *stream);
int launch_read_stream(const void *buf, size_t vec16, void *sink, void *stream);
int launch_read(const void *buf, size_t vec16, void *sink, void *stream);
int launch_copy(void *dst, const void *src, size_t vec16, void *stream);
int launch_copy_stream(void *dst, const void *src, size_t vec16, size_t run16, void *stream);
const char *hip_error_string(int err);

}  // namespace cap
