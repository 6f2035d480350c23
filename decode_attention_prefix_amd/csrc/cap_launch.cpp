// cap_launch.cpp -- host side of libcap: the entry points that launch
// kernels (decode, merge, the fused step, K/V growth, the wide-row workloads
// and the measurement helpers): argument checks and kernel arguments.
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
#include "cap_host_internal.h"

using namespace cap::host;

extern "C" {

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

// Partial workspace: o / l [slots][D] fp16 | m [slots] | l [slots] | o / l
// [slots][D] fp32 for the groups whose fp16 form is not finite; each region
// starts on a 256-byte boundary.
static cap_status split_workspace(const cap_plan *p, const void *ws, size_t ws_bytes, uint16_t **o,
                                  float **m, float **l, float **w)
{
    if ((size_t)p->stats.workspace_bytes > ws_bytes || (reinterpret_cast<uintptr_t>(ws) & (kAlign - 1)))
        return fail(CAP_ERR_WORKSPACE, "workspace: %zu bytes given, %lld needed (256-byte aligned)",
                    ws_bytes, (long long)p->stats.workspace_bytes);
    const size_t slots = (size_t)p->stats.partial_rows * p->tree->attn.num_q_heads;
    const size_t o_bytes = align_up(slots * p->tree->attn.head_dim * 2);
    const size_t s_bytes = align_up(slots * 4);
    char *b = (char *)ws;
    *o = (uint16_t *)b;
    *m = (float *)(b + o_bytes);
    *l = (float *)(b + o_bytes + s_bytes);
    *w = (float *)(b + o_bytes + 2 * s_bytes);
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
    cap_status st = split_workspace(plan, workspace, ws_bytes, &a.part_o, &a.part_m, &a.part_l, &a.part_w);
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

cap_status cap_bench_decode_timed(const cap_plan *plan, const void *q, const void *k_pool, const void *v_pool,
                                  void *workspace, size_t ws_bytes, cap_stream_t stream, float *us)
{
    if (!us) return fail(CAP_ERR_INVALID_ARG, "NULL argument");
    cap::DecodeArgs a;
    cap_status st = decode_args(plan, q, k_pool, v_pool, workspace, ws_bytes, a);
    if (st != CAP_OK) return st;
    hipEvent_t e0 = nullptr, e1 = nullptr;
    hipError_t he = hipEventCreate(&e0);
    if (he == hipSuccess) he = hipEventCreate(&e1);
    int e = he == hipSuccess ? cap::launch_decode(a, plan->tree->attn.head_dim, stream, e0, e1) : 0;
    if (he == hipSuccess && e == 0) he = hipEventSynchronize(e1);
    float ms = 0.f;
    if (he == hipSuccess && e == 0) he = hipEventElapsedTime(&ms, e0, e1);
    if (e0) (void)hipEventDestroy(e0);
    if (e1) (void)hipEventDestroy(e1);
    if (e != 0) return fail(CAP_ERR_HIP, "decode launch failed: %s", cap::hip_error_string(e));
    if (he != hipSuccess) return fail(CAP_ERR_HIP, "timing events: %s", hipGetErrorString(he));
    *us = ms * 1000.f;
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

static_assert(CAP_NOALLOC_WORKSPACE_BYTES == cap::kScratchBytes, "static workspace size");

cap_status cap_decode_step_noalloc(const cap_plan *plan, const void *q, const void *k_pool, const void *v_pool,
                                   void *out, cap_stream_t stream)
{
    if (!plan) return fail(CAP_ERR_INVALID_ARG, "NULL argument");
    if ((uint64_t)plan->stats.workspace_bytes > cap::kScratchBytes)
        return fail(CAP_ERR_UNSUPPORTED, "the plan needs a %lld-byte partial workspace; the static one holds %zu "
                    "(use cap_decode_step with a caller workspace)", (long long)plan->stats.workspace_bytes,
                    cap::kScratchBytes);
    void *ws = nullptr;
    const int e = cap::scratch_address(&ws);
    if (e != 0) return fail(CAP_ERR_HIP, "static workspace lookup failed: %s", cap::hip_error_string(e));
    return cap_decode_step(plan, q, k_pool, v_pool, ws, cap::kScratchBytes, out, stream);
}

cap_status cap_merge_partials(const cap_plan *plan, const void *workspace, size_t ws_bytes, void *out,
                              cap_stream_t stream)
{
    if (!plan || !workspace || !out) return fail(CAP_ERR_INVALID_ARG, "NULL argument");
    if (!plan->dev) return fail(CAP_ERR_STATE, "plan not uploaded (call cap_plan_upload first)");
    if ((uintptr_t)out & 15) return fail(CAP_ERR_INVALID_ARG, "out must be 16-byte aligned");
    cap::MergeArgs a{};
    uint16_t *o;
    float *m, *l, *w;
    cap_status st = split_workspace(plan, workspace, ws_bytes, &o, &m, &l, &w);
    if (st != CAP_OK) return st;
    const char *d = static_cast<const char *>(plan->dev);
    a.merge_off = reinterpret_cast<const int32_t *>(d + plan->off_moff);
    a.part_o = o;
    a.part_m = m;
    a.part_l = l;
    a.part_w = w;
    a.out = static_cast<uint16_t *>(out);
    a.R = plan->tree->R;
    a.Hq = plan->tree->attn.num_q_heads;
    const int e = cap::launch_merge(a, plan->tree->attn.head_dim, stream);
    if (e != 0) return fail(CAP_ERR_HIP, "merge launch failed: %s", cap::hip_error_string(e));
    return CAP_OK;
}


// ------------------------------------------------------- wide-row workloads

// Auto mode takes the pipelined schedule where it measured faster than one
// row per workgroup: LayerNorm rows of 8K-16K values with 16-byte accesses
// (3-15% faster; gamma and beta stay in registers across a workgroup's
// rows), with rows enough to give every resident workgroup two.  Softmax
// keeps one row per workgroup (as fast or faster from 8K to 32K), and so do
// rows of 4K values and less (where a row's latency, not bandwidth, decides).
static bool auto_pipelined(const cap::RowArgs &a, bool vec4)
{
    return vec4 && a.kind == cap::kRowLayerNorm && a.width >= 8192 && a.width <= 16384 && a.rows >= 1024;
}

static cap_status rows_launch(cap::RowArgs &a, int32_t mode, cap_stream_t stream)
{
    if (!a.x || !a.y) return fail(CAP_ERR_INVALID_ARG, "NULL argument");
    if (a.rows < 0 || a.width < 1) return fail(CAP_ERR_INVALID_ARG, "rows %lld / width %lld out of range",
                                             (long long)a.rows, (long long)a.width);
    if (mode < 0 || mode > 3) return fail(CAP_ERR_INVALID_ARG, "mode %d not in {0, 1, 2, 3}", mode);
    if (a.rows > std::numeric_limits<int32_t>::max())
        return fail(CAP_ERR_UNSUPPORTED, "%lld rows: at most 2^31 - 1", (long long)a.rows);
    if (a.width > ((int64_t)1 << 24))
        return fail(CAP_ERR_UNSUPPORTED, "width %lld above 2^24", (long long)a.width);
    if ((mode == 1 || mode == 3) && a.width > cap::kMaxRetainedWidth)
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
    const bool retained = mode == 1 || mode == 3 || (mode == 0 && a.width <= (vec4 ? cap::kMaxRetainedWidth : 16384));
    a.pipelined = (mode == 3 || (mode == 0 && auto_pipelined(a, vec4))) ? 1 : 0;
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

cap_status cap_bench_copy_stream(void *dst, const void *src, size_t bytes, size_t run_bytes, cap_stream_t stream)
{
    if (!dst || !src || bytes == 0 || (bytes & 15) || (((uintptr_t)dst | (uintptr_t)src) & 15))
        return fail(CAP_ERR_INVALID_ARG, "copy: bad buffer or size");
    if (run_bytes == 0) run_bytes = (size_t)256 << 10;
    if (run_bytes & 15) return fail(CAP_ERR_INVALID_ARG, "copy: run_bytes must be a multiple of 16");
    const int e = cap::launch_copy_stream(dst, src, bytes / 16, run_bytes / 16, stream);
    return e ? fail(CAP_ERR_HIP, "copy launch failed: %s", cap::hip_error_string(e)) : CAP_OK;
}

}  // extern "C"
