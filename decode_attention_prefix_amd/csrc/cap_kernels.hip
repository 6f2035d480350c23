// cap_kernels.hip -- gfx950 (CDNA4) kernels of libcap.
//
// decode_kernel: a 4-wave workgroup per work item (or, with work queues, two
// resident workgroups per CU taking items in turn).  A work item is a run of
// KV pages of one KV head together with the query rows (requests x GQA
// heads) that read those pages, so the pages come from HBM once for the
// whole row group -- the point of the Capillary Kernels project page
// (abstract, first paragraph): shared prefixes should not be fetched once per
// request.  Private items (<= 16 rows) stream pages straight into VGPRs,
// their 4 waves splitting the pages; shared items (<= 128 rows) stream each
// step into an LDS ring with global->LDS loads and every wave applies it to
// its own 32 rows.  Both contractions run on the matrix cores with
// v_mfma_f32_16x16x32_bf16:
//
//   S^T[16 tokens x 16 rows] = K_page[16 x D] . Q^T[D x 16]     (D/32 MFMAs per page)
//   O^T[16 dims  x 16 rows] += V^T[16 dims x 32 tokens] . P^T   (D/16 MFMAs per 2 pages)
//
// K pages are [D/8][16][8] (a lane's 8 dims of one token are 16 contiguous
// bytes; the 16 tokens of one dim chunk are a contiguous 256-byte line), V
// pages are [D][16] (tokens contiguous per dim).  The PV k-order maps lane
// group c to tokens 8(c & 1)..+7 of page c >> 1, so a lane's V operand is
// one 16-byte piece of a page row; the probabilities, which the QK MFMA
// leaves as tokens 4c..4c+3 of both pages, are moved to that order with two
// lane swaps per register pair.
//
// A workgroup reads its item once into registers; the item carries its first
// page ids and its first request id, so the first K/V and Q loads need no
// other table.  Softmax is online in base 2 (scale folded with log2 e, exp
// via v_exp_f32) with a lazily moved per-row reference maximum.  Each item
// writes (m, l, o/l) for its rows into write-once partial rows (each
// request's rows one contiguous block); merge_kernel (or, in the fused
// step, the item that completes a request) combines the partials of each
// (request, head) with log-sum-exp rescaling -- the partial-result
// combination of the project page's second paragraph, through global
// memory/L2 because CDNA4 has no cross-CU shared memory.
#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>

#include <algorithm>
#include <mutex>

#include "cap_internal.h"

namespace cap {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

__device__ __forceinline__ u32x4 ld16(const uint16_t *p)
{
    return *reinterpret_cast<const u32x4 *>(p);
}

// K/V pages are read once per item: non-temporal loads (the nt cache policy:
// streamed, not kept in L2).  A read-only probe streams ~12% faster with
// them (7.1 vs 6.3 TB/s with per-workgroup contiguous runs).
constexpr bool kKvNonTemporal = true;
constexpr int kKvDmaPolicy = 0;          // cache-policy bits of the ring's global->LDS loads

__device__ __forceinline__ u32x4 ld16_kv(const uint16_t *p)
{
    if constexpr (kKvNonTemporal)
        return __builtin_nontemporal_load(reinterpret_cast<const u32x4 *>(p));
    else
        return *reinterpret_cast<const u32x4 *>(p);
}

__device__ __forceinline__ f32x4 mfma(u32x4 a, u32x4 b, f32x4 c)
{
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                   __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}

__device__ __forceinline__ float fast_exp2(float x)
{
    return __builtin_amdgcn_exp2f(x);
}

// Rows rescale their accumulators only when their maximum logit (base-2
// units) exceeds the reference they were accumulated against by more than
// this; otherwise p = 2^(x - m_ref) <= 2^8 stays exact enough in fp32 and
// bf16, and (m_ref, l, o) is still a valid partial for any reference.
constexpr float kRescaleThreshold = 8.0f;

// One work item, read once when the workgroup starts it: the fields as
// uniform values, the inline page entries one per lane (lane i < 16: entry i).
// Later reads of the item in memory would be vector loads with a wait on every
// outstanding load (the compiler treats the ring's global->LDS loads as
// possible writes to it), so nothing reads the item twice.
struct ItemRegs {
    int stream_off, npages, head, row_off, nreq, slot_base, mode, req0;
    int lane_ent;
};

__device__ __forceinline__ ItemRegs read_item(const DevItem *items, int idx, int lane)
{
    const DevItem &d = items[idx];
    ItemRegs r;
    r.stream_off = d.stream_off;
    r.npages = d.npages;
    r.head = d.head;
    r.row_off = d.row_off;
    r.nreq = d.nreq;
    r.slot_base = d.slot_base;
    r.mode = d.mode;
    r.req0 = d.req0;
    r.lane_ent = lane < kInlineEntries ? d.ent[lane] : 0;
    // a use on every path: the wait for the record lands here, before any
    // other load of the item is issued, and no later read of an entry waits
    asm volatile("" ::"v"(r.lane_ent));
    return r;
}

// KV fragments of one 2-page step, already in MFMA operand layout.
template <int D>
struct Step {
    u32x4 k0[D / 32], k1[D / 32];   // QK A operands, page 0 / page 1
    u32x4 v[D / 16];                // PV A operands: lane (n, c) holds tokens 8(c&1)..+7 of page c>>1
    int nt0, nt1;                   // valid tokens in page 0 / page 1 (nt1 = 0: no page)
};

// Issue the loads of step s (two pages) of a private wave's sub-stream of
// `count` pages.  Page ids: the sub-stream's first kInlinePerWave pages come
// from the item itself (no wait on the page stream for the first two steps),
// later ones from the wave's page table held in lanes (lane i: raw stream
// entry of page i) via v_readlane.  Every call issues the same number of
// loads whatever the step, so the wait counts of the software pipeline stay
// the same on every path: a missing second page re-reads the first, and a
// step past the end (the pipeline's last load) points every lane at the
// first 16 bytes of Q, which this item has just read (no HBM traffic; the
// values are never used).
template <int D>
__device__ __forceinline__ void load_step(Step<D> &f, const DecodeArgs &a, const ItemRegs &it, int wave, int count,
                                          int s, int lane_e, int n, int c)
{
    const int64_t blk = (int64_t)kPage * D;             // elements per (page, head)
    const int head = it.head;
    const int nsteps = (count + 1) >> 1;
    const int ss = s < nsteps ? s : nsteps - 1;
    const int i0 = 2 * ss;
    const bool has1 = i0 + 1 < count;
    const int i1 = has1 ? i0 + 1 : i0;
    int e0, e1;
    if (i1 < kInlinePerWave) {
        e0 = __builtin_amdgcn_readlane(it.lane_ent, kInlinePerWave * wave + i0);
        e1 = __builtin_amdgcn_readlane(it.lane_ent, kInlinePerWave * wave + i1);
    } else {
        e0 = __builtin_amdgcn_readlane(lane_e, i0);
        e1 = __builtin_amdgcn_readlane(lane_e, i1);
    }
    const int64_t p0 = e0 >> 5;
    const int64_t p1 = e1 >> 5;
    f.nt0 = (e0 & 31) + 1;
    f.nt1 = has1 ? (e1 & 31) + 1 : 0;
    const bool live = s < nsteps;
    const uint16_t *kb0 = live ? a.k_pool + (p0 * a.Hkv + head) * blk : a.q;
    const uint16_t *vb0 = live ? a.v_pool + (p0 * a.Hkv + head) * blk : a.q;
    const uint16_t *kb1 = live ? a.k_pool + (p1 * a.Hkv + head) * blk : a.q;
    const uint16_t *vb1 = live ? a.v_pool + (p1 * a.Hkv + head) * blk : a.q;
    const int koff = live ? (c * kPage + n) * 8 : 0;                 // lane offsets (elements)
    const int voff = live ? n * kPage + 8 * (c & 1) : 0;
    const int kstep = live ? 4 * kPage * 8 : 0, vstep = live ? 16 * kPage : 0;
#pragma unroll
    for (int i = 0; i < D / 32; ++i) {
        f.k0[i] = ld16_kv(kb0 + koff + i * kstep);
        f.k1[i] = ld16_kv(kb1 + koff + i * kstep);
    }
    const uint16_t *vb = ((c >> 1) ? vb1 : vb0) + voff;
#pragma unroll
    for (int j = 0; j < D / 16; ++j) f.v[j] = ld16_kv(vb + j * vstep);
}

// Zero the V elements of tokens >= nt -- those slots may hold NaN, and
// 0 * NaN would poison the MFMA sum.  Lane (n, c) holds tokens
// 8(c & 1) .. 8(c & 1) + 7 of page c >> 1, two per dword.
template <int D>
__device__ __forceinline__ void mask_v(u32x4 (&v)[D / 16], int nt0, int nt1, int c)
{
    const int lim = ((c >> 1) ? nt1 : nt0) - 8 * (c & 1);
    uint32_t m[4];
#pragma unroll
    for (int e = 0; e < 4; ++e)
        m[e] = (2 * e < lim ? 0x0000FFFFu : 0u) | (2 * e + 1 < lim ? 0xFFFF0000u : 0u);
#pragma unroll
    for (int j = 0; j < D / 16; ++j) {
        v[j].x &= m[0];
        v[j].y &= m[1];
        v[j].z &= m[2];
        v[j].w &= m[3];
    }
}

// PV B operand from the packed probabilities.  The QK output leaves lane
// (n, c) with tokens 4c..4c+3 of page 0 (.xy) and of page 1 (.zw) for row n;
// the PV MFMA wants lane (n, c) to hold the 8 k-values 8c..8c+7, which this
// kernel maps to tokens 8(c & 1)..+7 of page c >> 1 -- so each lane's V
// operand is one 16-byte piece of a page row.  Moving the pieces is a 4 x 4
// exchange of dword pairs across the four 16-lane rows: a lane-half swap
// (rows 2,3 of x with rows 0,1 of y) and then a row swap (rows 1,3 of x with
// rows 0,2 of y) take rows [A0 A1 A2 A3] / [B0 B1 B2 B3] to [A0 A2 B0 B2] /
// [A1 A3 B1 B3].  One asm block, with the VALU-to-permlane wait states.
__device__ __forceinline__ u32x4 p_operand(u32x4 pw)
{
    uint32_t a0 = pw.x, a1 = pw.y, b0 = pw.z, b1 = pw.w;
    asm volatile(
        "s_nop 1\n\t"
        "v_permlane32_swap_b32 %0, %2\n\t"
        "v_permlane32_swap_b32 %1, %3\n\t"
        "s_nop 1\n\t"
        "v_permlane16_swap_b32 %0, %2\n\t"
        "v_permlane16_swap_b32 %1, %3\n\t"
        "s_nop 1"
        : "+v"(a0), "+v"(a1), "+v"(b0), "+v"(b1));
    return u32x4{a0, a1, b0, b1};
}

// max over the four lanes n, n+16, n+32, n+48 that hold one query row, with
// gfx950's lane-half swaps (VALU, no LDS round trip): swapping lane halves of
// two copies and taking the max gives an xor-32, then an xor-16 reduction.
// Written as one asm block because this compiler folds max(first result,
// second result) of the swap intrinsic to the first result; the s_nop covers
// the VALU-write-to-permlane-read wait states.
__device__ __forceinline__ float row_max4(float v)
{
    float a = v, b = v;
    asm volatile(
        "s_nop 1\n\t"
        "v_permlane32_swap_b32 %0, %1\n\t"
        "v_max_f32 %0, %0, %1\n\t"
        "v_mov_b32 %1, %0\n\t"
        "s_nop 1\n\t"
        "v_permlane16_swap_b32 %0, %1\n\t"
        "v_max_f32 %0, %0, %1"
        : "+v"(a), "+v"(b));
    return a;
}

// max of three floats as one v_max3_f32.  Written out because fmaxf on
// values the compiler cannot prove canonical costs an extra NaN-quieting
// v_max per operand; the operands here are never signalling NaNs.
__device__ __forceinline__ float vmax3(float a, float b, float c)
{
    float r;
    asm("v_max3_f32 %0, %1, %2, %3" : "=v"(r) : "v"(a), "v"(b), "v"(c));
    return r;
}

// S^T tiles of one 2-page step for up to RB 16-row blocks: lane (n, c) gets
// the logits of tokens 4c..4c+3 of page 0 (s0) and page 1 (s1) for row n.
template <int D, int RB>
__device__ __forceinline__ void qk_step(const u32x4 (&k0)[D / 32], const u32x4 (&k1)[D / 32],
                                        const u32x4 (&qf)[RB][D / 32], f32x4 (&s0)[RB], f32x4 (&s1)[RB],
                                        int nblk)
{
#pragma unroll
    for (int b = 0; b < RB; ++b) {
        s0[b] = f32x4{0.f, 0.f, 0.f, 0.f};
        s1[b] = f32x4{0.f, 0.f, 0.f, 0.f};
        if (RB == 1 || b < nblk) {
#pragma unroll
            for (int i = 0; i < D / 32; ++i) {
                s0[b] = mfma(k0[i], qf[b][i], s0[b]);
                s1[b] = mfma(k1[i], qf[b][i], s1[b]);
            }
        }
    }
}

// The rest of a step, in phases so the blocks' independent work can overlap:
// the exponent arguments x = s * scale - m_ref against each row's current
// reference, one (rare) rescale, the probabilities 2^x, then all PV MFMAs.
// The common path needs no cross-lane work: a lane only checks that none of
// its arguments exceeds the rescale threshold; the exact row maxima are taken
// (over the four lanes of a row) only when some row must move its reference
// -- the first step, or a maximum that rose by more than the threshold.
// Masking (tokens past nt, a missing second page with nt1 = 0) runs only on
// tail steps.  MASKV: also zero the V tails in registers (pool tails may hold
// anything, and 0 * NaN would poison the sums).
template <int D, int RB, bool MASKV>
__device__ __forceinline__ void softmax_pv(const f32x4 (&s0)[RB], const f32x4 (&s1)[RB], u32x4 (&v)[D / 16],
                                           int nt0, int nt1, f32x4 (&o)[RB][D / 16], float (&m_ref)[RB],
                                           float (&l_run)[RB], int nblk, float scale, int c)
{
    const bool tail = nt0 < kPage || nt1 < kPage;               // wave-uniform
    if constexpr (MASKV) {
        if (tail) mask_v<D>(v, nt0, nt1, c);
    }
    const int lim0 = nt0 - 4 * c, lim1 = nt1 - 4 * c;   // lane holds tokens 4c..4c+3
    float x[RB][8];
    bool need = false;
#pragma unroll
    for (int b = 0; b < RB; ++b) {
        const float mneg = -m_ref[b];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            x[b][j] = __builtin_fmaf(s0[b][j], scale, mneg);
            x[b][4 + j] = __builtin_fmaf(s1[b][j], scale, mneg);
        }
        // checked before masking (an unmasked tail value can at worst send the
        // step down the exact rescale path below, which masks)
        const float lm = vmax3(vmax3(x[b][0], x[b][1], x[b][2]), vmax3(x[b][3], x[b][4], x[b][5]),
                               vmax3(x[b][6], x[b][7], x[b][7]));
        need |= lm > kRescaleThreshold;                  // also true while m_ref = -inf
        if (tail) {
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                x[b][j] = j < lim0 ? x[b][j] : -INFINITY;
                x[b][4 + j] = j < lim1 ? x[b][4 + j] : -INFINITY;
            }
        }
    }
    if (__builtin_amdgcn_ballot_w64(need)) {             // wave-uniform, rare after the first step
#pragma unroll
        for (int b = 0; b < RB; ++b) {
            float y[8];
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                y[j] = (!tail || j < lim0) ? s0[b][j] * scale : -INFINITY;
                y[4 + j] = (!tail || j < lim1) ? s1[b][j] * scale : -INFINITY;
            }
            float mx = fmaxf(fmaxf(fmaxf(y[0], y[1]), fmaxf(y[2], y[3])),
                             fmaxf(fmaxf(y[4], y[5]), fmaxf(y[6], y[7])));
            mx = row_max4(mx);                           // base-2 units (scale > 0)
            const float m_new = mx > m_ref[b] + kRescaleThreshold ? mx : m_ref[b];
            const float alpha = fast_exp2(m_ref[b] - m_new);   // 1 if unchanged, 0 from -inf
            m_ref[b] = m_new;
            l_run[b] *= alpha;
#pragma unroll
            for (int j = 0; j < D / 16; ++j) o[b][j] *= alpha;
#pragma unroll
            for (int j = 0; j < 8; ++j) x[b][j] = y[j] - m_new;
        }
    }
    u32x4 pw[RB];
#pragma unroll
    for (int b = 0; b < RB; ++b) {
        float p[8];
        bf16x8 pb;
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            p[j] = fast_exp2(x[b][j]);
            pb[j] = (__bf16)p[j];
        }
        l_run[b] += ((p[0] + p[1]) + (p[2] + p[3])) + ((p[4] + p[5]) + (p[6] + p[7]));
        pw[b] = __builtin_bit_cast(u32x4, pb);
    }
#pragma unroll
    for (int b = 0; b < RB; ++b) {
        if (RB == 1 || b < nblk) {
            const u32x4 pb = p_operand(pw[b]);
#pragma unroll
            for (int j = 0; j < D / 16; ++j) o[b][j] = mfma(v[j], pb, o[b][j]);
        }
    }
}

// The shared path's step, split so that the QK MFMAs of the next step can
// sit in one basic block with this step's softmax arithmetic (the matrix
// cores then run while the vector ALUs work).  softmax_prepare holds the
// branches: tail masking of the raw logits and of V, and the (rare) move of
// a row's reference maximum, decided on the raw logits: a lane's largest
// logit times the scale may exceed the reference by at most the threshold.
template <int D>
__device__ __forceinline__ void softmax_prepare(f32x4 (&s0)[2], f32x4 (&s1)[2], u32x4 (&v)[D / 16], int nt0,
                                                int nt1, f32x4 (&o)[2][D / 16], float (&m_ref)[2],
                                                float (&l_run)[2], float scale, int c)
{
    if (nt0 < kPage || nt1 < kPage) {                    // wave-uniform: only a node's last step
        mask_v<D>(v, nt0, nt1, c);
        const int lim0 = nt0 - 4 * c, lim1 = nt1 - 4 * c;
#pragma unroll
        for (int b = 0; b < 2; ++b)
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                s0[b][j] = j < lim0 ? s0[b][j] : -INFINITY;
                s1[b][j] = j < lim1 ? s1[b][j] : -INFINITY;
            }
    }
    float lm[2];
    bool need = false;
#pragma unroll
    for (int b = 0; b < 2; ++b) {
        lm[b] = vmax3(vmax3(s0[b][0], s0[b][1], s0[b][2]), vmax3(s0[b][3], s1[b][0], s1[b][1]),
                      vmax3(s1[b][2], s1[b][3], s1[b][3]));
        need |= __builtin_fmaf(lm[b], scale, -m_ref[b]) > kRescaleThreshold;   // true while m_ref = -inf
    }
    if (__builtin_amdgcn_ballot_w64(need)) {             // wave-uniform, rare after the first step
#pragma unroll
        for (int b = 0; b < 2; ++b) {
            const float mx = row_max4(lm[b]) * scale;    // base-2 units (scale > 0)
            const float m_new = mx > m_ref[b] + kRescaleThreshold ? mx : m_ref[b];
            const float alpha = fast_exp2(m_ref[b] - m_new);   // 1 if unchanged, 0 from -inf
            m_ref[b] = m_new;
            l_run[b] *= alpha;
#pragma unroll
            for (int j = 0; j < D / 16; ++j) o[b][j] *= alpha;
        }
    }
}

// Straight-line rest of a shared step: probabilities 2^(s * scale - m_ref),
// row sums, bf16 packing and exchange, PV MFMAs.
template <int D>
__device__ __forceinline__ void softmax_finish(const f32x4 (&s0)[2], const f32x4 (&s1)[2], const u32x4 (&v)[D / 16],
                                               f32x4 (&o)[2][D / 16], const float (&m_ref)[2],
                                               float (&l_run)[2], float scale)
{
    u32x4 pb[2];
#pragma unroll
    for (int b = 0; b < 2; ++b) {
        const float mneg = -m_ref[b];
        float p[8];
        bf16x8 pk;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            p[j] = fast_exp2(__builtin_fmaf(s0[b][j], scale, mneg));
            p[4 + j] = fast_exp2(__builtin_fmaf(s1[b][j], scale, mneg));
        }
#pragma unroll
        for (int j = 0; j < 8; ++j) pk[j] = (__bf16)p[j];
        l_run[b] += ((p[0] + p[1]) + (p[2] + p[3])) + ((p[4] + p[5]) + (p[6] + p[7]));
        pb[b] = p_operand(__builtin_bit_cast(u32x4, pk));
    }
#pragma unroll
    for (int b = 0; b < 2; ++b)
#pragma unroll
        for (int j = 0; j < D / 16; ++j) o[b][j] = mfma(v[j], pb[b], o[b][j]);
}

template <int D, int RB, bool MASKV>
__device__ __forceinline__ void compute_step(Step<D> &f, const u32x4 (&qf)[RB][D / 32],
                                             f32x4 (&o)[RB][D / 16], float (&m_ref)[RB],
                                             float (&l_run)[RB], int nblk, float scale, int c)
{
    f32x4 s0[RB], s1[RB];
    qk_step<D, RB>(f.k0, f.k1, qf, s0, s1, nblk);
    softmax_pv<D, RB, MASKV>(s0, s1, f.v, f.nt0, f.nt1, o, m_ref, l_run, nblk, scale, c);
}

// Q fragments (B operand of QK) for rows row0 + 16b + n of an item: lane
// (n, c) holds dims 8(4i+c)..+7.  Rows past nrows are zero.
template <int D, int RB>
__device__ __forceinline__ void load_q(u32x4 (&qf)[RB][D / 32], const DecodeArgs &a, const ItemRegs &it,
                                       int row0, int nrows, int n, int c)
{
    const int G = a.G;
#pragma unroll
    for (int b = 0; b < RB; ++b) {
        const int row = row0 + 16 * b + n;
        if (row < nrows) {
            const int req = it.req0 >= 0 ? it.req0 + (row >> a.log2G) : a.rows[it.row_off + (row >> a.log2G)];
            const int h = it.head * G + (row & (G - 1));
            const uint16_t *qb = a.q + ((int64_t)req * a.Hq + h) * D;
#pragma unroll
            for (int i = 0; i < D / 32; ++i) qf[b][i] = ld16(qb + 8 * (4 * i + c));
        } else {
#pragma unroll
            for (int i = 0; i < D / 32; ++i) qf[b][i] = u32x4{0, 0, 0, 0};
        }
    }
}

// Partial stores and loads.  The fused step hands partials from one
// workgroup to another inside the launch, possibly across XCDs (each with
// its own L2), so there they go through buffer instructions with the sc1
// cache policy -- the device-coherent form the compiler itself uses for
// device-scope atomic stores and loads: written through the L2, read past
// any stale copy -- instead of plain stores published by a whole-L2
// write-back.  The two-launch path writes them with plain stores.
constexpr int kCoherent = 16;                    // cache-policy bits: sc1

__device__ __forceinline__ __amdgpu_buffer_rsrc_t buf_rsrc(const void *p, int bytes)
{
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(p), (short)0, bytes, 0x00020000);
}

// True when one of the fp16 values packed in `w` (two per dword) is not
// finite (exponent field all ones: inf or NaN).
__device__ __forceinline__ bool f16_pair_nonfinite(uint32_t w)
{
    return (w & 0x7C00u) == 0x7C00u || (w & 0x7C000000u) == 0x7C000000u;
}

// Four dims d..d+3 (a 4-dim group) of a partial's normalised output o / l,
// as fp16: the value is a convex combination of V rows, so |o / l| <= max |v|,
// and fp16 keeps ~3 significant digits, far inside the output tolerance, at
// half the bytes of fp32.  bf16 V can exceed fp16's range (65504); a group
// whose fp16 form is not finite is also written in fp32 to the side region
// part_w, and the merge, which sees the same non-finite fp16 bits, reads it
// from there.  So every value keeps fp32 range, and N(0,1)-scale inputs
// write no extra byte.
template <int D, bool FUSED>
__device__ __forceinline__ void store_partial_o(const DecodeArgs &a, int64_t slot, int d, f32x4 v)
{
    typedef _Float16 f16x4 __attribute__((ext_vector_type(4)));
    const f16x4 h = {(_Float16)v[0], (_Float16)v[1], (_Float16)v[2], (_Float16)v[3]};
    const u32x2 bits = __builtin_bit_cast(u32x2, h);
    const bool wide = f16_pair_nonfinite(bits.x) || f16_pair_nonfinite(bits.y);
    if constexpr (FUSED) {
        __builtin_amdgcn_raw_buffer_store_b64(bits, buf_rsrc(a.part_o, a.slots * D * 2),
                                              (int)(slot * D + d) * 2, 0, kCoherent);
        if (wide)
            __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, v),
                                                   buf_rsrc(a.part_w + slot * D, D * 4), d * 4, 0, kCoherent);
    } else {
        *reinterpret_cast<u32x2 *>(a.part_o + slot * D + d) = bits;
        if (wide) *reinterpret_cast<f32x4 *>(a.part_w + slot * D + d) = v;
    }
}

template <bool FUSED>
__device__ __forceinline__ void store_partial_ml(const DecodeArgs &a, int64_t slot, float m, float l)
{
    if constexpr (FUSED) {
        __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(uint32_t, m), buf_rsrc(a.part_m, a.slots * 4),
                                              (int)slot * 4, 0, kCoherent);
        __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(uint32_t, l), buf_rsrc(a.part_l, a.slots * 4),
                                              (int)slot * 4, 0, kCoherent);
    } else {
        a.part_m[slot] = m;
        a.part_l[slot] = l;
    }
}

// Partial row of each of a lane's rows row0 + 16b + n (read when the item
// starts; used when its partials are written).
template <int RB>
__device__ __forceinline__ void load_slot_rows(int (&srow)[RB], const DecodeArgs &a, const ItemRegs &it, int row0,
                                               int nrows, int n)
{
#pragma unroll
    for (int b = 0; b < RB; ++b) {
        const int row = row0 + 16 * b + n;
        srow[b] = row < nrows ? a.slot_rows[it.slot_base + (row >> a.log2G)] : 0;
    }
}

// Partials of rows row0 + 16b + n: slot = srow[b] * Hq + head * G + row % G.
template <int D, int RB, bool FUSED>
__device__ __forceinline__ void write_partials(const DecodeArgs &a, const ItemRegs &it, const int (&srow)[RB],
                                               int row0, int nrows, int nblk, const f32x4 (&o)[RB][D / 16],
                                               const float (&m_ref)[RB], const float (&l_run)[RB], int n,
                                               int c)
{
    const int G = a.G;
#pragma unroll
    for (int b = 0; b < RB; ++b) {
        if (b >= nblk) break;
        float l = l_run[b];
        l += __shfl_xor(l, 16);
        l += __shfl_xor(l, 32);
        const float inv = l > 0.f ? 1.0f / l : 0.f;
        const int row = row0 + 16 * b + n;
        if (row < nrows) {
            const int64_t slot = (int64_t)srow[b] * a.Hq + it.head * G + (row & (G - 1));
#pragma unroll
            for (int j = 0; j < D / 16; ++j) store_partial_o<D, FUSED>(a, slot, 16 * j + 4 * c, o[b][j] * inv);
            if (c == 0) store_partial_ml<FUSED>(a, slot, m_ref[b], l);
        }
    }
}

// Page table of pages [first, first + count) of an item, one raw stream
// entry per lane (count <= 64; 0 past the end).
__device__ __forceinline__ int load_page_table(const DecodeArgs &a, const ItemRegs &it, int first, int count,
                                               int lane)
{
    return lane < count ? a.stream[it.stream_off + first + lane] : 0;
}

// Page table of a shared item (up to 2 x 64 pages): entry i of the run in
// lane i of `lo` (i < 64) or lane i - 64 of `hi`; i is uniform.
struct PageTab {
    int lo, hi;
};

__device__ __forceinline__ int page_entry(const PageTab &t, int i)
{
    return i < kWaveSize ? __builtin_amdgcn_readlane(t.lo, i) : __builtin_amdgcn_readlane(t.hi, i - kWaveSize);
}

// ---------------------------------------------------------------- private path
// One workgroup, one item of at most 16 rows.  The waves split the item's
// 2-page steps into contiguous sub-streams, one per wave; each streams its
// pages straight from HBM into registers (one step in flight while the
// previous computes) and keeps its own (m, l, o).  At the end the waves put
// their statistics in LDS and the workgroup writes one merged partial.
// Work queues: Q = min(kQueues, gridDim.x) of them; workgroup b draws from
// queue b mod Q, which holds items gridDim.x + Q t + (b mod Q), t = 0, 1, ...
__device__ __forceinline__ int num_queues() { return min(kQueues, (int)gridDim.x); }

// Next item of this workgroup from its ticket; without a queue, none.
__device__ __forceinline__ int next_item_of(const DecodeArgs &a, int ticket)
{
    const int nq = num_queues();
    return a.queue ? (int)gridDim.x + nq * ticket + (int)blockIdx.x % nq : a.n_items;
}

template <int D, bool FUSED>
__device__ __forceinline__ void private_item(const DecodeArgs &a, const ItemRegs &it, float *mrg, int tid,
                                             int lane, int n, int c, int *publish, int ticket)
{
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int nrows = it.nreq * a.G;
    const int nsteps_all = (it.npages + 1) >> 1;
    const int s_begin = nsteps_all * wave / kWaves, s_end = nsteps_all * (wave + 1) / kWaves;
    const int first = 2 * s_begin;
    const int count = min(it.npages, 2 * s_end) - first;      // this wave's pages (may be 0)

    u32x4 qf[1][D / 32];
    load_q<D, 1>(qf, a, it, 0, nrows, n, c);
    // partial row of the row this thread stores at the end (row tid / 16)
    int srow[1];
    load_slot_rows<1>(srow, a, it, 0, nrows, tid / (kSharedThreads / 16));
    f32x4 o[1][D / 16];
#pragma unroll
    for (int j = 0; j < D / 16; ++j) o[0][j] = f32x4{0.f, 0.f, 0.f, 0.f};
    float m_ref[1] = {-INFINITY}, l_run[1] = {0.f};
    if (count > 0) {
        const int lane_e = load_page_table(a, it, first, count, lane);
        const int nsteps = (count + 1) >> 1;
        const float sc = a.scale_log2;
        // Two steps in flight: steps 0 and 1 (pages from the item) are issued
        // at once, then each step's compute is followed by the loads of the
        // step two ahead.  The page table (steps 2 on) is waited for right
        // after the first loads, on every path, so no wait inside the loop
        // has to cover it; the scheduling barriers keep a step's first MFMA,
        // and its wait, below the loads issued before it.
        Step<D> fa, fb;
        load_step<D>(fa, a, it, wave, count, 0, lane_e, n, c);
        load_step<D>(fb, a, it, wave, count, 1, lane_e, n, c);
        asm volatile("" ::"v"(lane_e));
        __builtin_amdgcn_sched_barrier(0);
        for (int s = 0;; s += 2) {
            compute_step<D, 1, true>(fa, qf, o, m_ref, l_run, 1, sc, c);
            if (s + 1 >= nsteps) break;
            load_step<D>(fa, a, it, wave, count, s + 2, lane_e, n, c);
            __builtin_amdgcn_sched_barrier(0);
            compute_step<D, 1, true>(fb, qf, o, m_ref, l_run, 1, sc, c);
            if (s + 2 >= nsteps) break;
            load_step<D>(fb, a, it, wave, count, s + 3, lane_e, n, c);
            __builtin_amdgcn_sched_barrier(0);
        }
    }

    // this wave's statistics into LDS: o rows [wave][16][D], then m[wave][16], l[wave][16]
    float *ob = mrg, *mb = mrg + kWaves * 16 * D, *lb = mb + kWaves * 16;
    float l = l_run[0];
    l += __shfl_xor(l, 16);
    l += __shfl_xor(l, 32);
#pragma unroll
    for (int j = 0; j < D / 16; ++j)
        *reinterpret_cast<f32x4 *>(ob + (wave * 16 + n) * D + 16 * j + 4 * c) = o[0][j];
    if (c == 0) {
        mb[wave * 16 + n] = m_ref[0];
        lb[wave * 16 + n] = l;
    }
    if (tid == 0) *publish = next_item_of(a, ticket);   // the ticket has long returned
    __syncthreads();

    // merge: thread t takes row t / TPR and D/TPR consecutive dims
    constexpr int TPR = kSharedThreads / 16;             // threads per row
    constexpr int V = D / TPR;
    const int row = tid / TPR, d0 = (tid % TPR) * V;
    float M = -INFINITY;
#pragma unroll
    for (int w = 0; w < kWaves; ++w)
        if (lb[w * 16 + row] > 0.f) M = fmaxf(M, mb[w * 16 + row]);
    float L = 0.f, acc[V];
#pragma unroll
    for (int v = 0; v < V; ++v) acc[v] = 0.f;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) {
        const float lw = lb[w * 16 + row];
        const float wt = lw > 0.f ? fast_exp2(mb[w * 16 + row] - M) : 0.f;
        L += wt * lw;
#pragma unroll
        for (int v = 0; v < V; ++v) acc[v] += wt * ob[(w * 16 + row) * D + d0 + v];
    }
    if (row < nrows) {
        const int G = a.G;
        const int64_t slot = (int64_t)srow[0] * a.Hq + it.head * G + (row & (G - 1));
        const float inv = L > 0.f ? 1.0f / L : 0.f;
#pragma unroll
        for (int v = 0; v < V; v += 4)
            store_partial_o<D, FUSED>(a, slot, d0 + v,
                                      f32x4{acc[v], acc[v + 1], acc[v + 2], acc[v + 3]} * inv);
        if (tid % TPR == 0) store_partial_ml<FUSED>(a, slot, M, L);
    }
}

// ----------------------------------------------------------------- shared path
// One workgroup, one item of up to kSharedRows rows (nreq x G).  The waves
// stream each 2-page step of KV once, cooperatively, straight from HBM into
// a kSlots-deep LDS ring with gfx950's 16-byte global->LDS loads (no staging
// registers, no LDS write instructions), kSlots - 1 steps ahead of the
// compute; each wave applies the tile to its own 32 rows.  One barrier per
// step, after which the slot of the previous step is refilled.
//
// Tile of one step: K page 0, K page 1, V page 0, V page 1, each 16 x D bf16
// (kPage * D elements).  K blocks keep the pool layout ([D/8][16][8]: a
// wave's fragment read is 1 KB contiguous).  V blocks ([D][16], two 16-byte
// chunks per dim row) store chunk h of row d at chunk h ^ ((d >> 2) & 1): the
// sixteen lanes that read chunk h of rows 16j..16j+15 then spread evenly over
// the banks (two passes, no conflict).  A load lane picks its source chunk so
// that the chunk lands where this layout wants it.
constexpr int kSlots = 4;

template <int D>
struct SharedTile {
    static constexpr int kBlock = kPage * D;                 // elements of one K or V page block
    static constexpr int kStep = 4 * kBlock;                  // elements of one step (slot)
    static constexpr int kPPB = kBlock * 2 / (kWaveSize * 16); // 1 KB pieces per block (one per wave for D=128)
};

// Global->LDS loads of step `step` into `slot`: piece k of each wave covers
// block k * kWaves / kPPB ... (kPPB pieces per block, 4 blocks, kWaves waves).
template <int D>
__device__ __forceinline__ void issue_dma(const DecodeArgs &a, const ItemRegs &it, int step, const PageTab &pt,
                                          uint16_t *slot, int wave, int lane)
{
    using T = SharedTile<D>;
    const int head = it.head;
    const int i0 = 2 * step;
    const int i1 = i0 + 1 < it.npages ? i0 + 1 : i0;
    int e0, e1;
    if (i1 < kInlineEntries) {             // the first pages come with the item
        e0 = __builtin_amdgcn_readlane(it.lane_ent, i0);
        e1 = __builtin_amdgcn_readlane(it.lane_ent, i1);
    } else {
        e0 = page_entry(pt, i0);
        e1 = page_entry(pt, i1);
    }
    // byte offsets of the two pages' (page, head) blocks, computed once per
    // step (the pieces below only pick one of four bases)
    constexpr uint64_t kBlockBytes = (uint64_t)T::kBlock * 2;
    const uint64_t o0 = ((uint64_t)(uint32_t)(e0 >> 5) * (uint32_t)a.Hkv + (uint32_t)head) * kBlockBytes;
    const uint64_t o1 = ((uint64_t)(uint32_t)(e1 >> 5) * (uint32_t)a.Hkv + (uint32_t)head) * kBlockBytes;
    const char *kp = reinterpret_cast<const char *>(a.k_pool), *vp = reinterpret_cast<const char *>(a.v_pool);
    __builtin_assume(wave >= 0 && wave < kWaves);           // lets b fold to a constant when kPPB == kWaves
#pragma unroll
    for (int k = 0; k < T::kPPB; ++k) {
        const int piece = wave + kWaves * k;                 // 0 .. 4 * kPPB - 1
        const int b = piece / T::kPPB;                       // 0 K page0, 1 K page1, 2 V page0, 3 V page1
        const int c = (piece % T::kPPB) * kWaveSize + lane;  // destination 16-byte chunk in the block
        int src = c;
        if (b & 2) {                                         // V: row d, chunk h lands at h ^ ((d >> 2) & 1)
            const int d = c >> 1;
            src = 2 * d + ((c & 1) ^ ((d >> 2) & 1));
        }
        const char *base = (b & 2) ? vp + ((b & 1) ? o1 : o0) : kp + ((b & 1) ? o1 : o0);
        const char *g = base + src * 16;
        __builtin_amdgcn_global_load_lds(
            (const void __attribute__((address_space(1))) *)g,
            (void __attribute__((address_space(3))) *)(slot + b * T::kBlock + (piece % T::kPPB) * kWaveSize * 8),
            16, 0, kKvDmaPolicy);
    }
}

// Wait until this wave's loads of all but the newest `keep` issued steps have
// landed (and its LDS reads are done), then barrier: every wave's loads for
// the oldest step are in LDS and every wave has finished the step before.
// The asm barrier is also a compiler memory barrier; __syncthreads() would
// drain every outstanding global->LDS load instead.
template <int N>
__device__ __forceinline__ void wait_vm_lgkm0()
{
    static_assert(N >= 0 && N < 64, "vmcnt field");
    __builtin_amdgcn_s_waitcnt(0x0070 | (N & 15) | ((N >> 4) << 14));   // vmcnt(N) expcnt(7) lgkmcnt(0)
}

template <int PPB>
__device__ __forceinline__ void ring_barrier(int keep)
{
    if (keep >= 3)
        wait_vm_lgkm0<3 * PPB>();
    else if (keep == 2)
        wait_vm_lgkm0<2 * PPB>();
    else if (keep == 1)
        wait_vm_lgkm0<PPB>();
    else
        wait_vm_lgkm0<0>();
    asm volatile("s_barrier" ::: "memory");
}

// QK operands (K page blocks) of one step from the LDS tile.
template <int D>
__device__ __forceinline__ void lds_k(u32x4 (&k0)[D / 32], u32x4 (&k1)[D / 32], const uint16_t *slot, int n,
                                      int c)
{
    constexpr int blk = SharedTile<D>::kBlock;
#pragma unroll
    for (int i = 0; i < D / 32; ++i) {
        k0[i] = *reinterpret_cast<const u32x4 *>(slot + ((4 * i + c) * kPage + n) * 8);
        k1[i] = *reinterpret_cast<const u32x4 *>(slot + blk + ((4 * i + c) * kPage + n) * 8);
    }
}

// PV operands (V page blocks) of one step from the LDS tile: lane (n, c)
// reads tokens 8(c & 1)..+7 of row 16j + n of page c >> 1, one 16-byte chunk.
template <int D>
__device__ __forceinline__ void lds_v(u32x4 (&v)[D / 16], const uint16_t *slot, int n, int c)
{
    constexpr int blk = SharedTile<D>::kBlock;
    const uint16_t *vb = slot + (2 + (c >> 1)) * blk + 8 * ((c & 1) ^ ((n >> 2) & 1));
#pragma unroll
    for (int j = 0; j < D / 16; ++j) v[j] = *reinterpret_cast<const u32x4 *>(vb + (16 * j + n) * kPage);
}

// Ring bookkeeping shared by the computing and the idle waves: the prologue
// loads steps 0..kSlots-1 (one per slot) and waits for step 0; before step
// s + 1 is read, ring_next waits for it, and (from s = 1 on) refills the slot
// of step s - 1, which every wave finished reading before this barrier, with
// step s + kSlots - 1.
template <int D>
__device__ __forceinline__ void ring_start(const DecodeArgs &a, const ItemRegs &it, int nsteps, const PageTab &pt,
                                           uint16_t *lds, int wave, int lane)
{
#pragma unroll
    for (int q = 0; q < kSlots; ++q)
        if (q < nsteps) issue_dma<D>(a, it, q, pt, lds + q * SharedTile<D>::kStep, wave, lane);
    ring_barrier<SharedTile<D>::kPPB>(min(kSlots, nsteps) - 1);
}

template <int D>
__device__ __forceinline__ void ring_next(const DecodeArgs &a, const ItemRegs &it, int nsteps, int s,
                                          const PageTab &pt, uint16_t *lds, int wave, int lane)
{
    // issued so far: steps 0 .. min(nsteps, max(kSlots, s + kSlots - 1)) - 1; wait for step s + 1
    const int issued = min(nsteps, max(kSlots, s + kSlots - 1));
    ring_barrier<SharedTile<D>::kPPB>(issued - (s + 2));
    const int nxt = s + kSlots - 1;
    if (s >= 1 && nxt < nsteps)
        issue_dma<D>(a, it, nxt, pt, lds + (nxt % kSlots) * SharedTile<D>::kStep, wave, lane);
}

template <int D, bool FUSED>
__device__ __forceinline__ void shared_item(const DecodeArgs &a, const ItemRegs &it, uint16_t *lds, int tid,
                                            int lane, int n, int c, int *publish, int ticket)
{
    using T = SharedTile<D>;
    // A shared item's waves share each SIMD with a private item's wave, which
    // mostly waits on memory; their step (MFMA and softmax for up to 128
    // rows) sets the pace of the whole item, so they issue first.
    __builtin_amdgcn_s_setprio(1);
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int nrows = it.nreq * a.G;
    const int row0 = 32 * wave;
    const int nblk = nrows > row0 ? min(2, (nrows - row0 + 15) >> 4) : 0;
    PageTab pt;
    pt.lo = load_page_table(a, it, 0, min(it.npages, kWaveSize), lane);
    pt.hi = it.npages > kWaveSize ? load_page_table(a, it, kWaveSize, it.npages - kWaveSize, lane) : 0;
    u32x4 qf[2][D / 32];
    load_q<D, 2>(qf, a, it, row0, nrows, n, c);         // before the ring loads: loads land in order
    int srow[2];
    load_slot_rows<2>(srow, a, it, row0, nrows, n);
    const int nsteps = (it.npages + 1) >> 1;
    const int np = it.npages;
    ring_start<D>(a, it, nsteps, pt, lds, wave, lane);

    f32x4 o[2][D / 16];
#pragma unroll
    for (int b = 0; b < 2; ++b)
#pragma unroll
        for (int j = 0; j < D / 16; ++j) o[b][j] = f32x4{0.f, 0.f, 0.f, 0.f};
    float m_ref[2] = {-INFINITY, -INFINITY}, l_run[2] = {0.f, 0.f};
    const float sc = a.scale_log2;
    // A wave with rows computes both of its 16-row blocks (rows past nrows
    // have zero Q and are not written): wave 0 always has two, and the waves
    // wait for each other every step.  Software-pipelined: the QK MFMAs of
    // step s + 1 are issued before the softmax of step s, so the matrix cores
    // work while the vector ALUs do the softmax.  A wave without rows only
    // keeps the ring going.
    if (nblk > 0) {
        u32x4 k0[D / 32], k1[D / 32], v[D / 16];
        f32x4 sa0[2], sa1[2], sb0[2], sb1[2];
        lds_k<D>(k0, k1, lds, n, c);
        qk_step<D, 2>(k0, k1, qf, sa0, sa1, 2);
        // Per step: wait for the ring, read K of step s + 1 and V of step s,
        // settle masking and the reference maximum of step s (branches), then
        // one straight block: the QK MFMAs of step s + 1 (on the last step
        // they read a stale slot; the result is unused) and the softmax and
        // PV of step s.
        auto half = [&](int s, f32x4 (&c0)[2], f32x4 (&c1)[2], f32x4 (&n0)[2], f32x4 (&n1)[2]) {
            if (s + 1 < nsteps) ring_next<D>(a, it, nsteps, s, pt, lds, wave, lane);
            lds_k<D>(k0, k1, lds + ((s + 1) % kSlots) * T::kStep, n, c);
            const int nt0 = (page_entry(pt, 2 * s) & 31) + 1;
            const int nt1 = 2 * s + 1 < np ? (page_entry(pt, 2 * s + 1) & 31) + 1 : 0;
            lds_v<D>(v, lds + (s % kSlots) * T::kStep, n, c);
            softmax_prepare<D>(c0, c1, v, nt0, nt1, o, m_ref, l_run, sc, c);
            qk_step<D, 2>(k0, k1, qf, n0, n1, 2);
            softmax_finish<D>(c0, c1, v, o, m_ref, l_run, sc);
            // scheduling hint for this block: each QK MFMA followed by two
            // vector ops of the softmax, then each PV MFMA by one
#pragma unroll
            for (int i = 0; i < D / 8; ++i) {
                __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
                __builtin_amdgcn_sched_group_barrier(0x002, 2, 0);
            }
#pragma unroll
            for (int i = 0; i < D / 8; ++i) {
                __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
                __builtin_amdgcn_sched_group_barrier(0x002, 1, 0);
            }
        };
        for (int s = 0; s < nsteps; s += 2) {
            half(s, sa0, sa1, sb0, sb1);
            if (s + 1 < nsteps) half(s + 1, sb0, sb1, sa0, sa1);
        }
    } else {
        for (int s = 0; s + 1 < nsteps; ++s) ring_next<D>(a, it, nsteps, s, pt, lds, wave, lane);
    }
    if (tid == 0) *publish = next_item_of(a, ticket);   // the ticket has long returned
    write_partials<D, 2, FUSED>(a, it, srow, row0, nrows, nblk, o, m_ref, l_run, n, c);
    __builtin_amdgcn_s_setprio(0);
}

// ------------------------------------------------------------------ merge
// Where a merge reads its partials and writes its output.
struct MergeView {
    const int32_t *merge_off;    // [R+1]: request r's partial rows are merge_off[r] .. merge_off[r+1] - 1
    const uint16_t *part_o;      // fp16 o / l
    const float *part_m, *part_l;
    const float *part_w;         // fp32 o / l of the 4-dim groups whose fp16 form is not finite
    uint16_t *out;               // [R][Hq][D] bf16
    int32_t Hq, slots;
};

// Loads of one block of up to 16 partials (partial rows row0 .. row0 + nb - 1)
// of one merge row.
template <int D>
struct MergeBlock {
    static constexpr int NB = 16;
    float m[NB], l[NB];
    u32x4 x[NB];
};

template <int D, bool COHERENT>
__device__ __forceinline__ void merge_load(MergeBlock<D> &b, const MergeView &v, int row0, int nb, int qh, int dc)
{
#pragma unroll
    for (int i = 0; i < MergeBlock<D>::NB; ++i) {
        if (i < nb) {
            const int slot = (row0 + i) * v.Hq + qh;
            if constexpr (COHERENT) {
                b.m[i] = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(
                    buf_rsrc(v.part_m, v.slots * 4), slot * 4, 0, kCoherent));
                b.l[i] = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(
                    buf_rsrc(v.part_l, v.slots * 4), slot * 4, 0, kCoherent));
                b.x[i] = __builtin_amdgcn_raw_buffer_load_b128(buf_rsrc(v.part_o, v.slots * D * 2),
                                                               (slot * D + 8 * dc) * 2, 0, kCoherent);
            } else {
                b.m[i] = v.part_m[slot];
                b.l[i] = v.part_l[slot];
                b.x[i] = *reinterpret_cast<const u32x4 *>(v.part_o + (int64_t)slot * D + 8 * dc);
            }
        } else {
            b.m[i] = -INFINITY;
            b.l[i] = 0.f;
            b.x[i] = u32x4{0u, 0u, 0u, 0u};
        }
    }
}

// fp32 o / l of dims 8 dc + 4 g .. + 3 of one slot, from the side region
// (read only for a group whose fp16 form is not finite; see store_partial_o).
template <int D, bool COHERENT>
__device__ __forceinline__ f32x4 merge_wide(const MergeView &v, int slot, int dc, int g)
{
    if constexpr (COHERENT)
        return __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(
            buf_rsrc(v.part_w + (int64_t)slot * D, D * 4), (8 * dc + 4 * g) * 4, 0, kCoherent));
    else
        return *reinterpret_cast<const f32x4 *>(v.part_w + (int64_t)slot * D + 8 * dc + 4 * g);
}

// Fold a block into the running (M, L, acc): the reference M rises to the
// block maximum (rescaling what is summed so far), then each partial adds
// weight 2^(m_i - M) l_i.
template <int D>
__device__ __forceinline__ void merge_fold(const MergeBlock<D> &b, float &M, float &L, float (&acc)[8])
{
    typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
    constexpr int NB = MergeBlock<D>::NB;
    float mb = -INFINITY;
#pragma unroll
    for (int i = 0; i < NB; ++i)
        if (b.l[i] > 0.f) mb = fmaxf(mb, b.m[i]);
    const float M_new = fmaxf(M, mb);
    const float rescale = M_new == -INFINITY ? 0.f : fast_exp2(M - M_new);   // 0 on the first block
    L *= rescale;
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[e] *= rescale;
#pragma unroll
    for (int i = 0; i < NB; ++i) {
        const float w = b.l[i] > 0.f ? fast_exp2(b.m[i] - M_new) * b.l[i] : 0.f;
        const f16x8 h = __builtin_bit_cast(f16x8, b.x[i]);
        L += w;
#pragma unroll
        for (int e = 0; e < 8; ++e) acc[e] += w * (float)h[e];
    }
    M = M_new;
}

// The same fold for partials that may hold groups past fp16's range (see
// store_partial_o): such a group's values come from the fp32 side region, and
// a partial of weight 0 is skipped (0 x inf would poison the sums).  Partials
// of rows row0 .. of query head qh.
template <int D, bool COHERENT>
__device__ __forceinline__ void merge_fold_wide(const MergeBlock<D> &b, const MergeView &v, int row0, int qh,
                                                int dc, float &M, float &L, float (&acc)[8])
{
    typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
    constexpr int NB = MergeBlock<D>::NB;
    float mb = -INFINITY;
    for (int i = 0; i < NB; ++i)
        if (b.l[i] > 0.f) mb = fmaxf(mb, b.m[i]);
    const float M_new = fmaxf(M, mb);
    const float rescale = M_new == -INFINITY ? 0.f : fast_exp2(M - M_new);
    L *= rescale;
    for (int e = 0; e < 8; ++e) acc[e] *= rescale;
    for (int i = 0; i < NB; ++i) {
        const float w = b.l[i] > 0.f ? fast_exp2(b.m[i] - M_new) * b.l[i] : 0.f;
        L += w;
        if (w == 0.f) continue;
        const f16x8 h = __builtin_bit_cast(f16x8, b.x[i]);
        float x[8];
        for (int e = 0; e < 8; ++e) x[e] = (float)h[e];
        for (int g = 0; g < 2; ++g) {
            if (f16_pair_nonfinite(b.x[i][2 * g]) || f16_pair_nonfinite(b.x[i][2 * g + 1])) {
                const f32x4 f = merge_wide<D, COHERENT>(v, (row0 + i) * v.Hq + qh, dc, g);
                for (int e = 0; e < 4; ++e) x[4 * g + e] = f[e];
            }
        }
        for (int e = 0; e < 8; ++e) acc[e] += w * x[e];
    }
    M = M_new;
}

// One wave merges the partials of query heads qh0 .. qh0 + nh - 1 (nh <=
// RPW = 512 / D) of request r and writes their bf16 output rows:
//   out = sum_i 2^(m_i - M) l_i (o_i / l_i) / sum_i 2^(m_i - M) l_i,
// the partials holding the normalised o_i / l_i.  A request's partial rows
// are one block (merge_off), the same for all its query heads, so a wave only
// reads where the block starts.  Lane = (row rho, dim chunk dc): D / 8 lanes
// per row, 8 dims (one 16-byte fp16 load per partial) per lane; each lane
// also loads m and l of its row (the row's lanes share those addresses), so
// no lane exchanges anything.  Partials go 16 per block, the next block's
// loads in flight while a block is folded in.  COHERENT: sc1 loads (fused
// step, one block at a time).
template <int D, bool COHERENT>
__device__ __forceinline__ void merge_rows(const MergeView &v, int r, int beg, int np, int qh0, int nh, int lane)
{
    constexpr int LPR = D / 8;                 // lanes per row
    constexpr int NB = MergeBlock<D>::NB;
    const int rho = lane / LPR, dc = lane % LPR;
    const bool active = rho < nh;
    const int qh = qh0 + (active ? rho : 0);
    float M = -INFINITY, L = 0.f;
    float acc[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[e] = 0.f;
    if constexpr (COHERENT) {
        // inside the decode kernel: one block at a time (its register budget)
        for (int k = 0; k < np; k += NB) {
            MergeBlock<D> ba;
            merge_load<D, COHERENT>(ba, v, beg + k, min(NB, np - k), qh, dc);
            merge_fold<D>(ba, M, L, acc);
        }
    } else {
        MergeBlock<D> ba, bb;
        merge_load<D, COHERENT>(ba, v, beg, min(NB, np), qh, dc);
        for (int k = 0; k < np; k += 2 * NB) {
            if (k + NB < np) merge_load<D, COHERENT>(bb, v, beg + k + NB, min(NB, np - k - NB), qh, dc);
            merge_fold<D>(ba, M, L, acc);
            if (k + NB >= np) break;
            if (k + 2 * NB < np) merge_load<D, COHERENT>(ba, v, beg + k + 2 * NB, min(NB, np - k - 2 * NB), qh, dc);
            merge_fold<D>(bb, M, L, acc);
        }
    }
    // A non-finite sum means a partial group past fp16's range (stored as
    // inf, its fp32 value in the side region; or 0 x inf): merge this lane's
    // row again from the side region.  Never taken for N(0,1)-scale inputs.
    bool bad = false;
#pragma unroll
    for (int e = 0; e < 8; ++e) bad |= (__builtin_bit_cast(uint32_t, acc[e]) & 0x7F800000u) == 0x7F800000u;
    if (bad) {
        M = -INFINITY;
        L = 0.f;
        for (int e = 0; e < 8; ++e) acc[e] = 0.f;
        for (int k = 0; k < np; k += NB) {
            MergeBlock<D> ba;
            merge_load<D, COHERENT>(ba, v, beg + k, min(NB, np - k), qh, dc);
            merge_fold_wide<D, COHERENT>(ba, v, beg + k, qh, dc, M, L, acc);
        }
    }
    if (active) {
        const float inv = 1.0f / L;
        u32x4 o;
#pragma unroll
        for (int e = 0; e < 4; ++e)
            o[e] = __builtin_bit_cast(uint16_t, (__bf16)(acc[2 * e] * inv)) |
                   ((uint32_t)__builtin_bit_cast(uint16_t, (__bf16)(acc[2 * e + 1] * inv)) << 16);
        *reinterpret_cast<u32x4 *>(v.out + ((int64_t)r * v.Hq + qh) * D + 8 * dc) = o;
    }
}

// Fused step, after an item has written its partials (sc1 stores): wait for
// them to complete, then count the item in for each of its requests (one
// counter per request and KV head).  The item that completes a request's
// count merges that request's G query heads here, one wave per head, and
// resets the counter for the next step.  lst: LDS, [0] = count, then the
// completed request ids.
template <int D>
__device__ __forceinline__ void finish_item(const DecodeArgs &a, const ItemRegs &it, int *lst, int tid)
{
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");
    __builtin_amdgcn_s_waitcnt(0x0F70);          // vmcnt(0): this wave's partial stores are done
    __syncthreads();
    if (tid < it.nreq) {
        const int r = a.rows[it.row_off + tid];
        const int need = a.merge_off[r + 1] - a.merge_off[r];
        int *cp = a.counters + (int64_t)r * a.Hkv + it.head;
        const int seen = __hip_atomic_fetch_add(cp, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        if (seen == need - 1) {
            __hip_atomic_store(cp, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            lst[1 + atomicAdd(&lst[0], 1)] = r;
        }
    }
    __syncthreads();
    const int nlast = lst[0];
    if (nlast == 0) return;
    const MergeView v{a.merge_off, a.part_o, a.part_m, a.part_l, a.part_w, a.out, a.Hq, a.slots};
    // row sets of up to RPW query heads of this KV head, one wave each
    constexpr int RPW = kWaveSize / (D / 8);
    const int G = a.G, sets = (G + RPW - 1) / RPW;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    for (int t = wave; t < nlast * sets; t += kWaves) {
        const int g0 = (t % sets) * RPW;
        const int r = lst[1 + t / sets];
        const int beg = v.merge_off[r];
        merge_rows<D, true>(v, r, beg, v.merge_off[r + 1] - beg, it.head * G + g0, min(RPW, G - g0),
                            tid & (kWaveSize - 1));
    }
}

// Shared items stage KV in LDS for their row-waves; private items split
// their pages over the waves.  FUSED: the item that completes a request also
// merges it (no merge_kernel launch).
//
// Items in item order: workgroup b starts with item b; with work queues
// (a.queue) the grid is two workgroups per CU and each then takes its next
// item from queue b mod 8 (next_item_of), with a ticket from that queue's
// counter, taken when it starts an item (the ticket's latency hides behind
// the item's own loads).  Eight queues, one per XCD, keep the hardware's
// XCD placement of items and spread the counter traffic.  Each workgroup's
// last ticket is past the end; the workgroup that finishes last returns
// every counter to zero for the next launch.  Without a queue (one
// workgroup per item) the hardware starts workgroups in order, each bound to
// one shader engine, so a free slot can wait for a busy engine.
template <int D, bool FUSED>
__global__ __launch_bounds__(kSharedThreads) __attribute__((amdgpu_waves_per_eu(2)))
void decode_kernel(const DevItem *items, DecodeArgs a)
{
    constexpr int kTileBytes = kSlots * SharedTile<D>::kStep * 2;  // shared path: the LDS ring
    constexpr int kMergeBytes = (kWaves * 16 * D + 2 * kWaves * 16) * 4;   // private path: merge buffer
    constexpr int kLdsBytes = kTileBytes > kMergeBytes ? kTileBytes : kMergeBytes;
    constexpr int kLstInts = FUSED ? 1 + kSharedRows : 0;
    // One LDS object for everything: with several, the compiler's tracking of
    // global->LDS loads makes every ring read wait for all of them.  Layout:
    // ring / merge buffer, then the fused step's completion list, then the
    // next item by iteration parity.
    __shared__ __attribute__((aligned(16))) float lds[kLdsBytes / 4 + kLstInts + 2];
    int *const lst = reinterpret_cast<int *>(lds + kLdsBytes / 4);
    int *const next_item = lst + kLstInts;
    // The grid never exceeds the item count, so the first item needs no
    // check (and n_items no early wait).  `items` comes first among the
    // kernel arguments, which the build preloads into SGPRs: the first item's
    // read is the workgroup's first load, in flight while the other arguments
    // load.
    int cur = blockIdx.x;
    int par = 0;
    ItemRegs it = read_item(items, cur, threadIdx.x & (kWaveSize - 1));
    do {
        // the lane index is re-derived each item (opaque to the compiler), so
        // nothing lane-dependent is hoisted out of the loop to hold registers
        int tid = threadIdx.x;
        asm volatile("" : "+v"(tid));
        const int lane = tid & (kWaveSize - 1);
        const int n = lane & 15, c = lane >> 4;
        // thread 0's ticket; read only where the next item is published, which
        // is where the compiler waits for it (no value on the other paths, so
        // no copy at the branch join forces an early wait)
        int ticket;
        if (a.queue && tid == 0)
            ticket = __hip_atomic_fetch_add(a.queue + (blockIdx.x % num_queues()) * kQueueStride, 1,
                                            __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        if (FUSED && tid == 0) lst[0] = 0;     // read after the item's barriers
        if (it.mode == kModeShared)
            shared_item<D, FUSED>(a, it, reinterpret_cast<uint16_t *>(lds), tid, lane, n, c, &next_item[par], ticket);
        else
            private_item<D, FUSED>(a, it, lds, tid, lane, n, c, &next_item[par], ticket);
        if constexpr (FUSED) finish_item<D>(a, it, lst, tid);
        // every wave is done with this item's LDS (and next_item is written);
        // partial stores may still be in flight
        __builtin_amdgcn_s_waitcnt(0xC07F);    // lgkmcnt(0)
        asm volatile("s_barrier" ::: "memory");
        cur = __builtin_amdgcn_readfirstlane(next_item[par]);
        par ^= 1;
        if (cur < a.n_items) it = read_item(items, cur, lane);
    } while (cur < a.n_items);
    if (a.queue && threadIdx.x == 0) {
        // every ticket of this workgroup has returned (the last one ended the loop)
        int *const done_ctr = a.queue + kQueues * kQueueStride;
        const int done = __hip_atomic_fetch_add(done_ctr, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        if (done == (int)gridDim.x - 1) {
            for (int x = 0; x < kQueues; ++x)
                __hip_atomic_store(a.queue + x * kQueueStride, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            __hip_atomic_store(done_ctr, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
    }
}

// Two-launch step: one one-wave workgroup per request (grid x) and set of
// RPW = 512 / D query heads (grid y); the grid is exact, so a workgroup
// finds its request and heads without a bounds check or a division.  The
// merge offsets come first among the arguments (preloaded into SGPRs), so
// the request's offsets load at once.
template <int D>
__global__ __launch_bounds__(kWaveSize) void merge_kernel(const int32_t *merge_off, MergeArgs a)
{
    constexpr int RPW = kWaveSize / (D / 8);
    const int r = blockIdx.x;
    const int beg = merge_off[r], np = merge_off[r + 1] - beg;     // first: no argument needed
    const MergeView v{merge_off, a.part_o, a.part_m, a.part_l, a.part_w, a.out, a.Hq, 0};
    const int qh0 = blockIdx.y * RPW;
    merge_rows<D, false>(v, r, beg, np, qh0, min(RPW, a.Hq - qh0), threadIdx.x & (kWaveSize - 1));
}

}  // namespace

// CU count of the current device, cached per device.
static int device_cus(int *cus)
{
    static int cache[64] = {};
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return (int)e;
    if (dev >= 0 && dev < 64 && cache[dev] > 0) {
        *cus = cache[dev];
        return 0;
    }
    int n = 0;
    e = hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev);
    if (e != hipSuccess) return (int)e;
    *cus = n > 0 ? n : 1;
    if (dev >= 0 && dev < 64) cache[dev] = *cus;
    return 0;
}

// Partial workspace of cap_decode_step_noalloc: a fixed array in the code
// object, so that callers that cannot allocate (graph capture, allocation-
// free serving loops) get one.  Each GPU the library runs on holds its own
// copy until the process ends.  In host code `scratch` names a host-side
// stand-in, not device memory: its device address comes from
// hipGetSymbolAddress, looked up once per device with that device current,
// and only that address is ever passed to a kernel.
static __device__ __attribute__((aligned(256))) unsigned char scratch[kScratchBytes];

int scratch_address(void **ptr)
{
    static std::mutex mu;
    static void *addr[64] = {};
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return (int)e;
    if (dev < 0 || dev >= 64) return (int)hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lock(mu);
    if (!addr[dev]) {
        void *p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return (int)e;
        addr[dev] = p;
    }
    *ptr = addr[dev];
    return 0;
}

int launch_decode(const DecodeArgs &a, int head_dim, void *stream, void *ev_start, void *ev_stop)
{
    if (a.n_items <= 0) return 0;
    hipStream_t s = reinterpret_cast<hipStream_t>(stream);
    const bool fused = a.counters != nullptr;
    int grid = a.n_items;
    if (a.queue) {
        // two resident workgroups per CU (LDS and the two-waves-per-SIMD bound)
        int cus = 0;
        const int e = device_cus(&cus);
        if (e != 0) return e;
        grid = std::min(a.n_items, 2 * cus);
    }
    const dim3 g((unsigned)grid), b(kSharedThreads);
    hipEvent_t e0 = reinterpret_cast<hipEvent_t>(ev_start), e1 = reinterpret_cast<hipEvent_t>(ev_stop);
    auto k = head_dim == 128 ? (fused ? decode_kernel<128, true> : decode_kernel<128, false>)
                             : (fused ? decode_kernel<64, true> : decode_kernel<64, false>);
    if (e0 || e1)
        hipExtLaunchKernelGGL(k, g, b, 0, s, e0, e1, 0, a.items, a);
    else
        hipLaunchKernelGGL(k, g, b, 0, s, a.items, a);
    return (int)hipGetLastError();
}

int launch_merge(const MergeArgs &a, int head_dim, void *stream)
{
    const int rpw = kWaveSize / (head_dim / 8);
    if (a.R <= 0 || a.Hq <= 0) return 0;
    const dim3 grid((unsigned)a.R, (unsigned)((a.Hq + rpw - 1) / rpw));
    hipStream_t s = reinterpret_cast<hipStream_t>(stream);
    if (head_dim == 128)
        hipLaunchKernelGGL(merge_kernel<128>, grid, dim3(kWaveSize), 0, s, a.merge_off, a);
    else
        hipLaunchKernelGGL(merge_kernel<64>, grid, dim3(kWaveSize), 0, s, a.merge_off, a);
    return (int)hipGetLastError();
}

}  // namespace cap
