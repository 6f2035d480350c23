// cap_rows.hip -- gfx950 kernels of the wide-row reduction-reuse workloads:
// softmax over a row of logits and LayerNorm, FP32, one workgroup per row.
//
// The workload class is the one of the CREDIT summary (section III.B,
// "Reduction-Reuse Transformation"): each row is reduced to scalar
// statistics, which are then reused by an elementwise function of every
// element.  The memory-bound cost is the bytes read and written; a schedule
// that cannot keep the row must read it again for the elementwise pass.
// CREDIT keeps owner-local slices of a row spread over a Hopper thread-block
// cluster and exchanges the partial statistics through distributed shared
// memory.  On CDNA4 one workgroup of up to 1024 lanes can keep a whole row of
// up to 64K FP32 values in its registers (16 float4 per lane, 64 VGPRs), so
// the retained schedule needs no cross-CU exchange at all: the row is read
// from HBM once (all of it in flight at once), the statistics are reduced
// across the workgroup (wave shuffles, then one LDS slot per wave), and the
// output is computed from the registers and written once.
//
// rows_retained_kernel:  that schedule, for rows of at most 64K values.
// rows_pipelined_kernel: the same, several rows per workgroup, the next
//                        row's loads in flight while the current row is
//                        reduced and written.
// rows_reread_kernel:    the non-retaining schedule (and the only one for
//                        wider rows): a statistics pass over the row, then a
//                        second read for the output pass.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <atomic>

#include "cap_internal.h"

namespace cap {
namespace {

constexpr float kLog2e = 1.4426950408889634f;
constexpr int kMaxRowWaves = 16;

__device__ __forceinline__ float fexp2(float x) { return __builtin_amdgcn_exp2f(x); }

__device__ __forceinline__ float wave_max(float v)
{
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o));
    return v;
}

__device__ __forceinline__ float wave_sum(float v)
{
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o);
    return v;
}

// Workgroup reductions through one LDS slot per wave; every lane then folds
// the slots in the same order, so the result is identical in every lane and
// the same from run to run.  Each call site passes its own slot array, so no
// barrier is needed before the slots are written again.
template <int THREADS>
__device__ __forceinline__ float block_max(float v, float *slots)
{
    v = wave_max(v);
    if ((threadIdx.x & 63) == 0) slots[threadIdx.x >> 6] = v;
    __syncthreads();
    float r = slots[0];
#pragma unroll
    for (int i = 1; i < THREADS / 64; ++i) r = fmaxf(r, slots[i]);
    return r;
}

template <int THREADS>
__device__ __forceinline__ float block_sum(float v, float *slots)
{
    v = wave_sum(v);
    if ((threadIdx.x & 63) == 0) slots[threadIdx.x >> 6] = v;
    __syncthreads();
    float r = slots[0];
#pragma unroll
    for (int i = 1; i < THREADS / 64; ++i) r += slots[i];
    return r;
}

// VEC values per load: 4 (a float4; width % 4 == 0, 16-byte aligned rows)
// or 1.  Lane t holds loads t, t + THREADS, ..., so a wave's loads are
// contiguous.
template <int VEC>
struct Vec {
    float v[VEC];
};

template <int VEC>
__device__ __forceinline__ Vec<VEC> load_nt(const float *p)
{
    Vec<VEC> r;
    if constexpr (VEC == 4) {
        typedef float f4 __attribute__((ext_vector_type(4)));
        const f4 x = __builtin_nontemporal_load(reinterpret_cast<const f4 *>(p));
        r.v[0] = x.x, r.v[1] = x.y, r.v[2] = x.z, r.v[3] = x.w;
    } else {
        r.v[0] = __builtin_nontemporal_load(p);
    }
    return r;
}

template <int VEC>
__device__ __forceinline__ Vec<VEC> load_cached(const float *p)
{
    Vec<VEC> r;
    if constexpr (VEC == 4) {
        typedef float f4 __attribute__((ext_vector_type(4)));
        const f4 x = *reinterpret_cast<const f4 *>(p);
        r.v[0] = x.x, r.v[1] = x.y, r.v[2] = x.z, r.v[3] = x.w;
    } else {
        r.v[0] = *p;
    }
    return r;
}

// The retained schedules write their output with plain stores (write-back
// through L2): on this GPU they measured 4-17% faster than non-temporal
// stores for softmax rows of 8K-64K values, also where the output far
// exceeds the 256 MB Infinity Cache, and about as fast for LayerNorm.  The two-pass
// schedule keeps non-temporal stores: its second read finds the row in the
// Infinity Cache, and plain stores would evict it (5-6% slower measured).
template <int VEC>
__device__ __forceinline__ void store_nt(float *p, const Vec<VEC> &r)
{
    if constexpr (VEC == 4) {
        typedef float f4 __attribute__((ext_vector_type(4)));
        f4 x;
        x.x = r.v[0], x.y = r.v[1], x.z = r.v[2], x.w = r.v[3];
        __builtin_nontemporal_store(x, reinterpret_cast<f4 *>(p));
    } else {
        __builtin_nontemporal_store(r.v[0], p);
    }
}

template <int VEC>
__device__ __forceinline__ void store_row(float *p, const Vec<VEC> &r)
{
    if constexpr (VEC == 4) {
        typedef float f4 __attribute__((ext_vector_type(4)));
        f4 x;
        x.x = r.v[0], x.y = r.v[1], x.z = r.v[2], x.w = r.v[3];
        *reinterpret_cast<f4 *>(p) = x;
    } else {
        *p = r.v[0];
    }
}

// One row kept in registers: EPT loads of VEC values per lane (padding
// beyond the row: -inf for softmax, 0 for LayerNorm, neutral in the sums).
template <int KIND, int VEC, int EPT, int THREADS>
__device__ __forceinline__ void load_row(Vec<VEC> (&v)[EPT], const RowArgs &a, int64_t row)
{
    const int64_t nvec = a.width / VEC;
    const float *x = a.x + row * a.width;
#pragma unroll
    for (int k = 0; k < EPT; ++k) {
        const int64_t i = (int64_t)k * THREADS + threadIdx.x;
        if (i < nvec) {
            v[k] = load_nt<VEC>(x + i * VEC);
        } else {
#pragma unroll
            for (int j = 0; j < VEC; ++j) v[k].v[j] = KIND == kRowSoftmax ? -INFINITY : 0.f;
        }
    }
}

// The row's statistics from the registers, then its output, written once.
// red0 / red1: one LDS slot per wave for each of the two reductions.
template <int KIND, int VEC, int EPT, int THREADS, bool GB_REGS = false>
__device__ __forceinline__ void finish_row(Vec<VEC> (&v)[EPT], const RowArgs &a, int64_t row, float *red0,
                                           float *red1, const Vec<VEC> *gam = nullptr,
                                           const Vec<VEC> *bet = nullptr)
{
    const int64_t nvec = a.width / VEC;
    float *y = a.y + row * a.width;
    const int tid = threadIdx.x;
    if constexpr (KIND == kRowSoftmax) {
        float m = -INFINITY;
#pragma unroll
        for (int k = 0; k < EPT; ++k)
#pragma unroll
            for (int j = 0; j < VEC; ++j) m = fmaxf(m, v[k].v[j]);
        m = block_max<THREADS>(m, red0);
        // exp(x - m) = 2^(x log2 e - m log2 e): one fma per value; the
        // rounding of m log2 e is common to every term and cancels in y
        const float mb = m * kLog2e;
        float s = 0.f;
#pragma unroll
        for (int k = 0; k < EPT; ++k)
#pragma unroll
            for (int j = 0; j < VEC; ++j) {
                const float e = fexp2(__builtin_fmaf(v[k].v[j], kLog2e, -mb));   // 0 for padding
                v[k].v[j] = e;
                s += e;
            }
        s = block_sum<THREADS>(s, red1);
        const float inv = 1.f / s;
#pragma unroll
        for (int k = 0; k < EPT; ++k) {
            const int64_t i = (int64_t)k * THREADS + tid;
            if (i < nvec) {
#pragma unroll
                for (int j = 0; j < VEC; ++j) v[k].v[j] *= inv;
                store_row<VEC>(y + i * VEC, v[k]);
            }
        }
    } else {
        float s = 0.f;
#pragma unroll
        for (int k = 0; k < EPT; ++k)
#pragma unroll
            for (int j = 0; j < VEC; ++j) s += v[k].v[j];
        const float mean = block_sum<THREADS>(s, red0) / (float)a.width;
        // second statistic from the registers: sum of squared deviations
        float q = 0.f;
#pragma unroll
        for (int k = 0; k < EPT; ++k) {
            const int64_t i = (int64_t)k * THREADS + tid;
            if (i < nvec) {
#pragma unroll
                for (int j = 0; j < VEC; ++j) {
                    const float d = v[k].v[j] - mean;
                    q = __builtin_fmaf(d, d, q);
                }
            }
        }
        const float var = block_sum<THREADS>(q, red1) / (float)a.width;
        const float rstd = 1.f / sqrtf(var + a.eps);
#pragma unroll
        for (int k = 0; k < EPT; ++k) {
            const int64_t i = (int64_t)k * THREADS + tid;
            if (i < nvec) {
                Vec<VEC> g, b;
                if constexpr (GB_REGS) {
                    g = gam[k];
                    b = bet[k];
                } else {
                    g = load_cached<VEC>(a.gamma + i * VEC);
                    b = load_cached<VEC>(a.beta + i * VEC);
                }
#pragma unroll
                for (int j = 0; j < VEC; ++j)
                    v[k].v[j] = __builtin_fmaf((v[k].v[j] - mean) * rstd, g.v[j], b.v[j]);
                store_row<VEC>(y + i * VEC, v[k]);
            }
        }
    }
}

// One row per workgroup, kept in registers.
template <int KIND, int VEC, int EPT, int THREADS>
__global__ __launch_bounds__(THREADS) void rows_retained_kernel(RowArgs a)
{
    __shared__ float red0[kMaxRowWaves], red1[kMaxRowWaves];
    Vec<VEC> v[EPT];
    load_row<KIND, VEC, EPT, THREADS>(v, a, blockIdx.x);
    finish_row<KIND, VEC, EPT, THREADS>(v, a, blockIdx.x, red0, red1);
}

// Rows blockIdx.x, + gridDim.x, ... per workgroup, each kept in registers,
// with the next row's loads in flight while the current row is reduced and
// written (the launch picks the grid, so rows per workgroup; see
// launch_pipelined): the workgroup's reads and writes overlap, where one-row
// workgroups that all start together read the whole input first and write
// it all afterwards.  LayerNorm's gamma and beta are loaded once per
// workgroup and kept in registers (when a lane holds at most 16 values of a
// row), not read again from L2 for every row.  Same arithmetic per row as
// rows_retained_kernel, so the same bits.  The reductions' LDS slots are
// reused row after row: a wave writes a slot again only after every wave
// has passed the barrier of the other reduction, i.e. after every read of
// the slot's previous value.
template <int KIND, int VEC, int EPT, int THREADS>
__global__ __launch_bounds__(THREADS) void rows_pipelined_kernel(RowArgs a)
{
    constexpr bool GB = KIND == kRowLayerNorm && EPT * VEC <= 16;
    __shared__ float red0[kMaxRowWaves], red1[kMaxRowWaves];
    const int64_t g = gridDim.x;
    int64_t row = blockIdx.x;
    Vec<VEC> v[EPT], w[EPT];
    Vec<VEC> gam[GB ? EPT : 1], bet[GB ? EPT : 1];
    load_row<KIND, VEC, EPT, THREADS>(v, a, row);
    if constexpr (GB) {
        const int64_t nvec = a.width / VEC;
#pragma unroll
        for (int k = 0; k < EPT; ++k) {
            const int64_t i = (int64_t)k * THREADS + threadIdx.x;
            if (i < nvec) {
                gam[k] = load_cached<VEC>(a.gamma + i * VEC);
                bet[k] = load_cached<VEC>(a.beta + i * VEC);
            }
        }
    }
    for (;;) {
        if (row + g < a.rows) load_row<KIND, VEC, EPT, THREADS>(w, a, row + g);
        finish_row<KIND, VEC, EPT, THREADS, GB>(v, a, row, red0, red1, gam, bet);
        row += g;
        if (row >= a.rows) break;
        if (row + g < a.rows) load_row<KIND, VEC, EPT, THREADS>(v, a, row + g);
        finish_row<KIND, VEC, EPT, THREADS, GB>(w, a, row, red0, red1, gam, bet);
        row += g;
        if (row >= a.rows) break;
    }
}

// Chan et al.'s combination of two (count, mean, sum of squared deviations)
// triples: the parallel form of Welford's one-pass variance.
struct Moments {
    float n, mean, m2;
};

__device__ __forceinline__ Moments combine(const Moments &a, const Moments &b)
{
    const float n = a.n + b.n;
    if (n == 0.f) return a;
    const float d = b.mean - a.mean;
    const float fb = b.n / n;
    return Moments{n, __builtin_fmaf(d, fb, a.mean), a.m2 + b.m2 + d * d * a.n * fb};
}

// Two passes over global memory: statistics, then the output from a second
// read of the row (served by L2 or the Infinity Cache when the row is small).
template <int KIND, int VEC, int THREADS>
__global__ __launch_bounds__(THREADS) void rows_reread_kernel(RowArgs a)
{
    __shared__ float red0[kMaxRowWaves], red1[kMaxRowWaves], red2[kMaxRowWaves];
    const int64_t row = blockIdx.x;
    const int64_t nvec = a.width / VEC;
    const float *x = a.x + row * a.width;
    float *y = a.y + row * a.width;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    if constexpr (KIND == kRowSoftmax) {
        // online maximum and rescaled sum per lane
        float m = -INFINITY, s = 0.f;
        for (int64_t i = tid; i < nvec; i += THREADS) {
            const Vec<VEC> r = load_cached<VEC>(x + i * VEC);
#pragma unroll
            for (int j = 0; j < VEC; ++j) {
                const float t = r.v[j];
                if (t > m) {
                    s = s * fexp2((m - t) * kLog2e) + 1.f;
                    m = t;
                } else if (t != -INFINITY) {
                    // a masked logit adds nothing; while m is still -inf,
                    // its exponent would be -inf - -inf = NaN
                    s += fexp2((t - m) * kLog2e);
                }
            }
        }
        const float M = block_max<THREADS>(m, red0);
        const float S = block_sum<THREADS>(m == -INFINITY ? 0.f : s * fexp2((m - M) * kLog2e), red1);
        // the same form of the exponent as in the sums above, so that their
        // rounding matches term for term
        const float inv = 1.f / S;
        for (int64_t i = tid; i < nvec; i += THREADS) {
            Vec<VEC> r = load_nt<VEC>(x + i * VEC);
#pragma unroll
            for (int j = 0; j < VEC; ++j) r.v[j] = fexp2((r.v[j] - M) * kLog2e) * inv;
            store_nt<VEC>(y + i * VEC, r);
        }
    } else {
        // Welford per lane, Chan across lanes (shuffles) and waves (LDS)
        Moments mo{0.f, 0.f, 0.f};
        for (int64_t i = tid; i < nvec; i += THREADS) {
            const Vec<VEC> r = load_cached<VEC>(x + i * VEC);
#pragma unroll
            for (int j = 0; j < VEC; ++j) {
                mo.n += 1.f;
                const float d = r.v[j] - mo.mean;
                mo.mean += d / mo.n;
                mo.m2 = __builtin_fmaf(d, r.v[j] - mo.mean, mo.m2);
            }
        }
#pragma unroll
        for (int o = 1; o < 64; o <<= 1) {
            const Moments other{__shfl_xor(mo.n, o), __shfl_xor(mo.mean, o), __shfl_xor(mo.m2, o)};
            mo = (lane & o) ? combine(other, mo) : combine(mo, other);
        }
        if (lane == 0) red0[wave] = mo.n, red1[wave] = mo.mean, red2[wave] = mo.m2;
        __syncthreads();
        Moments t{red0[0], red1[0], red2[0]};
#pragma unroll
        for (int w = 1; w < THREADS / 64; ++w) t = combine(t, Moments{red0[w], red1[w], red2[w]});
        const float mean = t.mean;
        const float rstd = 1.f / sqrtf(t.m2 / (float)a.width + a.eps);
        for (int64_t i = tid; i < nvec; i += THREADS) {
            Vec<VEC> r = load_nt<VEC>(x + i * VEC);
            const Vec<VEC> g = load_cached<VEC>(a.gamma + i * VEC);
            const Vec<VEC> b = load_cached<VEC>(a.beta + i * VEC);
#pragma unroll
            for (int j = 0; j < VEC; ++j) r.v[j] = __builtin_fmaf((r.v[j] - mean) * rstd, g.v[j], b.v[j]);
            store_nt<VEC>(y + i * VEC, r);
        }
    }
}

template <int KIND, int VEC, int EPT, int THREADS>
int launch_retained(const RowArgs &a, hipStream_t s)
{
    hipLaunchKernelGGL((rows_retained_kernel<KIND, VEC, EPT, THREADS>), dim3((unsigned)a.rows), dim3(THREADS),
                       0, s, a);
    return (int)hipGetLastError();
}

// Workgroups of `kernel` the current device holds at once (its occupancy per
// CU times the CU count), looked up once per kernel and device; 0 if the
// runtime cannot say.
template <typename K>
int resident_workgroups(K kernel, int threads)
{
    static std::atomic<int> cache[64];
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) return 0;
    if (dev >= 0 && dev < 64) {
        const int c = cache[dev].load(std::memory_order_relaxed);
        if (c > 0) return c;
    }
    int per_cu = 0, cus = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, kernel, threads, 0) != hipSuccess) return 0;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return 0;
    const int r = std::max(1, per_cu) * std::max(1, cus);
    if (dev >= 0 && dev < 64) cache[dev].store(r, std::memory_order_relaxed);
    return r;
}

// The pipelined schedule runs one round of resident workgroups: each takes
// ceil(rows / resident) rows (at least 2), so no workgroup waits for a slot
// and every one has a next row to load while it finishes the current one.
// (Measured on LayerNorm at 16K values, 2048 rows, one 1024-lane workgroup
// per CU: 8 rows per workgroup 49.3 us against 51.1 with 4; at 8K, two
// 512-lane workgroups per CU: 4 rows 26.3 us against 31.3 with 8.)
template <int KIND, int VEC, int EPT, int THREADS>
int launch_pipelined(const RowArgs &a, hipStream_t s)
{
    auto kernel = rows_pipelined_kernel<KIND, VEC, EPT, THREADS>;
    const int64_t resident = resident_workgroups(kernel, THREADS);
    const int64_t rpw = resident > 0 ? std::max<int64_t>(2, (a.rows + resident - 1) / resident) : 4;
    const int64_t grid = (a.rows + rpw - 1) / rpw;
    hipLaunchKernelGGL(kernel, dim3((unsigned)grid), dim3(THREADS), 0, s, a);
    return (int)hipGetLastError();
}

template <int KIND, int VEC>
int dispatch_retained(const RowArgs &a, hipStream_t s)
{
    const int64_t nvec = a.width / VEC;
    if constexpr (VEC == 4) {
        if (nvec <= 256) return launch_retained<KIND, 4, 1, 256>(a, s);
        if (nvec <= 512) return launch_retained<KIND, 4, 2, 256>(a, s);
        if (nvec <= 1024) return launch_retained<KIND, 4, 4, 256>(a, s);
        if (nvec <= 2048) return launch_retained<KIND, 4, 8, 256>(a, s);
        if (nvec <= 4096) return launch_retained<KIND, 4, 8, 512>(a, s);
        if (nvec <= 8192) return launch_retained<KIND, 4, 8, 1024>(a, s);
        return launch_retained<KIND, 4, 16, 1024>(a, s);
    } else {
        if (nvec <= 1024) return launch_retained<KIND, 1, 4, 256>(a, s);
        if (nvec <= 4096) return launch_retained<KIND, 1, 16, 256>(a, s);
        if (nvec <= 16384) return launch_retained<KIND, 1, 16, 1024>(a, s);
        return launch_retained<KIND, 1, 64, 1024>(a, s);
    }
}

// The pipelined schedule holds two rows per lane, so it spreads a row over
// more lanes than the one-row kernel does (at most 4 float4 per lane and
// row up to 16K values).  Wider rows (softmax: above 32K; LayerNorm, which
// also holds gamma and beta: above 16K; either with 4-byte accesses: above
// 16K) would not fit twice in a lane's registers: they take the one-row
// kernel.
template <int KIND, int VEC>
int dispatch_pipelined(const RowArgs &a, hipStream_t s)
{
    const int64_t nvec = a.width / VEC;
    if constexpr (VEC == 4) {
        if (nvec <= 256) return launch_pipelined<KIND, 4, 1, 256>(a, s);
        if (nvec <= 512) return launch_pipelined<KIND, 4, 2, 256>(a, s);
        if (nvec <= 1024) return launch_pipelined<KIND, 4, 4, 256>(a, s);
        if (nvec <= 2048) return launch_pipelined<KIND, 4, 4, 512>(a, s);
        if (nvec <= 4096) return launch_pipelined<KIND, 4, 4, 1024>(a, s);
        if constexpr (KIND == kRowSoftmax)
            if (nvec <= 8192) return launch_pipelined<KIND, 4, 8, 1024>(a, s);
    } else {
        if (nvec <= 1024) return launch_pipelined<KIND, 1, 4, 256>(a, s);
        if (nvec <= 4096) return launch_pipelined<KIND, 1, 16, 256>(a, s);
        if (nvec <= 16384) return launch_pipelined<KIND, 1, 16, 1024>(a, s);
    }
    return dispatch_retained<KIND, VEC>(a, s);
}

template <int KIND>
int dispatch(const RowArgs &a, bool vec4, bool retained, hipStream_t s)
{
    if (retained && a.pipelined)
        return vec4 ? dispatch_pipelined<KIND, 4>(a, s) : dispatch_pipelined<KIND, 1>(a, s);
    if (retained) return vec4 ? dispatch_retained<KIND, 4>(a, s) : dispatch_retained<KIND, 1>(a, s);
    const int threads = a.width >= 16384 ? 1024 : 256;
    if (vec4) {
        if (threads == 1024)
            hipLaunchKernelGGL((rows_reread_kernel<KIND, 4, 1024>), dim3((unsigned)a.rows), dim3(1024), 0, s, a);
        else
            hipLaunchKernelGGL((rows_reread_kernel<KIND, 4, 256>), dim3((unsigned)a.rows), dim3(256), 0, s, a);
    } else {
        if (threads == 1024)
            hipLaunchKernelGGL((rows_reread_kernel<KIND, 1, 1024>), dim3((unsigned)a.rows), dim3(1024), 0, s, a);
        else
            hipLaunchKernelGGL((rows_reread_kernel<KIND, 1, 256>), dim3((unsigned)a.rows), dim3(256), 0, s, a);
    }
    return (int)hipGetLastError();
}

}  // namespace

int launch_rows(const RowArgs &a, bool vec4, bool retained, void *stream)
{
    if (a.rows <= 0) return 0;
    hipStream_t s = reinterpret_cast<hipStream_t>(stream);
    return a.kind == kRowSoftmax ? dispatch<kRowSoftmax>(a, vec4, retained, s)
                                 : dispatch<kRowLayerNorm>(a, vec4, retained, s);
}

}  // namespace cap
