// Adapter pool of the paged layout: a host free-page list and a batched loader
// (S-LoRA summary, "Unified Paging" and "Adapter Loading, Prefetching, and Overlapping
// I/O with Computation"; Punica summary, "On-Demand LoRA Weight Loading").
//
// Pages all hold P fp16 elements, so allocation is a stack of page ids and never
// fragments.  Loading takes one of two routes:
//   direct: when the adapters' pages form few runs of consecutive ids (a fresh pool, or
//     pages released and taken again in order) and the blob holds its job table and page
//     ids ahead of all rank-rows, the rank-rows go host-to-device straight into the pool,
//     one copy per run (the copy engine; no kernel reads or writes them), and only the
//     job table and page ids go to the staging buffer for a small kernel that writes the
//     page-table entries and each slot's rank, scale and offsets;
//   staged: otherwise one host-to-device copy of the whole blob into the staging buffer,
//     then one kernel with a small fixed grid that scatters every page as well.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cstdint>
#include <cstring>
#include <string>
#include <tuple>
#include <unordered_map>
#include <vector>

#include "lora_internal.hpp"

namespace lora {
namespace {

// ------------------------------------------------------------------------ free-page list
// Caller-owned state: header, a stack of free ids (top = most recently returned) and one
// byte per page (1 = taken).
struct PoolHeader {
    uint64_t magic;
    int64_t num_pages;
    int64_t free_top;  // number of ids on the stack
    int64_t reserved;
};
constexpr uint64_t kPoolMagic = 0x4c6f5241506f6f6cULL;

inline size_t state_bytes(int64_t num_pages)
{
    const size_t b = sizeof(PoolHeader) + (size_t)num_pages * sizeof(int32_t) + (size_t)num_pages;
    return (b + 15) & ~size_t(15);
}

inline int32_t *stack_of(PoolHeader *h) { return reinterpret_cast<int32_t *>(h + 1); }
inline uint8_t *taken_of(PoolHeader *h) { return reinterpret_cast<uint8_t *>(stack_of(h) + h->num_pages); }

PoolHeader *pool_state(void *state)
{
    auto *h = static_cast<PoolHeader *>(state);
    return (h && h->magic == kPoolMagic) ? h : nullptr;
}

// ------------------------------------------------------------------------ loader
// One job as the scatter kernel reads it from the staging buffer.
struct alignas(16) LoadJobDev {
    uint16_t *pool;
    int32_t *page_table;
    int64_t *a_pt_off, *b_pt_off;
    int32_t *rank;
    float *scale;
    int64_t pt_off, data_off, pages_off;  // offsets into the page table / the staging buffer
    int32_t d_in, d_out, P, slot, r, n_pages;
    float sc;
    int32_t pad[3];
};
static_assert(sizeof(LoadJobDev) % 16 == 0, "job records keep 16-byte alignment");

constexpr int kLoadThreads = 256;
constexpr int kLoadUnroll = 8;        // pages per lane group per work item (loads in flight per lane)
#ifndef LORA_LOAD_WORKGROUPS
#define LORA_LOAD_WORKGROUPS 1024
#endif
constexpr int kLoadWorkgroups = LORA_LOAD_WORKGROUPS;  // the scatter's grid: four workgroups per CU

constexpr int kMetaWorkgroups = 256;  // the direct route's kernel: page-table entries and slot fields only
constexpr size_t kDirectRuns = 64;    // most runs of consecutive pages the direct route copies one by one

// The direct route's kernel (the pages are already in place): work item f (of n_jobs *
// gx) is job f / gx, entries [256 (f % gx), 256 (f % gx) + 256) of its page-table range,
// one per thread; the first item of a job also writes the slot's rank, scale and
// page-table offsets.
__global__ __launch_bounds__(kLoadThreads) void lora_pool_meta_kernel(const unsigned char *staging, int32_t n_jobs,
                                                                      int64_t gx)
{
    const LoadJobDev *jobs = reinterpret_cast<const LoadJobDev *>(staging);
    const int tid = threadIdx.x;
    for (int64_t f = blockIdx.x; f < (int64_t)n_jobs * gx; f += gridDim.x) {
        const int64_t jx = f / gx, bx = f - jx * gx;
        const LoadJobDev &jb = jobs[jx];
        if (bx == 0 && tid == 0) {
            jb.rank[jb.slot] = jb.r;
            if (jb.r > 0) {
                jb.scale[jb.slot] = jb.sc;
                jb.a_pt_off[jb.slot] = jb.pt_off;
                jb.b_pt_off[jb.slot] = jb.pt_off + (int64_t)jb.r * (jb.d_in / jb.P);
            }
        }
        const int64_t e = bx * kLoadThreads + tid;
        if (e < jb.n_pages)
            jb.page_table[jb.pt_off + e] = reinterpret_cast<const int32_t *>(staging + jb.pages_off)[e];
    }
}

// Work item f (of n_jobs * gx) is job f / gx, page block f % gx: kLoadUnroll groups of
// ppw pages, each page copied by P/8 lanes (16 bytes per lane) or, for P > 2048, by the
// whole workgroup in a loop.  The small fixed grid walks the items in a grid-stride loop,
// so a load takes few CU slots from kernels running beside it, and each lane has
// kLoadUnroll loads in flight before its stores.  The first item of a job also writes
// the slot's rank, scale and page-table offsets.
__global__ __launch_bounds__(kLoadThreads) void lora_pool_scatter_kernel(const unsigned char *staging, int32_t n_jobs,
                                                                         int64_t gx)
{
    const LoadJobDev *jobs = reinterpret_cast<const LoadJobDev *>(staging);
    const int tid = threadIdx.x;
    for (int64_t f = blockIdx.x; f < (int64_t)n_jobs * gx; f += gridDim.x) {
        const int64_t jx = f / gx, bx = f - jx * gx;
        const LoadJobDev &jb = jobs[jx];
        if (bx == 0 && tid == 0) {
            jb.rank[jb.slot] = jb.r;
            if (jb.r > 0) {
                jb.scale[jb.slot] = jb.sc;
                jb.a_pt_off[jb.slot] = jb.pt_off;
                jb.b_pt_off[jb.slot] = jb.pt_off + (int64_t)jb.r * (jb.d_in / jb.P);
            }
        }
        const int lanes = min(kLoadThreads, jb.P / 8);  // lanes per page
        const int ppw = kLoadThreads / lanes;             // pages per workgroup and unroll step
        const int g = tid / lanes, lane = tid % lanes;
        if (g >= ppw) continue;
        const int64_t a_pages = (int64_t)jb.r * (jb.d_in / jb.P);
        const uint16_t *data = reinterpret_cast<const uint16_t *>(staging + jb.data_off);
        const int32_t *ids = reinterpret_cast<const int32_t *>(staging + jb.pages_off);
        int64_t e0 = bx * ppw * kLoadUnroll + g;
        // element offset of page e's first element in the job's data
        auto src_of = [&](int64_t e) {
            if (e < a_pages) {
                const int64_t per = jb.d_in / jb.P, j = e / per, q = e - j * per;
                return j * jb.d_in + q * jb.P;
            }
            const int64_t per = jb.d_out / jb.P, e2 = e - a_pages, j = e2 / per, q = e2 - j * per;
            return (int64_t)jb.r * jb.d_in + j * jb.d_out + q * jb.P;
        };
        for (int k = 8 * lane; k < jb.P; k += 8 * lanes) {
            uint4 v[kLoadUnroll];
#pragma unroll
            for (int u = 0; u < kLoadUnroll; ++u) {
                const int64_t e = e0 + (int64_t)u * ppw;
                if (e < jb.n_pages) v[u] = *reinterpret_cast<const uint4 *>(data + src_of(e) + k);
            }
#pragma unroll
            for (int u = 0; u < kLoadUnroll; ++u) {
                const int64_t e = e0 + (int64_t)u * ppw;
                if (e < jb.n_pages) *reinterpret_cast<uint4 *>(jb.pool + (int64_t)ids[e] * jb.P + k) = v[u];
            }
        }
        if (lane == 0) {
#pragma unroll
            for (int u = 0; u < kLoadUnroll; ++u) {
                const int64_t e = e0 + (int64_t)u * ppw;
                if (e < jb.n_pages) jb.page_table[jb.pt_off + e] = ids[e];
            }
        }
    }
}

int64_t pages_for(const lora_weights *w, int32_t r)
{
    const int32_t P = w->page_elems;
    return (int64_t)r * (w->d_in / P + w->d_out / P);
}

}  // namespace
}  // namespace lora

using namespace lora;

extern "C" {

size_t lora_pool_state_bytes(int64_t num_pages)
{
    if (num_pages < 1 || num_pages > INT32_MAX) return 0;
    return state_bytes(num_pages);
}

int lora_pool_init(void *state, size_t bytes, int64_t num_pages)
{
    clear_error();
    if (!state) return fail(LORA_E_NULL, "pool state is NULL");
    if (num_pages < 1 || num_pages > INT32_MAX)
        return fail(LORA_E_SHAPE, "num_pages = %lld outside 1..%d", (long long)num_pages, INT32_MAX);
    if (bytes < state_bytes(num_pages))
        return fail(LORA_E_CAPACITY, "pool state needs %zu bytes, got %zu", state_bytes(num_pages), bytes);
    auto *h = static_cast<PoolHeader *>(state);
    h->magic = kPoolMagic;
    h->num_pages = num_pages;
    h->free_top = num_pages;
    h->reserved = 0;
    int32_t *st = stack_of(h);
    for (int64_t i = 0; i < num_pages; ++i) st[i] = (int32_t)(num_pages - 1 - i);  // page 0 on top
    std::memset(taken_of(h), 0, (size_t)num_pages);
    return LORA_OK;
}

int lora_pool_alloc(void *state, int32_t n, int32_t *pages)
{
    clear_error();
    PoolHeader *h = pool_state(state);
    if (!h) return fail(LORA_E_NULL, "pool state is NULL or not initialised");
    if (n < 0) return fail(LORA_E_SHAPE, "n = %d", n);
    if (n > 0 && !pages) return fail(LORA_E_NULL, "pages is NULL");
    if (n > h->free_top)
        return fail(LORA_E_CAPACITY, "%d pages requested, %lld free", n, (long long)h->free_top);
    int32_t *st = stack_of(h);
    uint8_t *tk = taken_of(h);
    for (int32_t i = 0; i < n; ++i) {
        const int32_t id = st[--h->free_top];
        tk[id] = 1;
        pages[i] = id;
    }
    return LORA_OK;
}

int lora_pool_release(void *state, int32_t n, const int32_t *pages)
{
    clear_error();
    PoolHeader *h = pool_state(state);
    if (!h) return fail(LORA_E_NULL, "pool state is NULL or not initialised");
    if (n < 0) return fail(LORA_E_SHAPE, "n = %d", n);
    if (n > 0 && !pages) return fail(LORA_E_NULL, "pages is NULL");
    uint8_t *tk = taken_of(h);
    // check all (marking each id once), then undo the marks or commit
    int32_t bad = -1;
    for (int32_t i = 0; i < n && bad < 0; ++i) {
        const int32_t id = pages[i];
        if (id < 0 || id >= h->num_pages || tk[id] != 1) bad = i;
        else tk[id] = 2;
    }
    for (int32_t i = 0; i < (bad < 0 ? n : bad); ++i) tk[pages[i]] = 1;
    if (bad >= 0)
        return fail(LORA_E_INDEX, "page %d (entry %d) is out of range, not taken, or listed twice", pages[bad], bad);
    // pushed last to first: the next lora_pool_alloc hands them out in the order listed,
    // so pages released in ascending runs come back as the same runs
    int32_t *st = stack_of(h);
    for (int32_t i = n - 1; i >= 0; --i) {
        tk[pages[i]] = 0;
        st[h->free_top++] = pages[i];
    }
    return LORA_OK;
}

int64_t lora_pool_free_count(const void *state)
{
    const auto *h = static_cast<const PoolHeader *>(state);
    return (h && h->magic == kPoolMagic) ? h->free_top : -1;
}

int64_t lora_pool_pages_for(int32_t rank, int32_t d_in, int32_t d_out, int32_t page_elems)
{
    clear_error();
    if (rank < 0 || d_in <= 0 || d_out <= 0 || page_elems < 8 || page_elems % 8 || d_in % page_elems ||
        d_out % page_elems)
        return fail(LORA_E_SHAPE, "rank %d, d_in %d, d_out %d, page_elems %d", rank, d_in, d_out, page_elems);
    return (int64_t)rank * (d_in / page_elems + d_out / page_elems);
}

size_t lora_pool_load_header_bytes(int32_t n_jobs)
{
    return n_jobs > 0 ? (size_t)n_jobs * sizeof(LoadJobDev) : 0;
}

int lora_pool_load(void *stream, int32_t n_jobs, const lora_load_job *jobs, void *blob, size_t blob_bytes,
                   void *staging, size_t staging_bytes)
{
    clear_error();
    if (n_jobs < 0) return fail(LORA_E_SHAPE, "n_jobs = %d", n_jobs);
    if (n_jobs == 0) return LORA_OK;
    if (!jobs || !blob || !staging) return fail(LORA_E_NULL, "jobs, blob and staging are required");
    if (!aligned16(blob) || !aligned16(staging)) return fail(LORA_E_ALIGN, "blob and staging must be 16-byte aligned");
    const size_t header = lora_pool_load_header_bytes(n_jobs);
    if (blob_bytes < header) return fail(LORA_E_CAPACITY, "blob of %zu bytes is smaller than the %zu-byte job table",
                                         blob_bytes, header);
    if (staging_bytes < blob_bytes)
        return fail(LORA_E_CAPACITY, "staging of %zu bytes is smaller than the blob (%zu)", staging_bytes, blob_bytes);
    const unsigned char *bytes = static_cast<const unsigned char *>(blob);
    // (pool, page) pairs, (page table, first, last) ranges and (offset array, slot) / (rank array, slot) keys
    std::unordered_map<const void *, std::vector<uint8_t>> pages_named;  // per pool: page already named
    std::vector<std::tuple<const void *, int64_t, int64_t>> ranges;
    std::vector<std::tuple<const void *, int32_t, int32_t>> offset_keys;
    std::vector<std::tuple<const void *, int32_t, int32_t, float>> rank_keys;
    for (int32_t i = 0; i < n_jobs; ++i) {
        const lora_load_job &jb = jobs[i];
        int st = check_weights_desc(jb.w);
        if (st) {
            const std::string why = lora_last_error();  // fail() rewrites that buffer
            return fail(st, "job %d: %s", i, why.c_str());
        }
        const lora_weights *w = jb.w;
        if (w->layout != LORA_LAYOUT_PAGED) return fail(LORA_E_UNSUPPORTED, "job %d: target is not paged", i);
        if (jb.slot < 0 || jb.slot >= w->num_slots)
            return fail(LORA_E_INDEX, "job %d: slot %d outside 0..%d", i, jb.slot, w->num_slots - 1);
        if (jb.rank < 0 || jb.rank > w->r_max)
            return fail(LORA_E_SHAPE, "job %d: rank %d outside 0..%d", i, jb.rank, w->r_max);
        if (jb.reserved != 0) return fail(LORA_E_SHAPE, "job %d: reserved field must be 0", i);
        rank_keys.emplace_back(w->rank, jb.slot, jb.rank, jb.scale);
        if (jb.rank == 0) continue;
        offset_keys.emplace_back(w->a_pt_off, jb.slot, i);
        const int64_t np = pages_for(w, jb.rank);
        if (jb.pt_off < 0 || jb.pt_off > w->pt_entries - np)
            return fail(LORA_E_INDEX, "job %d: page-table entries %lld..%lld outside 0..%lld", i, (long long)jb.pt_off,
                        (long long)(jb.pt_off + np - 1), (long long)w->pt_entries - 1);
        const int64_t data_bytes = 2 * (int64_t)jb.rank * ((int64_t)w->d_in + w->d_out);
        if (jb.data_off % 16) return fail(LORA_E_ALIGN, "job %d: data_off %lld is not a multiple of 16", i,
                                          (long long)jb.data_off);
        if (jb.pages_off % 4) return fail(LORA_E_ALIGN, "job %d: pages_off %lld is not a multiple of 4", i,
                                          (long long)jb.pages_off);
        if (jb.data_off < (int64_t)header || jb.data_off > (int64_t)blob_bytes - data_bytes)
            return fail(LORA_E_SHAPE, "job %d: data bytes %lld..%lld outside the blob after the job table", i,
                        (long long)jb.data_off, (long long)(jb.data_off + data_bytes));
        if (jb.pages_off < (int64_t)header || jb.pages_off > (int64_t)blob_bytes - 4 * np)
            return fail(LORA_E_SHAPE, "job %d: page ids %lld..%lld outside the blob after the job table", i,
                        (long long)jb.pages_off, (long long)(jb.pages_off + 4 * np));
        const int32_t *ids = reinterpret_cast<const int32_t *>(bytes + jb.pages_off);
        std::vector<uint8_t> &named = pages_named[w->pool];
        if ((int64_t)named.size() < w->num_pages) named.resize((size_t)w->num_pages, 0);
        for (int64_t e = 0; e < np; ++e) {
            if (ids[e] < 0 || ids[e] >= w->num_pages)
                return fail(LORA_E_INDEX, "job %d: page id %d (entry %lld) outside 0..%lld", i, ids[e], (long long)e,
                            (long long)w->num_pages - 1);
            if (named[ids[e]]) return fail(LORA_E_INDEX, "page %d of one pool is named twice", ids[e]);
            named[ids[e]] = 1;
        }
        ranges.emplace_back(w->page_table, jb.pt_off, jb.pt_off + np);
    }
    std::sort(ranges.begin(), ranges.end());
    for (size_t i = 1; i < ranges.size(); ++i)
        if (std::get<0>(ranges[i]) == std::get<0>(ranges[i - 1]) && std::get<1>(ranges[i]) < std::get<2>(ranges[i - 1]))
            return fail(LORA_E_INDEX, "page-table ranges of two jobs overlap at entry %lld",
                        (long long)std::get<1>(ranges[i]));
    std::sort(offset_keys.begin(), offset_keys.end());
    for (size_t i = 1; i < offset_keys.size(); ++i)
        if (std::get<0>(offset_keys[i]) == std::get<0>(offset_keys[i - 1]) &&
            std::get<1>(offset_keys[i]) == std::get<1>(offset_keys[i - 1]))
            return fail(LORA_E_INDEX, "two jobs load slot %d of one target", std::get<1>(offset_keys[i]));
    std::sort(rank_keys.begin(), rank_keys.end(), [](const auto &x, const auto &y) {
        return std::get<0>(x) != std::get<0>(y) ? std::get<0>(x) < std::get<0>(y) : std::get<1>(x) < std::get<1>(y);
    });
    for (size_t i = 1; i < rank_keys.size(); ++i)
        if (std::get<0>(rank_keys[i]) == std::get<0>(rank_keys[i - 1]) &&
            std::get<1>(rank_keys[i]) == std::get<1>(rank_keys[i - 1]) &&
            (std::get<2>(rank_keys[i]) != std::get<2>(rank_keys[i - 1]) ||
             std::get<3>(rank_keys[i]) != std::get<3>(rank_keys[i - 1])))
            return fail(LORA_E_INDEX, "two jobs give slot %d of one rank array different ranks or scales",
                        std::get<1>(rank_keys[i]));

    // job table into the blob's header
    LoadJobDev *table = static_cast<LoadJobDev *>(blob);
    for (int32_t i = 0; i < n_jobs; ++i) {
        const lora_load_job &jb = jobs[i];
        const lora_weights *w = jb.w;
        LoadJobDev d{};
        d.pool = static_cast<uint16_t *>(const_cast<void *>(w->pool));
        d.page_table = const_cast<int32_t *>(w->page_table);
        d.a_pt_off = const_cast<int64_t *>(w->a_pt_off);
        d.b_pt_off = const_cast<int64_t *>(w->b_pt_off);
        d.rank = const_cast<int32_t *>(w->rank);
        d.scale = const_cast<float *>(w->scale);
        d.pt_off = jb.pt_off;
        d.data_off = jb.data_off;
        d.pages_off = jb.pages_off;
        d.d_in = w->d_in;
        d.d_out = w->d_out;
        d.P = w->page_elems;
        d.slot = jb.slot;
        d.r = jb.rank;
        d.n_pages = jb.rank > 0 ? (int32_t)pages_for(w, jb.rank) : 0;
        d.sc = jb.scale;
        table[i] = d;
    }
    // The direct route's runs: page e of a job sits at data_off + e * 2P bytes of the blob
    // (its rank-rows are contiguous) and goes to page ids[e] of its pool; consecutive
    // pages extend a run while both sides stay contiguous, across jobs too.
    struct Run {
        unsigned char *dst;
        int64_t src, bytes;
    };
    std::vector<Run> runs;
    size_t meta_end = header;  // the job table and every page-id list end here ...
    int64_t data_begin = (int64_t)blob_bytes;  // ... and must not reach into the rank-rows
    bool direct = true;
    for (int32_t i = 0; i < n_jobs && direct; ++i) {
        const LoadJobDev &d = table[i];
        if (d.n_pages == 0) continue;
        meta_end = std::max(meta_end, (size_t)(d.pages_off + 4 * (int64_t)d.n_pages));
        data_begin = std::min(data_begin, d.data_off);
        const int32_t *ids = reinterpret_cast<const int32_t *>(bytes + d.pages_off);
        const int64_t pb = 2 * (int64_t)d.P;
        auto *pool = reinterpret_cast<unsigned char *>(d.pool);
        for (int64_t e = 0; e < d.n_pages; ++e) {
            unsigned char *dst = pool + (int64_t)ids[e] * pb;
            const int64_t src = d.data_off + e * pb;
            if (!runs.empty() && runs.back().dst + runs.back().bytes == dst && runs.back().src + runs.back().bytes == src) {
                runs.back().bytes += pb;
            } else if (runs.size() == kDirectRuns) {
                direct = false;
                break;
            } else {
                runs.push_back(Run{dst, src, pb});
            }
        }
    }
    direct = direct && (int64_t)meta_end <= data_begin;
    hipStream_t s = static_cast<hipStream_t>(stream);
    hipError_t e = hipMemcpyAsync(staging, blob, direct ? meta_end : blob_bytes, hipMemcpyHostToDevice, s);
    if (e != hipSuccess) return fail(LORA_E_HIP, "pool load copy: %s", hipGetErrorString(e));
    // work items per job: enough blocks (of pages, or of page-table entries on the direct
    // route) for the job with the most pages
    int64_t gx = 1;
    for (int32_t i = 0; i < n_jobs; ++i) {
        const LoadJobDev &d = table[i];
        const int64_t block =
            direct ? kLoadThreads : (int64_t)(kLoadThreads / std::min(kLoadThreads, d.P / 8)) * kLoadUnroll;
        gx = std::max<int64_t>(gx, (d.n_pages + block - 1) / block);
    }
    const int64_t items = (int64_t)n_jobs * gx;
    const dim3 grid((unsigned)std::min<int64_t>(items, direct ? kMetaWorkgroups : kLoadWorkgroups));
    const auto *stg = static_cast<const unsigned char *>(staging);
    // The direct route's kernel runs right after the small staging copy and before the
    // rank-rows' copies: a kernel queued behind a long copy would hold its compute queue
    // (and whatever else shares that queue) until the copy is done.  The page-table
    // entries and slot fields may land before the pages; readers order themselves after
    // the whole load anyway.
    if (direct) hipLaunchKernelGGL(lora_pool_meta_kernel, grid, dim3(kLoadThreads), 0, s, stg, n_jobs, gx);
    else hipLaunchKernelGGL(lora_pool_scatter_kernel, grid, dim3(kLoadThreads), 0, s, stg, n_jobs, gx);
    e = hipGetLastError();
    if (e != hipSuccess) return fail(LORA_E_HIP, "pool load launch: %s", hipGetErrorString(e));
    if (direct) {
        for (const Run &r : runs) {
            e = hipMemcpyAsync(r.dst, bytes + r.src, (size_t)r.bytes, hipMemcpyHostToDevice, s);
            if (e != hipSuccess) return fail(LORA_E_HIP, "pool load copy: %s", hipGetErrorString(e));
        }
    }
    return LORA_OK;
}

}  // extern "C"
