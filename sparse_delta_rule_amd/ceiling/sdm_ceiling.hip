// Reference access patterns over a bank of rows (include/sdm_ceiling.h): what
// random rows allow on this device, measured with the row layout the decode
// and gather kernels use (16-byte vectors on consecutive lanes, several rows in
// flight per lane group, every load of a batch issued before any is used).
// None of the method's arithmetic is here.

#include <hip/hip_runtime.h>
#include <stdarg.h>
#include <stdint.h>
#include <stdio.h>

#include "../../include/sdm_ceiling.h"

namespace {

constexpr int kThreads = 256;
constexpr int kMaxBlocks = 2048;  // at most 8 workgroups of 256 threads on each of 256 compute units

thread_local char g_error[512] = "";

int fail(int code, const char* fmt, ...) {
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(g_error, sizeof g_error, fmt, ap);
    va_end(ap);
    return code;
}

typedef uint32_t U32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ uint4 load_nt(const uint4* p) {
    const U32x4 w = __builtin_nontemporal_load(reinterpret_cast<const U32x4*>(p));
    return make_uint4(w.x, w.y, w.z, w.w);
}
__device__ __forceinline__ void store_nt(uint4* p, uint4 v) {
    const U32x4 w = {v.x, v.y, v.z, v.w};
    __builtin_nontemporal_store(w, reinterpret_cast<U32x4*>(p));
}
__device__ __forceinline__ uint32_t fold(uint4 v) { return v.x ^ v.y ^ v.z ^ v.w; }
__device__ __forceinline__ uint4 flip(uint4 v) {
    const uint32_t m = 0x00010001u;
    return make_uint4(v.x ^ m, v.y ^ m, v.z ^ m, v.w ^ m);
}

// A lane group of lpr lanes (a power of two) per row; lane l owns vector l of
// every row (vpr vectors; lanes past the row repeat the last vector, and their
// stores write the same bits to the same place). Group g takes batches of NB
// units [b, b + NB), b = g NB, g NB + stride, ...; units past n repeat unit
// n - 1 (the same row and the same bits), so no load or store sits under a
// branch. The next batch's row numbers are requested while this batch's rows
// are in flight, so a batch costs one memory round trip, not two.
template <int MODE>
__device__ __forceinline__ void load_slots(int64_t (&slot)[8], int64_t (&rslot)[8], const int64_t* rows, int64_t b,
                                           int64_t n, int nb) {
#pragma unroll
    for (int j = 0; j < 8; ++j) {
        if (j >= nb) break;
        const int64_t u = b + j < n ? b + j : n - 1;
        slot[j] = rows[MODE == SDM_CEIL_MIX ? 2 * u : u];
        if constexpr (MODE == SDM_CEIL_MIX) rslot[j] = rows[2 * u + 1];
    }
}

template <int MODE, int NB>
__global__ __launch_bounds__(kThreads) void ceiling_rows_kernel(uint4* bank, int vpr, int lpr, const int64_t* rows,
                                                                int64_t n, uint4* stash, uint32_t* sink) {
    const int lane = threadIdx.x & (lpr - 1);
    const int grp = threadIdx.x / lpr;
    const int groups = kThreads / lpr;
    const bool active = lane < vpr;
    const int vl = active ? lane : vpr - 1;
    const int64_t stride = int64_t(gridDim.x) * groups * NB;
    uint32_t acc = 0;
    int64_t slot[8], rslot[8];
    int64_t b = (int64_t(blockIdx.x) * groups + grp) * NB;
    if (b < n) load_slots<MODE>(slot, rslot, rows, b, n, NB);
    for (; b < n; b += stride) {
        uint4 r[NB], q[NB];
#pragma unroll
        for (int j = 0; j < NB; ++j) {
            const uint4* p = bank + slot[j] * vpr + vl;
            if constexpr (MODE == SDM_CEIL_READ || MODE == SDM_CEIL_STASH)
                r[j] = load_nt(p);
            else
                r[j] = *p;
            if constexpr (MODE == SDM_CEIL_MIX) q[j] = bank[rslot[j] * vpr + vl];
        }
        int64_t wslot[NB];
#pragma unroll
        for (int j = 0; j < NB; ++j) wslot[j] = slot[j];
        // the next batch's row numbers (clamped into the list; unused past the end)
        const int64_t nb = b + stride < n ? b + stride : b;
        load_slots<MODE>(slot, rslot, rows, nb, n, NB);
#pragma unroll
        for (int j = 0; j < NB; ++j) {
            const bool use = active && b + j < n;
            const int64_t u = b + j < n ? b + j : n - 1;
            if constexpr (MODE == SDM_CEIL_READ) acc ^= use ? fold(r[j]) : 0u;
            if constexpr (MODE == SDM_CEIL_STASH) store_nt(stash + u * vpr + vl, r[j]);
            if constexpr (MODE == SDM_CEIL_RMW || MODE == SDM_CEIL_MIX) bank[wslot[j] * vpr + vl] = flip(r[j]);
            if constexpr (MODE == SDM_CEIL_MIX) acc ^= use ? fold(q[j]) : 0u;
        }
    }
    if constexpr (MODE == SDM_CEIL_READ || MODE == SDM_CEIL_MIX)
        sink[int64_t(blockIdx.x) * kThreads + threadIdx.x] = acc;
}

// Streaming copy: workgroup b copies the contiguous chunk of kThreads * NB
// vectors starting at b kThreads NB, NB vectors in flight per thread (vector
// j kThreads + t of the chunk for thread t); vectors past the end repeat the
// last one (the same bits to the same place). NT: non-temporal loads and stores.
template <int NB, bool NT>
__global__ __launch_bounds__(kThreads) void ceiling_copy_kernel(uint4* dst, const uint4* src, int64_t nvec) {
    const int64_t base = int64_t(blockIdx.x) * kThreads * NB + threadIdx.x;
    uint4 v[NB];
#pragma unroll
    for (int j = 0; j < NB; ++j) {
        const int64_t i = base + int64_t(j) * kThreads;
        const uint4* p = src + (i < nvec ? i : nvec - 1);
        v[j] = NT ? load_nt(p) : *p;
    }
#pragma unroll
    for (int j = 0; j < NB; ++j) {
        const int64_t i = base + int64_t(j) * kThreads;
        uint4* p = dst + (i < nvec ? i : nvec - 1);
        if constexpr (NT)
            store_nt(p, v[j]);
        else
            *p = v[j];
    }
}

int pow2_ceil(int64_t x) {
    int p = 1;
    while (p < x) p <<= 1;
    return p;
}

// Workgroups of a persistent grid: as many as are resident at once on the
// current device (at most kMaxBlocks), so that no workgroup waits for another to
// finish before it starts.
template <typename K>
int64_t resident_blocks(K kernel) {
    int dev = 0, cus = 0, per_cu = 0;
    if (hipGetDevice(&dev) != hipSuccess || hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) !=
                                                hipSuccess ||
        hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, kernel, kThreads, 0) != hipSuccess || cus * per_cu < 1)
        return kMaxBlocks;
    const int64_t r = int64_t(cus) * per_cu;
    return r < kMaxBlocks ? r : kMaxBlocks;
}

template <int MODE, int NB>
hipError_t launch_rows(uint4* bank, int vpr, const int64_t* rows, int64_t n, uint4* stash, uint32_t* sink,
                       hipStream_t stream) {
    const int lpr = pow2_ceil(vpr);
    const int64_t per_block = int64_t(kThreads / lpr) * NB;
    int64_t blocks = (n + per_block - 1) / per_block;
    const int64_t cap = resident_blocks(ceiling_rows_kernel<MODE, NB>);
    if (blocks > cap) blocks = cap;
    hipLaunchKernelGGL((ceiling_rows_kernel<MODE, NB>), dim3(unsigned(blocks)), dim3(kThreads), 0, stream, bank, vpr,
                       lpr, rows, n, stash, sink);
    return hipGetLastError();
}

}  // namespace

extern "C" {

int sdm_ceiling_rows(int mode, void* bank, int64_t num_rows, int64_t row_bytes, const int64_t* rows, int64_t n,
                     void* stash, uint32_t* sink, void* hip_stream) {
    if (mode < SDM_CEIL_READ || mode > SDM_CEIL_MIX) return fail(2, "sdm_ceiling_rows: unknown mode %d", mode);
    if (num_rows < 1 || row_bytes < 16 || row_bytes > 1024 || row_bytes % 16 != 0 || n < 0)
        return fail(2, "sdm_ceiling_rows: need num_rows >= 1, row_bytes a multiple of 16 in [16, 1024] and n >= 0 "
                    "(got %lld, %lld, %lld)", (long long)num_rows, (long long)row_bytes, (long long)n);
    if (n == 0) return 0;
    if (bank == nullptr || rows == nullptr) return fail(6, "sdm_ceiling_rows: bank and rows are required");
    if (mode == SDM_CEIL_STASH && stash == nullptr) return fail(6, "sdm_ceiling_rows: the stash pattern needs a stash");
    if ((mode == SDM_CEIL_READ || mode == SDM_CEIL_MIX) && sink == nullptr)
        return fail(6, "sdm_ceiling_rows: the read patterns need a sink");
    if (reinterpret_cast<uintptr_t>(bank) % 16 != 0 || (stash && reinterpret_cast<uintptr_t>(stash) % 16 != 0))
        return fail(2, "sdm_ceiling_rows: bank and stash must be 16-byte aligned");
    const int vpr = int(row_bytes / 16);
    uint4* b = static_cast<uint4*>(bank);
    uint4* st = static_cast<uint4*>(stash);
    hipStream_t stream = static_cast<hipStream_t>(hip_stream);
    hipError_t e;
    switch (mode) {
        case SDM_CEIL_READ: e = launch_rows<SDM_CEIL_READ, 8>(b, vpr, rows, n, st, sink, stream); break;
        case SDM_CEIL_STASH: e = launch_rows<SDM_CEIL_STASH, 8>(b, vpr, rows, n, st, sink, stream); break;
        case SDM_CEIL_RMW: e = launch_rows<SDM_CEIL_RMW, 8>(b, vpr, rows, n, st, sink, stream); break;
        default: e = launch_rows<SDM_CEIL_MIX, 4>(b, vpr, rows, n, st, sink, stream); break;
    }
    if (e != hipSuccess) return fail(8, "sdm_ceiling_rows: launch failed: %s", hipGetErrorString(e));
    return 0;
}

int64_t sdm_ceiling_sink_words(void) { return int64_t(kMaxBlocks) * kThreads; }

int sdm_ceiling_copy(void* dst, const void* src, int64_t bytes, int nontemporal, void* hip_stream) {
    if (bytes < 0 || bytes % 16 != 0) return fail(2, "sdm_ceiling_copy: bytes must be a multiple of 16, got %lld",
                                                  (long long)bytes);
    if (bytes == 0) return 0;
    if (dst == nullptr || src == nullptr) return fail(6, "sdm_ceiling_copy: dst and src are required");
    if (reinterpret_cast<uintptr_t>(dst) % 16 != 0 || reinterpret_cast<uintptr_t>(src) % 16 != 0)
        return fail(2, "sdm_ceiling_copy: dst and src must be 16-byte aligned");
    const int64_t nvec = bytes / 16;
    constexpr int NB = 8;
    const int64_t blocks = (nvec + int64_t(kThreads) * NB - 1) / (int64_t(kThreads) * NB);
    if (blocks > 0x7fffffffLL) return fail(2, "sdm_ceiling_copy: %lld bytes is too many", (long long)bytes);
    if (nontemporal)
        hipLaunchKernelGGL((ceiling_copy_kernel<NB, true>), dim3(unsigned(blocks)), dim3(kThreads), 0,
                           static_cast<hipStream_t>(hip_stream), static_cast<uint4*>(dst),
                           static_cast<const uint4*>(src), nvec);
    else
        hipLaunchKernelGGL((ceiling_copy_kernel<NB, false>), dim3(unsigned(blocks)), dim3(kThreads), 0,
                           static_cast<hipStream_t>(hip_stream), static_cast<uint4*>(dst),
                           static_cast<const uint4*>(src), nvec);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return fail(8, "sdm_ceiling_copy: launch failed: %s", hipGetErrorString(e));
    return 0;
}

const char* sdm_ceiling_last_error(void) { return g_error; }

}  // extern "C"
