// SDM token gather on gfx950.
//
// Per token and operand a float32-accumulated weighted sum of random bank rows,
// a raw copy of operand 0's rows (the stash), and zeros for padding positions
// (page "sparse_delta_memory/cuda/gather_cuda.py", module docstring).
//
// Layout: a token is handled by LPR consecutive lanes (a power of two, up to a
// whole 64-lane wavefront); lane l owns vector (slice * LPR + l) of every row,
// so each row is read with 16-byte loads (narrower when a row is not a multiple
// of 16 bytes) and each lane accumulates its own columns. A lane walks the
// entries in ascending order, one fused multiply-add chain per output element:
// no cross-lane reduction, and the result depends on the inputs alone.
//
// Memory pipeline: the slots and weights of the block's live tokens are staged
// in LDS with contiguous loads (CH entries per token at a time), so the only
// global round trips inside a token's loop are its row loads. Entries are then
// taken NB at a time (both operands together while both have entries), all of
// a batch's row loads issued before the first is used; the HBM latency is
// hidden by those and by the many tokens resident per CU. Padding tokens read
// no slot, weight or row.

#include "sdm_kernels.h"

namespace sdm {

namespace {

constexpr int kThreads = 256;
constexpr int kStageEntries = 1024;  // tokens per block x entries per token staged at once

// N consecutive entries [n0, n0 + N) of the operands selected by DO0 / DO1, all
// valid: every row load is issued before the first row is used, and nothing
// in between is conditional (a guarded use would let the compiler move its
// load next to it and wait there).
template <typename E, int VB, int N, bool DO0, bool DO1, typename IdxT, typename WT>
__device__ __forceinline__ void gather_batch(const E* __restrict__ bank, int64_t hd, int64_t col, int n0, int krel,
                                             const IdxT* s_idx0, const WT* s_w0, const IdxT* s_idx1,
                                             const WT* s_w1, E* stash_row, float (&acc0)[VB / sizeof(E)],
                                             float (&acc1)[VB / sizeof(E)]) {
    using V = typename RawVec<VB>::T;
    constexpr int VEC = VB / int(sizeof(E));
    V r0[N], r1[N];
    float x0[N], x1[N];
#pragma unroll
    for (int i = 0; i < N; ++i) {
        if (DO0) {
            r0[i] = *reinterpret_cast<const V*>(bank + int64_t(s_idx0[krel + i]) * hd + col);
            x0[i] = value_of<WT>(s_w0[krel + i]);
        }
        if (DO1) {
            r1[i] = *reinterpret_cast<const V*>(bank + int64_t(s_idx1[krel + i]) * hd + col);
            x1[i] = value_of<WT>(s_w1[krel + i]);
        }
    }
#pragma unroll
    for (int i = 0; i < N; ++i) {
        if (DO0) {
            if (stash_row != nullptr) store_stream(reinterpret_cast<V*>(stash_row + int64_t(n0 + i) * hd + col), r0[i]);
            E el[VEC];
            __builtin_memcpy(el, &r0[i], VB);
#pragma unroll
            for (int e = 0; e < VEC; ++e) acc0[e] = __builtin_fmaf(x0[i], widen(el[e]), acc0[e]);
        }
        if (DO1) {
            E el[VEC];
            __builtin_memcpy(el, &r1[i], VB);
#pragma unroll
            for (int e = 0; e < VEC; ++e) acc1[e] = __builtin_fmaf(x1[i], widen(el[e]), acc1[e]);
        }
    }
}

template <typename E, int VB, bool TWO, int NB, typename IdxT, typename WT>
__global__ __launch_bounds__(kThreads) void sdm_gather_kernel(const GatherParams p) {
    using V = typename RawVec<VB>::T;
    constexpr int VEC = VB / int(sizeof(E));
    extern __shared__ __align__(16) char s_raw[];

    const int tid = threadIdx.x;
    const int tpb = kThreads / p.lpr;      // tokens per block
    const int ch = kStageEntries / tpb;    // entries per token staged at once
    const int lane = tid & (p.lpr - 1);
    const int g = tid / p.lpr;
    const int64_t t_first = int64_t(blockIdx.x) * tpb;
    const int64_t t = t_first + g;
    const int vi = int(blockIdx.y) * p.lpr + lane;
    const bool lane_on = t < p.tokens && vi < p.vpr;
    const int64_t col = int64_t(vi < p.vpr ? vi : 0) * VEC;

    // LDS: [tpb][ch] slots and weights per operand, then one live flag per token.
    IdxT* s_idx0 = reinterpret_cast<IdxT*>(s_raw);
    IdxT* s_idx1 = s_idx0 + tpb * ch;
    WT* s_w0 = reinterpret_cast<WT*>(s_idx1 + (TWO ? tpb * ch : 0));
    WT* s_w1 = s_w0 + tpb * ch;
    int* s_live = reinterpret_cast<int*>(s_w1 + (TWO ? tpb * ch : 0));

    bool live = false;
    if (t < p.tokens) {
        const int64_t chunk_no = t / p.chunk;
        const int64_t limit = p.chunk_valid != nullptr ? int64_t(p.chunk_valid[chunk_no]) : p.valid;
        live = (t - chunk_no * p.chunk) < limit;
    }
    if (lane == 0) s_live[g] = live ? 1 : 0;

    const E* bank = static_cast<const E*>(p.bank);
    E* stash_row = p.stash != nullptr && lane_on ? static_cast<E*>(p.stash) + t * p.width0 * p.hd : nullptr;
    const IdxT* idx0 = static_cast<const IdxT*>(p.idx0);
    const IdxT* idx1 = static_cast<const IdxT*>(p.idx1);
    const WT* w0 = static_cast<const WT*>(p.w0);
    const WT* w1 = static_cast<const WT*>(p.w1);

    float acc0[VEC], acc1[VEC];
#pragma unroll
    for (int e = 0; e < VEC; ++e) {
        acc0[e] = 0.0f;
        acc1[e] = 0.0f;
    }

    if (!live && stash_row != nullptr) {
        V zero;
        __builtin_memset(&zero, 0, VB);
        for (int n = 0; n < p.width0; ++n) store_stream(reinterpret_cast<V*>(stash_row + int64_t(n) * p.hd + col), zero);
    }

    const int wmax = TWO && p.width1 > p.width0 ? p.width1 : p.width0;
    for (int base = 0; base < wmax; base += ch) {
        // ---- stage entries [base, base + ch) of every live token of the block.
        __syncthreads();  // s_live written; the previous chunk's entries consumed
        for (int k = tid; k < tpb * ch; k += kThreads) {
            const int tt = k / ch, n = base + (k - tt * ch);
            const int64_t tok = t_first + tt;
            if (tok < p.tokens && s_live[tt]) {
                if (n < p.width0) {
                    s_idx0[k] = idx0[tok * p.width0 + n];
                    s_w0[k] = w0[tok * p.width0 + n];
                }
                if (TWO && n < p.width1) {
                    s_idx1[k] = idx1[tok * p.width1 + n];
                    s_w1[k] = w1[tok * p.width1 + n];
                }
            }
        }
        __syncthreads();
        if (!(live && lane_on)) continue;

        // ---- entries in ascending order: full batches of both operands, then of
        // each operand alone, then single entries.
        const int k_base = g * ch - base;  // LDS index of entry n is k_base + n
        const int end0 = min(p.width0, base + ch);
        const int end1 = TWO ? min(p.width1, base + ch) : base;
        int n = base;
        if (TWO)
            for (; n + NB <= min(end0, end1); n += NB)
                gather_batch<E, VB, NB, true, true>(bank, p.hd, col, n, k_base + n, s_idx0, s_w0, s_idx1, s_w1,
                                                    stash_row, acc0, acc1);
        int n_0 = n, n_1 = n;
        for (; n_0 + NB <= end0; n_0 += NB)
            gather_batch<E, VB, NB, true, false>(bank, p.hd, col, n_0, k_base + n_0, s_idx0, s_w0, s_idx1, s_w1,
                                                 stash_row, acc0, acc1);
        for (; n_0 < end0; ++n_0)
            gather_batch<E, VB, 1, true, false>(bank, p.hd, col, n_0, k_base + n_0, s_idx0, s_w0, s_idx1, s_w1,
                                                stash_row, acc0, acc1);
        if (TWO) {
            for (; n_1 + NB <= end1; n_1 += NB)
                gather_batch<E, VB, NB, false, true>(bank, p.hd, col, n_1, k_base + n_1, s_idx0, s_w0, s_idx1,
                                                     s_w1, stash_row, acc0, acc1);
            for (; n_1 < end1; ++n_1)
                gather_batch<E, VB, 1, false, true>(bank, p.hd, col, n_1, k_base + n_1, s_idx0, s_w0, s_idx1,
                                                    s_w1, stash_row, acc0, acc1);
        }
    }
    if (!lane_on) return;

    float* o0 = p.out0 + t * p.hd + col;
    float* o1 = TWO ? p.out1 + t * p.hd + col : nullptr;
    if (p.out_vec && VEC % 4 == 0) {
#pragma unroll
        for (int e = 0; e < VEC; e += 4) {
            store_stream(reinterpret_cast<float4*>(o0 + e), make_float4(acc0[e], acc0[e + 1], acc0[e + 2], acc0[e + 3]));
            if (TWO)
                store_stream(reinterpret_cast<float4*>(o1 + e), make_float4(acc1[e], acc1[e + 1], acc1[e + 2], acc1[e + 3]));
        }
    } else {
#pragma unroll
        for (int e = 0; e < VEC; ++e) {
            store_stream(o0 + e, acc0[e]);
            if (TWO) store_stream(o1 + e, acc1[e]);
        }
    }
}

template <typename E, int VB, bool TWO, typename IdxT, typename WT>
hipError_t launch_typed(const GatherParams& p, const GatherGeometry& geo, hipStream_t stream) {
    const int64_t blocks = (p.tokens + geo.tokens_per_block - 1) / geo.tokens_per_block;
    const dim3 grid(unsigned(blocks), unsigned(geo.slices));
    const dim3 block(kThreads);
    const size_t lds = size_t(kStageEntries) * (TWO ? 2 : 1) * (sizeof(IdxT) + sizeof(WT)) +
                       size_t(geo.tokens_per_block) * sizeof(int);
    hipLaunchKernelGGL((sdm_gather_kernel<E, VB, TWO, TWO ? 4 : 8, IdxT, WT>), grid, block, lds, stream, p);
    return hipGetLastError();
}

template <typename E, int VB, bool TWO>
hipError_t launch_ops(const GatherParams& p, const GatherGeometry& geo, hipStream_t stream) {
    if (p.idx64)
        return p.w_bf16 ? launch_typed<E, VB, TWO, int64_t, uint16_t>(p, geo, stream)
                        : launch_typed<E, VB, TWO, int64_t, float>(p, geo, stream);
    return p.w_bf16 ? launch_typed<E, VB, TWO, int32_t, uint16_t>(p, geo, stream)
                    : launch_typed<E, VB, TWO, int32_t, float>(p, geo, stream);
}

template <typename E, int VB>
hipError_t launch_vb(const GatherParams& p, const GatherGeometry& geo, bool two, hipStream_t stream) {
    return two ? launch_ops<E, VB, true>(p, geo, stream) : launch_ops<E, VB, false>(p, geo, stream);
}

int pow2_ceil(int64_t x) {
    int p = 1;
    while (p < x) p <<= 1;
    return p;
}

}  // namespace

GatherGeometry gather_geometry(int es, int64_t hd, uintptr_t bank_addr, uintptr_t stash_addr) {
    GatherGeometry g{};
    const int64_t row_bytes = hd * es;
    g.vb = es;
    for (int vb : {16, 8, 4}) {
        if (vb >= es && row_bytes % vb == 0 && bank_addr % vb == 0 && stash_addr % vb == 0) {
            g.vb = vb;
            break;
        }
    }
    g.vpr = int(row_bytes / g.vb);
    g.lpr = g.vpr >= 64 ? 64 : pow2_ceil(g.vpr);
    g.slices = (g.vpr + g.lpr - 1) / g.lpr;
    g.tokens_per_block = kThreads / g.lpr;
    g.threads = kThreads;
    return g;
}

hipError_t launch_gather(const GatherParams& p, const GatherGeometry& geo, bool bf16, bool two,
                         hipStream_t stream) {
    if (bf16) {
        switch (geo.vb) {
            case 16: return launch_vb<uint16_t, 16>(p, geo, two, stream);
            case 8: return launch_vb<uint16_t, 8>(p, geo, two, stream);
            case 4: return launch_vb<uint16_t, 4>(p, geo, two, stream);
            default: return launch_vb<uint16_t, 2>(p, geo, two, stream);
        }
    }
    switch (geo.vb) {
        case 16: return launch_vb<float, 16>(p, geo, two, stream);
        case 8: return launch_vb<float, 8>(p, geo, two, stream);
        default: return launch_vb<float, 4>(p, geo, two, stream);
    }
}

}  // namespace sdm
