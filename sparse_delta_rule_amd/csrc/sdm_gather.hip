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
// no cross-lane reduction, no LDS and no barrier, and the result depends on the
// inputs alone. Entries are taken NB at a time per operand, with all of a
// batch's row loads issued before the first is used, so NB (one operand) or
// 2 * NB (two operands) random rows per lane are in flight; the HBM latency is
// hidden by that and by the many tokens resident per CU.

#include "sdm_kernels.h"

namespace sdm {

namespace {

constexpr int kThreads = 256;

template <typename E, int VB, bool TWO, int NB>
__global__ __launch_bounds__(kThreads) void sdm_gather_kernel(const GatherParams p) {
    using V = typename RawVec<VB>::T;
    constexpr int VEC = VB / int(sizeof(E));
    const int tid = threadIdx.x;
    const int lane = tid & (p.lpr - 1);
    const int64_t t = int64_t(blockIdx.x) * (kThreads / p.lpr) + tid / p.lpr;
    const int vi = int(blockIdx.y) * p.lpr + lane;
    if (t >= p.tokens || vi >= p.vpr) return;
    const int64_t col = int64_t(vi) * VEC;
    const int64_t chunk_no = t / p.chunk;
    const int64_t limit = p.chunk_valid != nullptr ? int64_t(p.chunk_valid[chunk_no]) : p.valid;
    const bool live = (t - chunk_no * p.chunk) < limit;
    const E* bank = static_cast<const E*>(p.bank);
    E* stash = static_cast<E*>(p.stash);

    float acc0[VEC], acc1[VEC];
#pragma unroll
    for (int e = 0; e < VEC; ++e) {
        acc0[e] = 0.0f;
        acc1[e] = 0.0f;
    }

    if (!live) {
        if (stash != nullptr) {
            V zero;
            __builtin_memset(&zero, 0, VB);
            for (int n = 0; n < p.width0; ++n)
                *reinterpret_cast<V*>(stash + (t * p.width0 + n) * p.hd + col) = zero;
        }
    } else {
        const int wmax = TWO && p.width1 > p.width0 ? p.width1 : p.width0;
        for (int n0 = 0; n0 < wmax; n0 += NB) {
            // Every load is unconditional: an entry past an operand's width re-reads
            // that operand's last entry and is ignored. Guarded loads would let the
            // compiler wait for each row next to its load.
            V r0[NB], r1[NB];
            float w0[NB], w1[NB];
#pragma unroll
            for (int i = 0; i < NB; ++i) {
                const int n = n0 + i;
                const int64_t at = t * p.width0 + (n < p.width0 ? n : p.width0 - 1);
                r0[i] = *reinterpret_cast<const V*>(bank + load_slot(p.idx0, at, p.idx64) * p.hd + col);
                w0[i] = load_value(p.w0, at, p.w_bf16);
                if (TWO) {
                    const int64_t at1 = t * p.width1 + (n < p.width1 ? n : p.width1 - 1);
                    r1[i] = *reinterpret_cast<const V*>(bank + load_slot(p.idx1, at1, p.idx64) * p.hd + col);
                    w1[i] = load_value(p.w1, at1, p.w_bf16);
                }
            }
#pragma unroll
            for (int i = 0; i < NB; ++i) {
                const int n = n0 + i;
                if (n < p.width0) {
                    if (stash != nullptr) *reinterpret_cast<V*>(stash + (t * p.width0 + n) * p.hd + col) = r0[i];
                    E el[VEC];
                    __builtin_memcpy(el, &r0[i], VB);
#pragma unroll
                    for (int e = 0; e < VEC; ++e) acc0[e] = __builtin_fmaf(w0[i], widen(el[e]), acc0[e]);
                }
                if (TWO && n < p.width1) {
                    E el[VEC];
                    __builtin_memcpy(el, &r1[i], VB);
#pragma unroll
                    for (int e = 0; e < VEC; ++e) acc1[e] = __builtin_fmaf(w1[i], widen(el[e]), acc1[e]);
                }
            }
        }
    }

    float* o0 = p.out0 + t * p.hd + col;
    float* o1 = TWO ? p.out1 + t * p.hd + col : nullptr;
    if (p.out_vec && VEC % 4 == 0) {
#pragma unroll
        for (int e = 0; e < VEC; e += 4) {
            *reinterpret_cast<float4*>(o0 + e) = make_float4(acc0[e], acc0[e + 1], acc0[e + 2], acc0[e + 3]);
            if (TWO) *reinterpret_cast<float4*>(o1 + e) = make_float4(acc1[e], acc1[e + 1], acc1[e + 2], acc1[e + 3]);
        }
    } else {
#pragma unroll
        for (int e = 0; e < VEC; ++e) {
            o0[e] = acc0[e];
            if (TWO) o1[e] = acc1[e];
        }
    }
}

template <typename E, int VB>
hipError_t launch_vb(const GatherParams& p, const GatherGeometry& geo, bool two, hipStream_t stream) {
    const int64_t blocks = (p.tokens + geo.tokens_per_block - 1) / geo.tokens_per_block;
    const dim3 grid(unsigned(blocks), unsigned(geo.slices));
    const dim3 block(kThreads);
    if (two)
        hipLaunchKernelGGL((sdm_gather_kernel<E, VB, true, 4>), grid, block, 0, stream, p);
    else
        hipLaunchKernelGGL((sdm_gather_kernel<E, VB, false, 8>), grid, block, 0, stream, p);
    return hipGetLastError();
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
