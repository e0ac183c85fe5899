// SDM decode step on gfx950: one workgroup per (stream, column slice).
//
// The step (page "sparse_delta_memory/decode.py", docstring of sdm_decode_step)
// gathers the W written rows of a stream, forms retrieved and delta_v per
// column, writes the W rows back decayed and updated, and reads the R rows back
// as a weighted sum after the write. Every quantity is per column, so column
// slices are independent and a workgroup owns all W and R rows of its stream
// within its slice: only its own stores can change what its reads see (the
// same argument as the prior-art Triton kernel on that page, whose programs own
// 16-column blocks).
//
// Layout of a workgroup: RG row groups of LPR lanes. Lane l of row group j
// holds vector (slice * LPR + l) of rows j, j + RG, j + 2 RG, ... (JN <= 8 rows
// per phase), so every row is read with 16-byte loads (narrower when a row is
// not a multiple of 16 bytes) spread over LPR lanes, and the rows stay in
// registers between the retrieval and the write-back.
//
// Phases: the W rows are requested together, used for the retrieval and
// written back; then, after a workgroup barrier that orders the write-back
// before any read, the R rows are requested together into the same registers
// (a lane holds one phase's rows at a time, which keeps occupancy high) and
// summed. (Comparing the slot lists to skip that barrier where no read slot is
// written cost more than it saved.)
//
// The per-group partial sums meet in LDS, where one thread per column adds them
// in group order. This is an HBM-bound gather/scatter (about 1 flop per byte):
// vector memory and VALU FMAs, no MFMA.

#include "sdm_kernels.h"

namespace sdm {

namespace {

// Rows a lane holds per phase at most: fixes RG, and with it the summation order.
constexpr int kRowsPerLane = 4;

struct DecodeLds {
    int64_t* kslot;  // [W]
    int64_t* qslot;  // [R]
    float* kv;       // [W] k_val rounded to the bank dtype
    float* d;        // [W] exp(g)
    float* coef;     // [W] kv * d
    float* qv;       // [R] q_val rounded to the bank dtype
    float* v;        // [slice_cols] v rounded to the bank dtype
    float* partial;  // [RG][slice_cols]
    float* dv;       // [slice_cols]
    float* beta;     // [1]
};

__device__ __forceinline__ DecodeLds carve(char* base, int W, int R, int rg, int slice_cols) {
    DecodeLds l;
    l.kslot = reinterpret_cast<int64_t*>(base);
    l.qslot = l.kslot + W;
    float* f = reinterpret_cast<float*>(l.qslot + R);
    l.kv = f;
    l.d = l.kv + W;
    l.coef = l.d + W;
    l.qv = l.coef + W;
    l.v = l.qv + R;
    l.partial = l.v + slice_cols;
    l.dv = l.partial + rg * slice_cols;
    l.beta = l.dv + slice_cols;
    return l;
}

// Stage stream s's slots, rounded weights, decays, v (this slice) and beta in LDS.
template <typename E, typename KI, typename QI, typename VT>
__device__ __forceinline__ void stage(const DecodeParams& p, const DecodeLds& L, int64_t s, int64_t col0,
                                      int slice_cols) {
    const int tid = threadIdx.x, nthr = blockDim.x;
    const KI* k_idx = static_cast<const KI*>(p.k_idx);
    const QI* q_idx = static_cast<const QI*>(p.q_idx);
    const VT* k_val = static_cast<const VT*>(p.k_val);
    const VT* q_val = static_cast<const VT*>(p.q_val);
    const VT* v = static_cast<const VT*>(p.v);
    for (int i = tid; i < p.W; i += nthr) {
        const int64_t at = s * p.W + i;
        const float kv = to_bank<E>(value_of<VT>(k_val[at]));
        const float d = float(exp(double(p.g[s * p.G + (p.G == 1 ? 0 : i)])));
        L.kslot[i] = int64_t(k_idx[at]);
        L.kv[i] = kv;
        L.d[i] = d;
        L.coef[i] = kv * d;
    }
    for (int i = tid; i < p.R; i += nthr) {
        const int64_t at = s * p.R + i;
        L.qslot[i] = int64_t(q_idx[at]);
        L.qv[i] = to_bank<E>(value_of<VT>(q_val[at]));
    }
    for (int col = tid; col < slice_cols; col += nthr) {
        const int64_t c = col0 + col;
        L.v[col] = c < p.hd ? to_bank<E>(value_of<VT>(v[s * p.hd + c])) : 0.0f;
    }
    if (tid == 0) L.beta[0] = p.beta[s];
}

// JN: rows a lane holds per phase (a power of two >= ceil(max(W, R) / RG)).
template <typename E, int VB, int JN>
__global__ __launch_bounds__(1024) void sdm_decode_kernel(const DecodeParams p) {
    using V = typename RawVec<VB>::T;
    constexpr int VEC = VB / int(sizeof(E));
    extern __shared__ __align__(16) char s_raw[];

    const int tid = threadIdx.x;
    const int nthr = blockDim.x;
    const int lane = tid & (p.lpr - 1);
    const int grp = tid / p.lpr;
    const int64_t s = blockIdx.x;
    const int slice_cols = p.lpr * VEC;
    const int vi = int(blockIdx.y) * p.lpr + lane;
    const bool active = vi < p.vpr;
    const int64_t col0 = int64_t(blockIdx.y) * slice_cols;
    const DecodeLds L = carve(s_raw, p.W, p.R, p.rg, slice_cols);
    E* bank = static_cast<E*>(p.bank);

    // ---- the stream's slots, weights (rounded to the bank dtype), decays, v.
    // One branch-free copy per (index types, value type): all of a thread's
    // loads are issued together.
    switch (p.k64 | (p.q64 << 1) | (p.val_bf16 << 2)) {
        case 0: stage<E, int32_t, int32_t, float>(p, L, s, col0, slice_cols); break;
        case 1: stage<E, int64_t, int32_t, float>(p, L, s, col0, slice_cols); break;
        case 2: stage<E, int32_t, int64_t, float>(p, L, s, col0, slice_cols); break;
        case 3: stage<E, int64_t, int64_t, float>(p, L, s, col0, slice_cols); break;
        case 4: stage<E, int32_t, int32_t, uint16_t>(p, L, s, col0, slice_cols); break;
        case 5: stage<E, int64_t, int32_t, uint16_t>(p, L, s, col0, slice_cols); break;
        case 6: stage<E, int32_t, int64_t, uint16_t>(p, L, s, col0, slice_cols); break;
        default: stage<E, int64_t, int64_t, uint16_t>(p, L, s, col0, slice_cols); break;
    }
    __syncthreads();

    // ---- request every W row before using any. The loads are unconditional: a
    // lane past the row end or a row past W reads a clamped address (a line the
    // wavefront fetches anyway) and ignores it. Guarded loads would let the
    // compiler wait for each row next to its load.
    const int64_t vcol = int64_t(active ? vi : p.vpr - 1) * VEC;
    V row[JN];
#pragma unroll
    for (int j = 0; j < JN; ++j) {
        const int w = grp + j * p.rg;
        row[j] = *reinterpret_cast<const V*>(bank + L.kslot[w < p.W ? w : p.W - 1] * p.hd + vcol);
    }

    // ---- retrieval partials, in ascending w within the row group.
    float acc[VEC];
#pragma unroll
    for (int e = 0; e < VEC; ++e) acc[e] = 0.0f;
#pragma unroll
    for (int j = 0; j < JN; ++j) {
        const int w = grp + j * p.rg;
        if (active && w < p.W) {
            E el[VEC];
            __builtin_memcpy(el, &row[j], VB);
            const float c = L.coef[w];
#pragma unroll
            for (int e = 0; e < VEC; ++e) acc[e] = __builtin_fmaf(c, widen(el[e]), acc[e]);
        }
    }
#pragma unroll
    for (int e = 0; e < VEC; ++e) L.partial[grp * slice_cols + lane * VEC + e] = acc[e];
    __syncthreads();

    // retrieved (group partials in group order) and delta_v, one thread per column.
    for (int col = tid; col < slice_cols; col += nthr) {
        if (col0 + col < p.hd) {
            float total = 0.0f;
            for (int j = 0; j < p.rg; ++j) total += L.partial[j * slice_cols + col];
            L.dv[col] = L.beta[0] * (L.v[col] - total);
        }
    }
    __syncthreads();

    // ---- decay-and-write of the rows this lane holds. Write slots are distinct
    // within a stream, so plain stores suffice. opaque() hides the raw bits from
    // the optimiser, so the rows are widened again here instead of being kept
    // widened (twice the registers for bfloat16) across the two barriers above.
#pragma unroll
    for (int j = 0; j < JN; ++j) opaque(row[j]);
#pragma unroll
    for (int j = 0; j < JN; ++j) {
        const int w = grp + j * p.rg;
        if (active && w < p.W) {
            E el[VEC], out[VEC];
            __builtin_memcpy(el, &row[j], VB);
            const float kv = L.kv[w], d = L.d[w];
#pragma unroll
            for (int e = 0; e < VEC; ++e) {
                const float decayed = widen(el[e]) * d;
                out[e] = narrow<E>(__builtin_fmaf(kv, L.dv[lane * VEC + e], decayed));
            }
            V o;
            __builtin_memcpy(&o, out, VB);
            *reinterpret_cast<V*>(bank + L.kslot[w] * p.hd + int64_t(vi) * VEC) = o;
        }
    }

    // ---- ordering point: the barrier (workgroup-scope release/acquire) makes
    // the stores above visible to the loads below, for read slots that are also
    // write slots. No other workgroup touches these columns of these slots.
    __syncthreads();
#pragma unroll
    for (int j = 0; j < JN; ++j) {
        const int r = grp + j * p.rg;
        row[j] = *reinterpret_cast<const V*>(bank + L.qslot[r < p.R ? r : p.R - 1] * p.hd + vcol);
    }

    // ---- readings: weighted sum of the R rows as stored, in group order.
#pragma unroll
    for (int e = 0; e < VEC; ++e) acc[e] = 0.0f;
#pragma unroll
    for (int j = 0; j < JN; ++j) {
        const int r = grp + j * p.rg;
        if (active && r < p.R) {
            E el[VEC];
            __builtin_memcpy(el, &row[j], VB);
            const float q = L.qv[r];
#pragma unroll
            for (int e = 0; e < VEC; ++e) acc[e] = __builtin_fmaf(q, widen(el[e]), acc[e]);
        }
    }
    // The partials of the write phase were last read before the barrier that
    // preceded the write-back, so they can be overwritten now.
#pragma unroll
    for (int e = 0; e < VEC; ++e) L.partial[grp * slice_cols + lane * VEC + e] = acc[e];
    __syncthreads();
    E* readings = static_cast<E*>(p.readings);
    for (int col = tid; col < slice_cols; col += nthr) {
        const int64_t c = col0 + col;
        if (c < p.hd) {
            float total = 0.0f;
            for (int j = 0; j < p.rg; ++j) total += L.partial[j * slice_cols + col];
            readings[s * p.hd + c] = narrow<E>(total);
        }
    }
}

template <typename E, int VB>
hipError_t launch_vb(const DecodeParams& p, const DecodeGeometry& geo, int64_t streams, hipStream_t stream) {
    const dim3 grid(unsigned(streams), unsigned(geo.slices));
    const dim3 block(unsigned(geo.threads));
    switch (geo.jn) {
        case 1: hipLaunchKernelGGL((sdm_decode_kernel<E, VB, 1>), grid, block, geo.lds, stream, p); break;
        case 2: hipLaunchKernelGGL((sdm_decode_kernel<E, VB, 2>), grid, block, geo.lds, stream, p); break;
        case 4: hipLaunchKernelGGL((sdm_decode_kernel<E, VB, 4>), grid, block, geo.lds, stream, p); break;
        default: hipLaunchKernelGGL((sdm_decode_kernel<E, VB, 8>), grid, block, geo.lds, stream, p); break;
    }
    return hipGetLastError();
}

int pow2_ceil(int64_t x) {
    int p = 1;
    while (p < x) p <<= 1;
    return p;
}

}  // namespace

DecodeGeometry decode_geometry(int es, int64_t hd, int W, int R, uintptr_t bank_addr) {
    DecodeGeometry g{};
    const int64_t row_bytes = hd * es;
    g.vb = es;
    for (int vb : {16, 8, 4}) {
        if (vb >= es && row_bytes % vb == 0 && bank_addr % vb == 0) {
            g.vb = vb;
            break;
        }
    }
    g.vpr = int(row_bytes / g.vb);
    g.lpr = g.vpr >= 32 ? 32 : pow2_ceil(g.vpr);
    g.slices = (g.vpr + g.lpr - 1) / g.lpr;
    const int wmax = W > R ? W : R;
    g.rg = pow2_ceil((wmax + kRowsPerLane - 1) / kRowsPerLane);
    if (g.rg > 32) g.rg = 32;
    g.jn = pow2_ceil((wmax + g.rg - 1) / g.rg);
    g.threads = g.lpr * g.rg;
    const int slice_cols = g.lpr * (g.vb / es);
    // kslot, qslot (8 B each); kv, d, coef, qv (4 B); v, partial, dv; beta
    g.lds = size_t(8) * (W + R) + size_t(4) * (3 * W + R) +
            size_t(4) * (size_t(slice_cols) * (g.rg + 2) + 1);
    g.lds = (g.lds + 15) & ~size_t(15);
    return g;
}

hipError_t launch_decode(const DecodeParams& p, const DecodeGeometry& geo, int64_t streams, bool bf16,
                         hipStream_t stream) {
    if (bf16) {
        switch (geo.vb) {
            case 16: return launch_vb<uint16_t, 16>(p, geo, streams, stream);
            case 8: return launch_vb<uint16_t, 8>(p, geo, streams, stream);
            case 4: return launch_vb<uint16_t, 4>(p, geo, streams, stream);
            default: return launch_vb<uint16_t, 2>(p, geo, streams, stream);
        }
    }
    switch (geo.vb) {
        case 16: return launch_vb<float, 16>(p, geo, streams, stream);
        case 8: return launch_vb<float, 8>(p, geo, streams, stream);
        default: return launch_vb<float, 4>(p, geo, streams, stream);
    }
}

}  // namespace sdm
