// SDM decode step on gfx950: one workgroup per (stream, column slice).
//
// The step (page "sparse_delta_memory/decode.py", docstring of sdm_decode_step)
// gathers the W written rows of a stream, forms retrieved and delta_v per
// column, writes the W rows back decayed and updated, and after a workgroup
// barrier reads the R rows back as a weighted sum. Every quantity is
// per column, so column slices are independent and a workgroup owns all W and R
// rows of its stream within its slice: the barrier alone orders its writes
// before its reads (the same argument as the prior-art Triton kernel on that
// page, whose programs own 16-column blocks).
//
// Layout of a workgroup: RG row groups of LPR lanes. Lane l of row group j
// holds vector (slice * LPR + l) of rows w = j, j + RG, j + 2 RG, ... (at most
// 8 rows per phase), so every row is read with 16-byte (or narrower, for rows
// that are not a multiple of 16 bytes) loads spread over LPR lanes, all of a
// phase's rows are requested before any is used, and the rows stay in
// registers between the retrieval and the write-back. The per-group partial
// sums meet in LDS, where one thread per column adds them in group order.
//
// This is an HBM-bound gather/scatter (about 1 flop per byte), so it uses
// vector memory and VALU FMAs, not MFMA.

#include "sdm_kernels.h"

namespace sdm {

namespace {

constexpr int kRowsPerThread = 8;  // rows a lane holds per phase

// JN: rows a lane holds per phase (a power of two, ceil(max(W, R) / RG) rounded up).
template <typename E, int VB, int JN>
__global__ __launch_bounds__(1024) void sdm_decode_kernel(const DecodeParams p) {
    using V = typename RawVec<VB>::T;
    constexpr int VEC = VB / int(sizeof(E));

    __shared__ int64_t s_kslot[kMaxWidth];
    __shared__ int64_t s_qslot[kMaxWidth];
    __shared__ float s_kv[kMaxWidth];
    __shared__ float s_d[kMaxWidth];
    __shared__ float s_coef[kMaxWidth];
    __shared__ float s_qv[kMaxWidth];
    __shared__ float s_beta;
    extern __shared__ float s_dyn[];  // partial [rg][slice_cols], then delta_v [slice_cols]

    const int tid = threadIdx.x;
    const int nthr = blockDim.x;
    const int lane = tid & (p.lpr - 1);
    const int grp = tid / p.lpr;
    const int64_t s = blockIdx.x;
    const int slice_cols = p.lpr * VEC;
    const int vi = int(blockIdx.y) * p.lpr + lane;
    const bool active = vi < p.vpr;
    const int64_t col0 = int64_t(blockIdx.y) * slice_cols;
    float* partial = s_dyn;
    float* s_dv = s_dyn + p.rg * slice_cols;
    E* bank = static_cast<E*>(p.bank);

    // Slots, weights (rounded to the bank dtype), decays and coefficients of this stream.
    for (int i = tid; i < p.W; i += nthr) {
        const int64_t at = s * p.W + i;
        const float kv = to_bank<E>(load_value(p.k_val, at, p.val_bf16));
        const float d = float(exp(double(p.g[s * p.G + (p.G == 1 ? 0 : i)])));
        s_kslot[i] = load_slot(p.k_idx, at, p.k64);
        s_kv[i] = kv;
        s_d[i] = d;
        s_coef[i] = kv * d;
    }
    for (int i = tid; i < p.R; i += nthr) {
        const int64_t at = s * p.R + i;
        s_qslot[i] = load_slot(p.q_idx, at, p.q64);
        s_qv[i] = to_bank<E>(load_value(p.q_val, at, p.val_bf16));
    }
    if (tid == 0) s_beta = p.beta[s];
    __syncthreads();

    // ---- write phase: gather the W rows, every load issued before any use.
    // The loads are unconditional: a lane past the row end or a row past W reads
    // a clamped address (a line the wavefront fetches anyway) and ignores it.
    // Guarded loads would let the compiler move each row's unpacking next to its
    // load and wait for it there, one row at a time.
    const int64_t vcol = int64_t(active ? vi : p.vpr - 1) * VEC;
    V raw[JN];
#pragma unroll
    for (int j = 0; j < JN; ++j) {
        const int w = grp + j * p.rg;
        raw[j] = *reinterpret_cast<const V*>(bank + s_kslot[w < p.W ? w : p.W - 1] * p.hd + vcol);
    }
    float acc[VEC];
#pragma unroll
    for (int e = 0; e < VEC; ++e) acc[e] = 0.0f;
#pragma unroll
    for (int j = 0; j < JN; ++j) {
        const int w = grp + j * p.rg;
        if (active && w < p.W) {
            E el[VEC];
            __builtin_memcpy(el, &raw[j], VB);
            const float c = s_coef[w];
#pragma unroll
            for (int e = 0; e < VEC; ++e) acc[e] = __builtin_fmaf(c, widen(el[e]), acc[e]);
        }
    }
#pragma unroll
    for (int e = 0; e < VEC; ++e) partial[grp * slice_cols + lane * VEC + e] = acc[e];
    __syncthreads();

    // retrieved (group partials in group order) and delta_v, one thread per column.
    for (int col = tid; col < slice_cols; col += nthr) {
        const int64_t c = col0 + col;
        if (c < p.hd) {
            float total = 0.0f;
            for (int j = 0; j < p.rg; ++j) total += partial[j * slice_cols + col];
            const float vc = to_bank<E>(load_value(p.v, s * p.hd + c, p.val_bf16));
            s_dv[col] = s_beta * (vc - total);
        }
    }
    __syncthreads();

    // Decay-and-write of the rows this lane holds. Write slots are distinct within
    // a stream, so plain stores suffice.
#pragma unroll
    for (int j = 0; j < JN; ++j) {
        const int w = grp + j * p.rg;
        if (active && w < p.W) {
            E el[VEC], out[VEC];
            __builtin_memcpy(el, &raw[j], VB);
            const float kv = s_kv[w], d = s_d[w];
#pragma unroll
            for (int e = 0; e < VEC; ++e) {
                const float decayed = widen(el[e]) * d;
                out[e] = narrow<E>(__builtin_fmaf(kv, s_dv[lane * VEC + e], decayed));
            }
            V o;
            __builtin_memcpy(&o, out, VB);
            *reinterpret_cast<V*>(bank + s_kslot[w] * p.hd + int64_t(vi) * VEC) = o;
        }
    }

    // Ordering point: the workgroup's stores above are visible to its loads below
    // (workgroup-scope release/acquire around the barrier). No other workgroup
    // touches these columns of this stream's slots.
    __syncthreads();

    // ---- read phase: gather the R rows as stored, weighted sum in group order.
#pragma unroll
    for (int j = 0; j < JN; ++j) {
        const int r = grp + j * p.rg;
        raw[j] = *reinterpret_cast<const V*>(bank + s_qslot[r < p.R ? r : p.R - 1] * p.hd + vcol);
    }
#pragma unroll
    for (int e = 0; e < VEC; ++e) acc[e] = 0.0f;
#pragma unroll
    for (int j = 0; j < JN; ++j) {
        const int r = grp + j * p.rg;
        if (active && r < p.R) {
            E el[VEC];
            __builtin_memcpy(el, &raw[j], VB);
            const float q = s_qv[r];
#pragma unroll
            for (int e = 0; e < VEC; ++e) acc[e] = __builtin_fmaf(q, widen(el[e]), acc[e]);
        }
    }
#pragma unroll
    for (int e = 0; e < VEC; ++e) partial[grp * slice_cols + lane * VEC + e] = acc[e];
    __syncthreads();
    E* readings = static_cast<E*>(p.readings);
    for (int col = tid; col < slice_cols; col += nthr) {
        const int64_t c = col0 + col;
        if (c < p.hd) {
            float total = 0.0f;
            for (int j = 0; j < p.rg; ++j) total += partial[j * slice_cols + col];
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
    const int need = (wmax + kRowsPerThread - 1) / kRowsPerThread;
    g.rg = pow2_ceil(need);
    if (g.rg > 32) g.rg = 32;
    g.jn = pow2_ceil((wmax + g.rg - 1) / g.rg);
    g.threads = g.lpr * g.rg;
    const int slice_cols = g.lpr * (g.vb / es);
    g.lds = size_t(g.rg + 1) * size_t(slice_cols) * sizeof(float);
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
