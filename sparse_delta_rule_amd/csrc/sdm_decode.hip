// SDM decode on gfx950: one workgroup per (stream, column slice).
//
// A decode step (page "sparse_delta_memory/decode.py", docstring of
// sdm_decode_step) gathers the W written rows of a stream, forms retrieved and
// delta_v per column, writes the W rows back decayed and updated, and reads the
// R rows back as a weighted sum after the write. Every quantity is per column,
// so column slices are independent and a workgroup owns all W and R rows of its
// stream within its slice: only its own stores can change what its reads see
// (the same argument as the prior-art Triton kernel on that page, whose
// programs own 16-column blocks).
//
// Layout of a workgroup: RG row groups of LPR lanes. Lane l of row group j
// holds vector (slice * LPR + l) of rows j, j + RG, j + 2 RG, ... (JN <= 8 rows
// per phase), so every row is read with 16-byte loads (narrower when a row is
// not a multiple of 16 bytes) spread over LPR lanes, and the W rows stay in
// registers between the retrieval and the write-back. The per-group partial
// sums meet in LDS, where one thread per column adds them in group order.
//
// sdm_decode_kernel (one step): stage the stream's slots and weights in LDS;
// request all W rows; retrieval, delta_v, write-back; a workgroup barrier
// (workgroup-scope release/acquire) orders the write-back before the reads;
// request all R rows into the same registers (one phase's rows at a time keeps
// occupancy high); readings.
//
// sdm_decode_steps_kernel and sdm_decode_steps_wide_kernel (T steps of one
// stream in one launch): the same step in a loop, software-pipelined so each
// step costs one wait for rows instead of two plus a launch: right after the
// barrier that publishes step t's writes, the R rows of step t and the W rows of
// step t + 1 are requested together (both may be rows step t wrote, which that
// barrier orders), with later steps' slots and weights. The compact loop, for
// grids that keep many waves on each SIMD, sums step t + 1's rows in the next
// iteration (fewer live registers) and takes five barriers per step; the wide
// loop, for grids that leave at most two waves on each SIMD, forms both sums in
// one pass, stages metadata two steps ahead and takes three barriers per step.
// Both give the same results, bit for bit, as T single steps.
//
// This is an HBM-bound gather/scatter (about 1 flop per byte): vector memory
// and VALU FMAs, no MFMA.

#include "sdm_kernels.h"

namespace sdm {

namespace {

// Rows a lane holds per phase at most: fixes RG, and with it the summation order.
constexpr int kRowsPerLane = 4;
// One step's staged metadata in LDS.
struct Stage {
    int64_t* kslot;  // [W]
    int64_t* qslot;  // [R]
    float* kv;       // [W] k_val rounded to the bank dtype
    float* d;        // [W] exp(g)
    float* coef;     // [W] kv * d
    float* qv;       // [R] q_val rounded to the bank dtype
    float* v;        // [slice_cols] v rounded to the bank dtype (0 past head_dim)
    float* beta;     // [1]
};

__device__ __host__ __forceinline__ size_t stage_bytes(int W, int R, int slice_cols) {
    const size_t b = size_t(8) * (W + R) + size_t(4) * (3 * W + R + slice_cols + 1);
    return (b + 15) & ~size_t(15);
}

__device__ __forceinline__ Stage carve_stage(char* base, int W, int R, int slice_cols) {
    Stage st;
    st.kslot = reinterpret_cast<int64_t*>(base);
    st.qslot = st.kslot + W;
    st.kv = reinterpret_cast<float*>(st.qslot + R);
    st.d = st.kv + W;
    st.coef = st.d + W;
    st.qv = st.coef + W;
    st.v = st.qv + R;
    st.beta = st.v + slice_cols;
    return st;
}

// A step's metadata as fetched ahead by one thread, into registers: items
// i = tid + m * threads, MK of W and R and MV of the slice's v. Every load is
// unconditional (indices clamped to the last item), so no load sits in a
// guarded block where the compiler would wait for it.
template <int MK, int MV>
struct Meta {
    int64_t ks[MK], qs[MK];
    float kraw[MK], graw[MK], qraw[MK], vraw[MV];
    float beta;
};

// VBETA: read beta with vector loads, which issue with the others (a load from an
// address that is the same for the whole workgroup otherwise becomes a scalar
// load, which the compiler may schedule late).
template <int MK, int MV, bool VBETA = false>
__device__ __forceinline__ void meta_load(const DecodeParams& p, int t, int64_t s, int64_t col0, Meta<MK, MV>& m) {
    const int tid = threadIdx.x, nthr = blockDim.x;
    const int64_t row = int64_t(t) * p.streams + s;
#pragma unroll
    for (int k = 0; k < MK; ++k) {
        const int i = min(tid + k * nthr, p.W - 1);
        m.ks[k] = slot_at(p.k_idx, row * p.W + i, p.k_bytes);
        m.kraw[k] = value_at(p.k_val, row * p.W + i, p.val_bytes);
        m.graw[k] = p.g[row * p.G + (p.G == 1 ? 0 : i)];
        const int r = min(tid + k * nthr, p.R - 1);
        m.qs[k] = slot_at(p.q_idx, row * p.R + r, p.q_bytes);
        m.qraw[k] = value_at(p.q_val, row * p.R + r, p.val_bytes);
    }
#pragma unroll
    for (int k = 0; k < MV; ++k) {
        const int64_t c = min(col0 + tid + k * nthr, p.hd - 1);
        m.vraw[k] = value_at(p.v, row * p.hd + c, p.val_bytes);
    }
    m.beta = VBETA ? value_at(p.beta, row, 4) : p.beta[row];
}

// Round fetched metadata to the bank dtype, form decays and coefficients, and
// store it in a Stage.
template <typename E, int MK, int MV>
__device__ __forceinline__ void meta_store(const DecodeParams& p, const Meta<MK, MV>& m, const Stage& st,
                                           int64_t col0, int slice_cols) {
    const int tid = threadIdx.x, nthr = blockDim.x;
#pragma unroll
    for (int k = 0; k < MK; ++k) {
        const int i = tid + k * nthr;
        if (i < p.W) {
            const float kv = to_bank<E>(m.kraw[k]);
            const float d = float(exp(double(m.graw[k])));
            st.kslot[i] = m.ks[k];
            st.kv[i] = kv;
            st.d[i] = d;
            st.coef[i] = kv * d;
        }
        if (i < p.R) {
            st.qslot[i] = m.qs[k];
            st.qv[i] = to_bank<E>(m.qraw[k]);
        }
    }
#pragma unroll
    for (int k = 0; k < MV; ++k) {
        const int col = tid + k * nthr;
        if (col < slice_cols) st.v[col] = col0 + col < p.hd ? to_bank<E>(m.vraw[k]) : 0.0f;
    }
    if (tid == 0) st.beta[0] = m.beta;
}

// Stage stream s's metadata of step t now: every load issued at once, then
// rounded and stored. The empty asm statement with a memory clobber keeps the
// loads above it, so none is moved down next to its (guarded) store and waited
// for there: the stage costs one memory round trip, not one per guarded store.
template <typename E, int MK, int MV>
__device__ __forceinline__ void stage_now(const DecodeParams& p, int t, int64_t s, const Stage& st, int64_t col0,
                                          int slice_cols) {
    Meta<MK, MV> m;
    meta_load<MK, MV, true>(p, t, s, col0, m);
    asm volatile("" ::: "memory");
    meta_store<E, MK, MV>(p, m, st, col0, slice_cols);
}

// Lane geometry shared by the phases.
struct Lane {
    int grp, lane, vi, slice_cols;
    bool active;   // the lane's vector lies inside the row
    int64_t vcol;  // element offset of the lane's vector (clamped for inactive lanes)
    int64_t col0;  // first column of the slice
};

// Request rows slots[j * RG + grp] (j < JN) of the bank, all before any is used.
// Rows past n re-read row n - 1 and are ignored.
template <typename E, int VB, int JN>
__device__ __forceinline__ void load_rows(typename RawVec<VB>::T (&row)[JN], const E* bank, const int64_t* slots,
                                          int n, int rg, int64_t hd, const Lane& ln) {
    using V = typename RawVec<VB>::T;
#pragma unroll
    for (int j = 0; j < JN; ++j) {
        const int w = ln.grp + j * rg;
        row[j] = *reinterpret_cast<const V*>(bank + slots[w < n ? w : n - 1] * hd + ln.vcol);
    }
}

// This lane's partial of sum_w weight[w] * row_w over its rows, ascending, into
// partial[grp][lane's columns]. Every row is used unconditionally and a select
// keeps or drops its term (a row used only inside a branch would have its load
// moved into that branch and waited for there); a dropped term cannot reach the
// sum, whatever its value.
template <typename E, int VB, int JN>
__device__ __forceinline__ void row_partials(const typename RawVec<VB>::T (&row)[JN], const float* weight, int n,
                                             int rg, const Lane& ln, float* partial) {
    constexpr int VEC = VB / int(sizeof(E));
    float acc[VEC];
#pragma unroll
    for (int e = 0; e < VEC; ++e) acc[e] = 0.0f;
#pragma unroll
    for (int j = 0; j < JN; ++j) {
        const int w = ln.grp + j * rg;
        const bool use = ln.active && w < n;
        E el[VEC];
        __builtin_memcpy(el, &row[j], VB);
        const float c = weight[w < n ? w : n - 1];
#pragma unroll
        for (int e = 0; e < VEC; ++e) {
            const float term = __builtin_fmaf(c, widen(el[e]), acc[e]);
            acc[e] = use ? term : acc[e];
        }
    }
#pragma unroll
    for (int e = 0; e < VEC; ++e) partial[ln.grp * ln.slice_cols + ln.lane * VEC + e] = acc[e];
}

// Column col's total over the row groups, in group order from +0. A chunk's LDS
// reads are all issued before its first add, so the reads do not wait for one
// another; the adds stay in group order.
__device__ __forceinline__ float column_total(const float* partial, int rg, int slice_cols, int col) {
    float total = 0.0f;
    int j = 0;
    for (; j + 8 <= rg; j += 8) {
        float x[8];
#pragma unroll
        for (int k = 0; k < 8; ++k) x[k] = partial[(j + k) * slice_cols + col];
#pragma unroll
        for (int k = 0; k < 8; ++k) total += x[k];
    }
    if (j + 4 <= rg) {
        float x[4];
#pragma unroll
        for (int k = 0; k < 4; ++k) x[k] = partial[(j + k) * slice_cols + col];
#pragma unroll
        for (int k = 0; k < 4; ++k) total += x[k];
        j += 4;
    }
    for (; j < rg; ++j) total += partial[j * slice_cols + col];
    return total;
}

// delta_v = beta (v - retrieved) per column of the slice.
__device__ __forceinline__ void form_delta(const DecodeParams& p, const Stage& st, const float* partial, float* dv,
                                          const Lane& ln) {
    for (int col = threadIdx.x; col < ln.slice_cols; col += blockDim.x)
        if (ln.col0 + col < p.hd) dv[col] = st.beta[0] * (st.v[col] - column_total(partial, p.rg, ln.slice_cols, col));
}

// Slot, k_val and decay of the W rows this lane holds (row w = grp + j RG; rows
// past W repeat row W - 1 and are never written), read out of a Stage into
// registers ahead of time (the wide loop does this while its row loads are in
// flight).
template <int JN>
struct Held {
    int64_t slot[JN];
    float kv[JN], d[JN];
    __device__ __forceinline__ int64_t slot_of(int j, int) const { return slot[j]; }
    __device__ __forceinline__ float kv_of(int j, int) const { return kv[j]; }
    __device__ __forceinline__ float d_of(int j, int) const { return d[j]; }
};

// The same three values read from the Stage in LDS at the point of use (fewer
// live registers, for the kernels that run at high occupancy).
struct Staged {
    const Stage* st;
    __device__ __forceinline__ int64_t slot_of(int, int w) const { return st->kslot[w]; }
    __device__ __forceinline__ float kv_of(int, int w) const { return st->kv[w]; }
    __device__ __forceinline__ float d_of(int, int w) const { return st->d[w]; }
};

template <int JN>
__device__ __forceinline__ void hold_write_meta(Held<JN>& h, const Stage& st, int W, int rg, const Lane& ln) {
#pragma unroll
    for (int j = 0; j < JN; ++j) {
        const int w = ln.grp + j * rg, wc = w < W ? w : W - 1;
        h.slot[j] = st.kslot[wc];
        h.kv[j] = st.kv[wc];
        h.d[j] = st.d[wc];
    }
}

// Request the held rows, all before any is used.
template <typename E, int VB, int JN>
__device__ __forceinline__ void load_held_rows(typename RawVec<VB>::T (&row)[JN], const E* bank, const Held<JN>& h,
                                               int64_t hd, const Lane& ln) {
    using V = typename RawVec<VB>::T;
#pragma unroll
    for (int j = 0; j < JN; ++j) row[j] = *reinterpret_cast<const V*>(bank + h.slot[j] * hd + ln.vcol);
}

// Decay-and-write of the W rows this lane holds. No two of a stream's writes go
// to one slot (a precondition of the call), and no other workgroup writes these
// columns of these slots, so each element is stored once, with an ordinary
// store, and no atomics are needed. opaque() hides the raw bits from the
// optimiser, so the rows are widened again here instead of being kept widened
// (twice the registers for bfloat16) across the barriers before this point.
template <typename E, int VB, int JN, typename RowMeta>
__device__ __forceinline__ void write_back(typename RawVec<VB>::T (&row)[JN], E* bank, const RowMeta& h,
                                           const float* dv, int W, int rg, int64_t hd, const Lane& ln) {
    using V = typename RawVec<VB>::T;
    constexpr int VEC = VB / int(sizeof(E));
#pragma unroll
    for (int j = 0; j < JN; ++j) opaque(row[j]);
    float dvl[VEC];
#pragma unroll
    for (int e = 0; e < VEC; ++e) dvl[e] = dv[ln.lane * VEC + e];
#pragma unroll
    for (int j = 0; j < JN; ++j) {
        const int w = ln.grp + j * rg;
        if (ln.active && w < W) {
            E el[VEC];
            float out[VEC];
            __builtin_memcpy(el, &row[j], VB);
#pragma unroll
            for (int e = 0; e < VEC; ++e) {
                const float decayed = widen(el[e]) * h.d_of(j, w);
                out[e] = __builtin_fmaf(h.kv_of(j, w), dvl[e], decayed);
            }
            *reinterpret_cast<V*>(bank + h.slot_of(j, w) * hd + ln.vcol) = Pack<E, VB>::of(out);
        }
    }
}

// readings[row][col] = the column totals, rounded to the bank dtype.
template <typename E>
__device__ __forceinline__ void store_readings(const DecodeParams& p, const float* partial, int64_t out_row,
                                               const Lane& ln) {
    E* readings = static_cast<E*>(p.readings);
    for (int col = threadIdx.x; col < ln.slice_cols; col += blockDim.x) {
        const int64_t c = ln.col0 + col;
        if (c < p.hd) readings[out_row * p.hd + c] = narrow<E>(column_total(partial, p.rg, ln.slice_cols, col));
    }
}

template <int VEC>
__device__ __forceinline__ Lane lane_geometry(const DecodeParams& p) {
    Lane ln;
    ln.lane = threadIdx.x & (p.lpr - 1);
    ln.grp = threadIdx.x / p.lpr;
    ln.slice_cols = p.lpr * VEC;
    ln.vi = int(blockIdx.y) * p.lpr + ln.lane;
    ln.active = ln.vi < p.vpr;
    ln.vcol = int64_t(ln.active ? ln.vi : p.vpr - 1) * VEC;
    ln.col0 = int64_t(blockIdx.y) * ln.slice_cols;
    return ln;
}

// JN: rows a lane holds per phase (a power of two >= ceil(max(W, R) / RG)).
// MK, MV: metadata items per thread (W, R <= MK threads; the slice's columns <=
// MV threads).
template <typename E, int VB, int JN, int MK, int MV>
__global__ __launch_bounds__(1024) void sdm_decode_kernel(const DecodeParams p) {
    using V = typename RawVec<VB>::T;
    constexpr int VEC = VB / int(sizeof(E));
    extern __shared__ __align__(16) char s_raw[];
    const Lane ln = lane_geometry<VEC>(p);
    const int64_t s = blockIdx.x;
    const Stage st = carve_stage(s_raw, p.W, p.R, ln.slice_cols);
    float* partial = reinterpret_cast<float*>(s_raw + stage_bytes(p.W, p.R, ln.slice_cols));
    float* dv = partial + p.rg * ln.slice_cols;
    E* bank = static_cast<E*>(p.bank);

    V row[JN];
    if constexpr (JN <= 4) {
        // The write rows wait for this lane's own slots only, read straight from
        // global memory; the rest of the metadata is staged under their latency.
        Meta<MK, MV> m;
        meta_load<MK, MV, true>(p, 0, s, ln.col0, m);
        int64_t ks[JN];
#pragma unroll
        for (int j = 0; j < JN; ++j) {
            const int w = ln.grp + j * p.rg;
            ks[j] = slot_at(p.k_idx, s * p.W + (w < p.W ? w : p.W - 1), p.k_bytes);
        }
#pragma unroll
        for (int j = 0; j < JN; ++j) row[j] = *reinterpret_cast<const V*>(bank + ks[j] * p.hd + ln.vcol);
        asm volatile("" ::: "memory");
        meta_store<E, MK, MV>(p, m, st, ln.col0, ln.slice_cols);
        __syncthreads();
    } else {
        // (eight rows per lane: the slots' registers would cost occupancy)
        stage_now<E, MK, MV>(p, 0, s, st, ln.col0, ln.slice_cols);
        __syncthreads();
        load_rows<E, VB, JN>(row, bank, st.kslot, p.W, p.rg, p.hd, ln);
    }
    row_partials<E, VB, JN>(row, st.coef, p.W, p.rg, ln, partial);
    __syncthreads();
    form_delta(p, st, partial, dv, ln);
    __syncthreads();
    write_back<E, VB, JN>(row, bank, Staged{&st}, dv, p.W, p.rg, p.hd, ln);

    // Ordering point: the write-back is visible to the loads below, for read slots
    // that are also write slots. No other workgroup touches these columns of
    // these slots.
    __syncthreads();
    load_rows<E, VB, JN>(row, bank, st.qslot, p.R, p.rg, p.hd, ln);
    // The write phase's partials were last read before the barrier preceding the
    // write-back, so they can be overwritten now.
    row_partials<E, VB, JN>(row, st.qv, p.R, p.rg, ln, partial);
    __syncthreads();
    store_readings<E>(p, partial, s, ln);
}

// MK, MV: metadata items per thread fetched ahead (W, R <= MK threads; the
// slice's columns <= MV threads).
//
// Compact loop, for grids that keep many waves on each SIMD: the write rows of
// step t + 1 are requested with the read rows of step t, but their sums wait
// for the next iteration, so fewer values are live at once (at most 128 VGPRs)
// and more workgroups fit on a CU. Four barriers per step: the read rows' partial
// sums have an LDS buffer of their own, so a step ends at its readings (c2 +0.8 %
// against one shared buffer and a fifth barrier; c4 unchanged).
template <typename E, int VB, int JN, int MK, int MV>
__global__ __launch_bounds__(1024) void sdm_decode_steps_kernel(const DecodeParams p) {
    using V = typename RawVec<VB>::T;
    constexpr int VEC = VB / int(sizeof(E));
    extern __shared__ __align__(16) char s_raw[];
    const Lane ln = lane_geometry<VEC>(p);
    const int64_t s = blockIdx.x;
    const size_t sb = stage_bytes(p.W, p.R, ln.slice_cols);  // two Stage buffers, alternating by step
    float* partial = reinterpret_cast<float*>(s_raw + 2 * sb);
    float* dv = partial + p.rg * ln.slice_cols;
    float* partial_r = dv + ln.slice_cols;  // the read rows' partials, apart from the write rows'
    E* bank = static_cast<E*>(p.bank);
    const int T = p.steps;

    stage_now<E, MK, MV>(p, 0, s, carve_stage(s_raw, p.W, p.R, ln.slice_cols), ln.col0, ln.slice_cols);
    __syncthreads();
    V wrow[JN], rrow[JN];
    load_rows<E, VB, JN>(wrow, bank, carve_stage(s_raw, p.W, p.R, ln.slice_cols).kslot, p.W, p.rg, p.hd, ln);
    Meta<MK, MV> m;
    meta_load(p, min(1, T - 1), s, ln.col0, m);

    for (int t = 0; t < T; ++t) {
        const Stage st = carve_stage(s_raw + (t & 1) * sb, p.W, p.R, ln.slice_cols);
        const Stage nx = carve_stage(s_raw + ((t + 1) & 1) * sb, p.W, p.R, ln.slice_cols);
        // step t: retrieval, delta_v, write-back.
        row_partials<E, VB, JN>(wrow, st.coef, p.W, p.rg, ln, partial);
        __syncthreads();
        form_delta(p, st, partial, dv, ln);
        __syncthreads();
        write_back<E, VB, JN>(wrow, bank, Staged{&st}, dv, p.W, p.rg, p.hd, ln);
        // step t + 1's metadata (fetched during step t - 1) into the other buffer,
        // whose last reader (step t - 1's readings) finished before the barrier
        // that ended step t - 1.
        if (t + 1 < T) meta_store<E, MK, MV>(p, m, nx, ln.col0, ln.slice_cols);
        // Ordering point: step t's write-back is visible to every load below (step
        // t's reads and step t + 1's writes), and step t + 1's metadata is staged.
        __syncthreads();
        load_rows<E, VB, JN>(rrow, bank, st.qslot, p.R, p.rg, p.hd, ln);
        if (t + 1 < T) {
            load_rows<E, VB, JN>(wrow, bank, nx.kslot, p.W, p.rg, p.hd, ln);
            meta_load(p, min(t + 2, T - 1), s, ln.col0, m);
        }
        // step t: readings.
        row_partials<E, VB, JN>(rrow, st.qv, p.R, p.rg, ln, partial_r);
        __syncthreads();
        store_readings<E>(p, partial_r, int64_t(t) * p.streams + s, ln);
        // No barrier ends the step: the next step's write rows sum into the other
        // partial buffer, the read rows' partials here are next written after the
        // next step's third barrier, and this step's Stage buffer after its second
        // (every thread then past its last read of it, the read rows' partials).
    }
}

// Wide loop, for grids that leave at most two waves on each SIMD, where the
// memory parallelism has to come from within each wave. Iteration t: request the
// R rows of step t and the W rows of step t + 1 together, and while they are in
// flight stage step t + 2's metadata (fetched during the previous iteration;
// three Stage buffers rotate) and fetch step t + 3's; keep the slot, k_val and
// decay of each held write row in registers; one pass forms both partial sums
// (separate LDS buffers); barrier; readings of step t and delta_v of step
// t + 1; barrier; write-back of step t + 1; barrier (the ordering point for the
// next iteration's loads). Three barriers per step. At most 256 threads per
// workgroup, and the register budget of two waves per SIMD, so the compiler
// keeps both row sets and the fetched metadata in flight at once instead of
// trading that for occupancy the grid cannot use.
template <typename E, int VB, int JN, int MK, int MV>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1, 2)))
void sdm_decode_steps_wide_kernel(const DecodeParams p) {
    using V = typename RawVec<VB>::T;
    constexpr int VEC = VB / int(sizeof(E));
    extern __shared__ __align__(16) char s_raw[];
    const Lane ln = lane_geometry<VEC>(p);
    const int64_t s = blockIdx.x;
    const size_t sb = stage_bytes(p.W, p.R, ln.slice_cols);  // three Stage buffers: step t in buffer t % 3
    float* wpart = reinterpret_cast<float*>(s_raw + 3 * sb);  // retrieval partials [RG][slice]
    float* rpart = wpart + p.rg * ln.slice_cols;              // readings partials [RG][slice]
    float* dv = rpart + p.rg * ln.slice_cols;
    E* bank = static_cast<E*>(p.bank);
    const int T = p.steps;

    // step 0's write, alone: stage, request rows, retrieval, delta_v, write-back;
    // step 1's metadata staged, step 2's fetched.
    const Stage st0 = carve_stage(s_raw, p.W, p.R, ln.slice_cols);
    stage_now<E, MK, MV>(p, 0, s, st0, ln.col0, ln.slice_cols);
    Meta<MK, MV> m;
    meta_load(p, min(1, T - 1), s, ln.col0, m);
    __syncthreads();
    V wrow[JN], rrow[JN];
    Held<JN> h;
    hold_write_meta(h, st0, p.W, p.rg, ln);
    load_held_rows<E, VB, JN>(wrow, bank, h, p.hd, ln);
    if (T > 1) meta_store<E, MK, MV>(p, m, carve_stage(s_raw + sb, p.W, p.R, ln.slice_cols), ln.col0,
                                     ln.slice_cols);
    meta_load(p, min(2, T - 1), s, ln.col0, m);
    row_partials<E, VB, JN>(wrow, st0.coef, p.W, p.rg, ln, wpart);
    __syncthreads();
    form_delta(p, st0, wpart, dv, ln);
    __syncthreads();
    write_back<E, VB, JN>(wrow, bank, h, dv, p.W, p.rg, p.hd, ln);
    __syncthreads();

    int b0 = 0, b1 = 1, b2 = 2;  // buffers of steps t, t + 1, t + 2
    for (int t = 0; t < T; ++t) {
        const Stage st = carve_stage(s_raw + b0 * sb, p.W, p.R, ln.slice_cols);
        const Stage nx = carve_stage(s_raw + b1 * sb, p.W, p.R, ln.slice_cols);
        const bool more = t + 1 < T;
        // Step t's writes are visible here (the barrier above); both row sets may
        // contain slots step t wrote. The load phase has no branch (a guarded load
        // would be waited for where it is used): after the last step, the rows and
        // weights of step t's own writes stand in for step t + 1's, and their sums
        // go unused.
        const Stage& ws = more ? nx : st;
        load_rows<E, VB, JN>(rrow, bank, st.qslot, p.R, p.rg, p.hd, ln);
        hold_write_meta(h, ws, p.W, p.rg, ln);
        load_held_rows<E, VB, JN>(wrow, bank, h, p.hd, ln);
        // Step t + 2's buffer last held step t - 1, whose readers all finished
        // before the barrier that ended the previous iteration; its new contents
        // are read after this iteration's barriers.
        if (t + 2 < T)
            meta_store<E, MK, MV>(p, m, carve_stage(s_raw + b2 * sb, p.W, p.R, ln.slice_cols), ln.col0,
                                  ln.slice_cols);
        meta_load(p, min(t + 3, T - 1), s, ln.col0, m);
        row_partials<E, VB, JN>(rrow, st.qv, p.R, p.rg, ln, rpart);
        row_partials<E, VB, JN>(wrow, ws.coef, p.W, p.rg, ln, wpart);
        __syncthreads();
        store_readings<E>(p, rpart, int64_t(t) * p.streams + s, ln);
        if (more) form_delta(p, nx, wpart, dv, ln);
        __syncthreads();
        if (more) write_back<E, VB, JN>(wrow, bank, h, dv, p.W, p.rg, p.hd, ln);
        // Ordering point: step t + 1's write-back is visible to the next iteration's
        // loads.
        __syncthreads();
        const int b = b0;
        b0 = b1;
        b1 = b2;
        b2 = b;
    }
}

template <typename E, int VB, int JN>
void launch_jn(const DecodeParams& p, const DecodeGeometry& geo, hipStream_t stream) {
    const dim3 grid(unsigned(p.streams), unsigned(geo.slices));
    const dim3 block(unsigned(geo.threads));
    const int slice_cols = geo.lpr * (VB / int(sizeof(E)));
    const bool mk1 = p.W <= geo.threads && p.R <= geo.threads && slice_cols <= geo.threads;
    if (geo.loop == kLoopSingle && mk1)
        hipLaunchKernelGGL((sdm_decode_kernel<E, VB, JN, 1, 1>), grid, block, geo.lds, stream, p);
    else if (geo.loop == kLoopSingle)
        hipLaunchKernelGGL((sdm_decode_kernel<E, VB, JN, 4, 8>), grid, block, geo.lds, stream, p);
    else if (geo.loop == kLoopWide && mk1)
        hipLaunchKernelGGL((sdm_decode_steps_wide_kernel<E, VB, JN, 1, 1>), grid, block, geo.lds, stream, p);
    else if (geo.loop == kLoopWide)
        hipLaunchKernelGGL((sdm_decode_steps_wide_kernel<E, VB, JN, 4, 8>), grid, block, geo.lds, stream, p);
    else if (mk1)
        hipLaunchKernelGGL((sdm_decode_steps_kernel<E, VB, JN, 1, 1>), grid, block, geo.lds, stream, p);
    else
        hipLaunchKernelGGL((sdm_decode_steps_kernel<E, VB, JN, 4, 8>), grid, block, geo.lds, stream, p);
}

template <typename E, int VB>
hipError_t launch_vb(const DecodeParams& p, const DecodeGeometry& geo, hipStream_t stream) {
    switch (geo.jn) {
        case 1: launch_jn<E, VB, 1>(p, geo, stream); break;
        case 2: launch_jn<E, VB, 2>(p, geo, stream); break;
        case 4: launch_jn<E, VB, 4>(p, geo, stream); break;
        default: launch_jn<E, VB, 8>(p, geo, stream); break;
    }
    return hipGetLastError();
}

int pow2_ceil(int64_t x) {
    int p = 1;
    while (p < x) p <<= 1;
    return p;
}

}  // namespace

DecodeGeometry decode_geometry(int es, int64_t hd, int W, int R, uintptr_t bank_addr, int64_t steps,
                               int64_t streams, int cus, int force_loop) {
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
    // A thread fetches at most 4 slots of W and of R ahead of a step (8 elements
    // of v are covered by any lane group): widen the lane group (extra lanes past
    // the row end are idle) where that would not cover them. RG, and with it the
    // summation order, stays as it is.
    while (g.lpr * g.rg * 4 < wmax) g.lpr *= 2;
    g.slices = (g.vpr + g.lpr - 1) / g.lpr;
    g.threads = g.lpr * g.rg;
    const int slice_cols = g.lpr * (g.vb / es);
    const size_t stage = stage_bytes(W, R, slice_cols), cols = size_t(4) * size_t(slice_cols);
    if (steps <= 1) {
        // one staging buffer, partial [RG][slice] and delta_v [slice]
        g.loop = kLoopSingle;
        g.lds = stage + cols * size_t(g.rg + 1);
        return g;
    }
    // waves per SIMD (4 per CU) once the grid is spread over the CUs
    const int64_t blocks = streams * g.slices, c = cus > 0 ? cus : 1;
    const int64_t waves_per_block = (g.threads + 63) / 64;
    const int64_t waves_per_simd = ((blocks + c - 1) / c * waves_per_block + 3) / 4;
    const bool wide_fits = g.threads <= 256;
    g.loop = wide_fits && waves_per_simd <= 2 ? kLoopWide : kLoopCompact;
    if (force_loop == kLoopCompact || (force_loop == kLoopWide && wide_fits)) g.loop = force_loop;
    // compact: two staging buffers, the write rows' partials, delta_v, the read
    // rows' partials; wide: three staging buffers, two partial buffers, delta_v
    g.lds = (g.loop == kLoopWide ? 3 : 2) * stage + cols * size_t(2 * g.rg + 1);
    return g;
}

hipError_t launch_decode(const DecodeParams& p, const DecodeGeometry& geo, bool bf16, hipStream_t stream) {
    if (bf16) {
        switch (geo.vb) {
            case 16: return launch_vb<uint16_t, 16>(p, geo, stream);
            case 8: return launch_vb<uint16_t, 8>(p, geo, stream);
            case 4: return launch_vb<uint16_t, 4>(p, geo, stream);
            default: return launch_vb<uint16_t, 2>(p, geo, stream);
        }
    }
    switch (geo.vb) {
        case 16: return launch_vb<float, 16>(p, geo, stream);
        case 8: return launch_vb<float, 8>(p, geo, stream);
        default: return launch_vb<float, 4>(p, geo, stream);
    }
}

}  // namespace sdm
