// SDM token gather on gfx950.
//
// Per token and operand a float32-accumulated weighted sum of random bank rows,
// a raw copy of operand 0's rows (the stash), and zeros for padding positions
// (page "sparse_delta_memory/cuda/gather_cuda.py", module docstring).
//
// Layout: the unit of work is a (token, operand) pair, handled by LPR
// consecutive lanes (a power of two, up to a whole 64-lane wavefront); with two
// operands a token's pairs sit side by side, so both operands of a token run at
// once, and which operand a lane group serves is data (its slot and weight
// arrays, width and output), not a branch. Lane l owns vector (slice * LPR + l)
// of every row, so each row is read with 16-byte loads (narrower when a row is
// not a multiple of 16 bytes) and each lane accumulates its own columns. A lane
// walks its operand's entries in ascending order, one fused multiply-add chain
// per output element: no cross-lane reduction, and the result depends on the
// inputs alone.
//
// Memory pipeline: the slots and weights of the block's tokens are staged in
// LDS with contiguous, unconditional loads (CH entries per token and operand at
// a time; indices clamped into range, entries past a width or of padding
// tokens never read), so the only global round trips inside a pair's loop are
// its row loads. Entries are taken 32 at a time (fewer round trips per pair:
// measured faster than 8 or 16 at the same bytes in flight per SIMD, although
// it leaves two waves per SIMD), all of a batch's row loads issued before the
// first is used. Padding tokens load no row. Rows are loaded and outputs and
// stash rows stored non-temporally: all of them are touched once.
//
// Compact stash (CMP): operand 0's entry positions (kpos) are staged with its
// slots and weights, and a live entry with a position p >= 0 stores its row at
// row p of its chunk's block of chunk * width0 rows instead of at (t, n); other
// entries and padding tokens store nothing.
//
// Launches without a stash whose rows are at least 9 lane-vectors wide take the
// pair layout instead (sdm_gather_pair_kernel, described where it is defined):
// no LDS staging, the slots passed round a lane group of 16, 32 or 64 lanes by
// cross-lane moves, few registers and so more wavefronts in flight. Which layout
// runs changes no bit of any result.

#include "sdm_kernels.h"

namespace sdm {

namespace {

constexpr int kThreads = 256;
constexpr int kStageEntries = 1024;  // (token, operand) pairs per block x entries per pair staged at once
constexpr int kNB = 32;              // row loads in flight per lane (a power of two)
constexpr int kLiveMaxChunks = 4096; // most chunks a launch in the live-token layout scans (per workgroup)

// N consecutive entries [n0, n0 + N) of one operand, all valid: every row load
// is issued before the first row is used, and each row feeds the sum
// unconditionally (a row used only under a branch would have its load moved
// next to that use and waited for there). Registers: each row address is formed
// just before its load, the sums are taken as the rows arrive with the weights
// read four at a time, and only then are the stash rows stored under one branch
// (stores under a branch per row made the compiler hold every address and every
// weight across the batch). stash_row: this token's stash rows, or (CMP) its
// chunk's block of crow rows, whose row s_kp[k] an entry names (a position
// outside [0, crow) stores nothing); NULL for none.
template <typename E, int VB, int N, bool CMP, typename IdxT, typename WT>
__device__ __forceinline__ void gather_batch(const E* __restrict__ bank, int64_t hd, int64_t col, int n0, int k0,
                                             const IdxT* s_idx, const WT* s_w, const int32_t* s_kp, E* stash_row,
                                             int64_t crow, float (&acc)[VB / sizeof(E)]) {
    using V = typename RawVec<VB>::T;
    constexpr int VEC = VB / int(sizeof(E));
    using U = std::conditional_t<sizeof(IdxT) == 8, uint64_t, uint32_t>;  // slots are >= 0
    const char* lane_row = reinterpret_cast<const char*>(bank + col);
    const uint32_t row_bytes = uint32_t(hd * int64_t(sizeof(E)));
    V r[N];
    // four slots read from LDS at a time, each row's address formed just before its
    // load (a compiler barrier after each load: N addresses are never held at once)
#pragma unroll
    for (int i0 = 0; i0 < N; i0 += 4) {
        U sl[4];
#pragma unroll
        for (int j = 0; j < 4 && i0 + j < N; ++j) sl[j] = U(s_idx[k0 + i0 + j]);
#pragma unroll
        for (int j = 0; j < 4 && i0 + j < N; ++j) {
            r[i0 + j] = load_stream(reinterpret_cast<const V*>(lane_row + uint64_t(sl[j]) * row_bytes));
            asm volatile("" ::: "memory");
        }
    }
    // the sums first, as the rows arrive (weights read from LDS four at a time, not
    // all N ahead), then the stash stores under one branch
#pragma unroll
    for (int i = 0; i < N; ++i) {
        if (i % 4 == 0) asm volatile("" ::: "memory");
        const float x = value_of<WT>(s_w[k0 + i]);
        E el[VEC];
        __builtin_memcpy(el, &r[i], VB);
#pragma unroll
        for (int e = 0; e < VEC; ++e) acc[e] = __builtin_fmaf(x, widen(el[e]), acc[e]);
    }
    if (stash_row != nullptr) {
#pragma unroll
        for (int i = 0; i < N; ++i) {
            if constexpr (CMP) {
                const int32_t kp = s_kp[k0 + i];
                if (kp >= 0 && kp < crow) store_stream(reinterpret_cast<V*>(stash_row + int64_t(kp) * hd + col), r[i]);
            } else {
                store_stream(reinterpret_cast<V*>(stash_row + int64_t(n0 + i) * hd + col), r[i]);
            }
        }
    }
}

// Inclusive sum over a wavefront's 64 lanes, called with every lane active: DPP
// shifts right by 1, 2, 4 and 8 lanes within each row of 16 lanes (a lane whose
// source lies outside its row adds 0), then each row adds the totals of the rows
// before it, read from lanes 15, 31 and 47 into scalar registers.
__device__ __forceinline__ int32_t wave_inclusive_sum(int32_t x) {
    x += __builtin_amdgcn_update_dpp(0, x, 0x111, 0xf, 0xf, false);  // row_shr:1
    x += __builtin_amdgcn_update_dpp(0, x, 0x112, 0xf, 0xf, false);  // row_shr:2
    x += __builtin_amdgcn_update_dpp(0, x, 0x114, 0xf, 0xf, false);  // row_shr:4
    x += __builtin_amdgcn_update_dpp(0, x, 0x118, 0xf, 0xf, false);  // row_shr:8
    const int32_t r0 = __builtin_amdgcn_readlane(x, 15);
    const int32_t r1 = r0 + __builtin_amdgcn_readlane(x, 31);
    const int32_t r2 = r1 + __builtin_amdgcn_readlane(x, 47);
    const int row = int(threadIdx.x & 63) >> 4;
    return x + (row == 0 ? 0 : row == 1 ? r0 : row == 2 ? r1 : r2);
}

// Live-token layout (LIVE): token block b takes live tokens [b tpb, b tpb + tpb)
// of the L live tokens in order (chunk by chunk, each chunk's live positions), so
// every block but the last is full of live tokens, and then writes the outputs
// (and zero stash rows) of an equal share of the padding tokens; blocks past
// ceil(L / tpb) (at least one block works) exit at once. Each workgroup finds
// its tokens from the per-chunk live counts (a scan of chunk_valid in LDS, or
// the closed form of a scalar valid), its padding share by a binary search of
// that prefix. Results do not depend on the layout.
struct LiveMap {
    const int32_t* pref;  // LDS: pref[c] = live tokens in chunks [0, c), c <= chunks (NULL: scalar valid)
    int64_t chunks, chunk, v;  // v: live tokens per chunk for a scalar valid
    __device__ __forceinline__ int64_t before(int64_t c) const { return pref ? int64_t(pref[c]) : c * v; }
    // token of live index j < before(chunks) for a scalar valid
    __device__ __forceinline__ int64_t live_token(int64_t j) const {
        const int64_t c = j / v;
        return c * chunk + (j - c * v);
    }
    // token of padding index j < chunks chunk - before(chunks): in the last chunk c
    // with c chunk - before(c) <= j (the padding tokens before chunk c)
    __device__ __forceinline__ int64_t pad_token(int64_t j) const {
        int64_t lo = 0, hi = chunks - 1;
        while (lo < hi) {
            const int64_t mid = (lo + hi + 1) / 2;
            if (mid * chunk - before(mid) <= j) lo = mid; else hi = mid - 1;
        }
        const int64_t c = lo;
        return c * chunk + (before(c + 1) - before(c)) + (j - (c * chunk - before(c)));
    }
};

// NOPS: operands (1 or 2). CMP: compact stash. LIVE: live-token layout.
template <typename E, int VB, int NOPS, bool CMP, bool LIVE, typename IdxT, typename WT>
__global__ __launch_bounds__(kThreads) void sdm_gather_kernel(const GatherParams p) {
    using V = typename RawVec<VB>::T;
    constexpr int VEC = VB / int(sizeof(E));
    constexpr int kStageRounds = kStageEntries / kThreads;
    extern __shared__ __align__(16) char s_raw[];

    const int tid = threadIdx.x;
    const int tpb = kThreads / p.lpr / NOPS;  // tokens per block
    const int ch = kStageEntries / (tpb * NOPS);  // entries per pair staged at once
    const int lane = tid & (p.lpr - 1);
    const int pair = tid / p.lpr;
    const int g = pair / NOPS;               // token within the block
    const int op = pair - g * NOPS;          // operand
    // Workgroups are handed to the XCDs in turn (workgroup i to XCD i mod 8). In the
    // token order, give XCD x a contiguous share of the (token block, slice) pairs,
    // so chunk positions (live heads, padding tails) mix evenly over the XCDs, and
    // let each XCD start its walk through its share at a different point (x times
    // an eighth of the share, plus x): the eight XCDs' concurrent stash stores then
    // do not lie a power of two apart, as equal progress through shares of a
    // power-of-two stash would put them (one operand with a stash +1.5 %). In the
    // live-token layout, where live blocks come first, keep the hardware's order,
    // which deals them out to the XCDs in turn.
    int64_t tblock = blockIdx.x, slice = blockIdx.y;
    if constexpr (!LIVE) {
        const int64_t n = int64_t(gridDim.x) * gridDim.y, i = int64_t(blockIdx.y) * gridDim.x + blockIdx.x;
        const int64_t q = n / 8, r = n % 8, x = i % 8, k = i / 8;
        const int64_t sz = q + (x < r ? 1 : 0);  // this XCD's share (>= 1 for every workgroup)
        const int64_t j = x * q + (x < r ? x : r) + (k + x * (sz / 8 + 1)) % sz;
        tblock = j % gridDim.x;
        slice = j / gridDim.x;
    }

    // LDS: slots [op][token][ch], weights [op][token][ch], then (CMP) positions
    // laid out like the slots (operand 0's part used); then (LIVE) the block's
    // tokens [tpb], the per-chunk prefix [chunks + 1] and the wavefronts' totals.
    IdxT* s_idx = reinterpret_cast<IdxT*>(s_raw);
    WT* s_w = reinterpret_cast<WT*>(s_idx + kStageEntries);
    int32_t* s_kp = reinterpret_cast<int32_t*>(s_w + kStageEntries);
    int64_t* s_tok = reinterpret_cast<int64_t*>(
        s_raw + kStageEntries * (sizeof(IdxT) + sizeof(WT) + (CMP ? sizeof(int32_t) : 0)));
    int32_t* s_pref = reinterpret_cast<int32_t*>(s_tok + kThreads);

    int64_t t;          // this thread's token (meaningful when has_tok)
    bool has_tok, live;
    LiveMap m;                           // LIVE: the layout
    int64_t pad_begin = 0, pad_end = 0;  // LIVE: this block's share of the padding tokens
    if constexpr (LIVE) {
        m.chunks = p.tokens / p.chunk;
        m.chunk = p.chunk;
        m.v = 0;
        m.pref = nullptr;
        const int64_t j0 = tblock * tpb;  // this block's first live index
        if (tid < tpb) s_tok[tid] = 0;    // entries past the live tokens: token 0, whose rows stay unused
        int64_t live_total;
        if (p.chunk_valid != nullptr) {
            // exclusive prefix of the clamped counts: each thread sums a run of chunks,
            // the runs are scanned within each wavefront (DPP and lane reads) and across the
            // wavefronts (LDS); then each thread fills in its run and places the
            // block's live tokens that fall in its chunks
            const int64_t per = (m.chunks + kThreads - 1) / kThreads, c0 = tid * per;
            int32_t run = 0;
            for (int64_t c = c0; c < c0 + per && c < m.chunks; ++c) {
                const int32_t v = p.chunk_valid[c];
                const int32_t n = v < 0 ? 0 : (v > p.chunk ? int32_t(p.chunk) : v);
                s_pref[c] = n;  // the clamped count, until this thread's pass below
                run += n;
            }
            const int wl = tid & 63, wave = tid >> 6;
            const int32_t x = wave_inclusive_sum(run);
            int32_t* s_wave = s_pref + m.chunks + 1;  // [kThreads / 64] wavefront totals
            if (wl == 63) s_wave[wave] = x;
            __syncthreads();  // (also orders the s_tok defaults before the placements below)
            int32_t acc = x - run;
            for (int w = 0; w < wave; ++w) acc += s_wave[w];
            for (int64_t c = c0; c < c0 + per && c < m.chunks; ++c) {
                const int32_t n = s_pref[c];
                s_pref[c] = acc;
                const int64_t lo = acc > j0 ? acc : j0, hi = acc + n < j0 + tpb ? acc + n : j0 + tpb;
                for (int64_t j = lo; j < hi; ++j) s_tok[j - j0] = c * p.chunk + (j - acc);
                acc += n;
            }
            int32_t total = 0;
            for (int w = 0; w < kThreads / 64; ++w) total += s_wave[w];
            live_total = total;
            if (tid == kThreads - 1) s_pref[m.chunks] = total;
            m.pref = s_pref;
        } else {
            m.v = p.valid < p.chunk ? p.valid : p.chunk;
            live_total = m.before(m.chunks);
            __syncthreads();  // the s_tok defaults before the placements
            if (tid < tpb && j0 + tid < live_total) s_tok[tid] = m.live_token(j0 + tid);
        }
        const int64_t pads = p.tokens - live_total;
        const int64_t live_blocks = (live_total + tpb - 1) / tpb;
        const int64_t workers = live_blocks > 0 ? live_blocks : 1;
        if (tblock >= workers) return;  // a uniform exit: nothing of this launch is left for this block
        // the padding tokens are shared out over the blocks that take live tokens
        const int64_t per_block = (pads + workers - 1) / workers;
        pad_begin = tblock * per_block < pads ? tblock * per_block : pads;
        pad_end = pad_begin + per_block < pads ? pad_begin + per_block : pads;
        __syncthreads();
        has_tok = j0 + g < live_total;
        live = has_tok;
        t = s_tok[g];
    } else {
        t = tblock * tpb + g;
        has_tok = t < p.tokens;
        live = false;
        if (has_tok) {
            const int64_t chunk_no = t / p.chunk;
            const int64_t limit = p.chunk_valid != nullptr ? int64_t(p.chunk_valid[chunk_no]) : p.valid;
            live = (t - chunk_no * p.chunk) < limit;
        }
    }
    const int vi = int(slice) * p.lpr + lane;
    const bool lane_on = has_tok && vi < p.vpr;
    const int64_t col = int64_t(vi < p.vpr ? vi : 0) * VEC;

    const E* bank = static_cast<const E*>(p.bank);
    const int width = op == 0 ? p.width0 : p.width1;
    float* out = op == 0 ? p.out0 : p.out1;
    // CMP: the block of crow rows of t's chunk; else t's own rows.
    const int64_t crow = p.chunk * p.width0;
    const int64_t stash_base = CMP ? t / p.chunk * crow * p.hd : t * p.width0 * p.hd;
    E* stash_row = p.stash != nullptr && op == 0 && lane_on ? static_cast<E*>(p.stash) + stash_base : nullptr;

    float acc[VEC];
#pragma unroll
    for (int e = 0; e < VEC; ++e) acc[e] = 0.0f;

    if (!CMP && !live && stash_row != nullptr) {
        V zero;
        __builtin_memset(&zero, 0, VB);
        for (int n = 0; n < p.width0; ++n) store_stream(reinterpret_cast<V*>(stash_row + int64_t(n) * p.hd + col), zero);
    }

    const int wmax = NOPS == 2 && p.width1 > p.width0 ? p.width1 : p.width0;
    const int64_t t_first = tblock * tpb, t_last = p.tokens - 1;
    for (int base = 0; base < wmax; base += ch) {
        // ---- stage entries [base, base + ch) of every pair of the block: entry k of
        // the staging area is (operand, token, n) = (k / (tpb ch), k / ch % tpb, base + k % ch).
        __syncthreads();  // the previous chunk's entries consumed
        IdxT si[NOPS][kStageRounds];
        WT sw[NOPS][kStageRounds];
        int32_t sk[kStageRounds];
#pragma unroll
        for (int o = 0; o < NOPS; ++o) {
            const IdxT* idx = static_cast<const IdxT*>(o == 0 ? p.idx0 : p.idx1);
            const WT* w = static_cast<const WT*>(o == 0 ? p.w0 : p.w1);
            const int wd = o == 0 ? p.width0 : p.width1;
#pragma unroll
            for (int r = 0; r < kStageRounds / NOPS; ++r) {
                const int k = tid + r * kThreads;  // within this operand's [tpb][ch]
                const int tt = k / ch;
                const int n = min(base + (k - tt * ch), wd - 1);
                const int64_t tok = LIVE ? s_tok[tt] : min(t_first + tt, t_last);
                si[o][r] = idx[tok * wd + n];
                sw[o][r] = w[tok * wd + n];
                if (CMP && o == 0) sk[r] = p.kpos[tok * wd + n];
            }
        }
#pragma unroll
        for (int o = 0; o < NOPS; ++o)
#pragma unroll
            for (int r = 0; r < kStageRounds / NOPS; ++r) {
                s_idx[o * (kStageEntries / NOPS) + tid + r * kThreads] = si[o][r];
                s_w[o * (kStageEntries / NOPS) + tid + r * kThreads] = sw[o][r];
                if (CMP && o == 0) s_kp[tid + r * kThreads] = sk[r];
            }
        __syncthreads();
        if (!(live && lane_on)) continue;

        // ---- this pair's entries in ascending order: full batches of kNB, then the
        // rest in batches of 16, 8, 4, 2 and 1 (each at most once), so a short
        // tail costs a few round trips, not one per entry.
        const int k_base = op * (kStageEntries / NOPS) + g * ch - base;  // LDS index of entry n
        const int end = min(width, base + ch);
        int n = base;
        for (; n + kNB <= end; n += kNB)
            gather_batch<E, VB, kNB, CMP>(bank, p.hd, col, n, k_base + n, s_idx, s_w, s_kp, stash_row, crow, acc);
        if (n + 16 <= end) {
            gather_batch<E, VB, 16, CMP>(bank, p.hd, col, n, k_base + n, s_idx, s_w, s_kp, stash_row, crow, acc);
            n += 16;
        }
        if (n + 8 <= end) {
            gather_batch<E, VB, 8, CMP>(bank, p.hd, col, n, k_base + n, s_idx, s_w, s_kp, stash_row, crow, acc);
            n += 8;
        }
        if (n + 4 <= end) {
            gather_batch<E, VB, 4, CMP>(bank, p.hd, col, n, k_base + n, s_idx, s_w, s_kp, stash_row, crow, acc);
            n += 4;
        }
        if (n + 2 <= end) {
            gather_batch<E, VB, 2, CMP>(bank, p.hd, col, n, k_base + n, s_idx, s_w, s_kp, stash_row, crow, acc);
            n += 2;
        }
        if (n < end) gather_batch<E, VB, 1, CMP>(bank, p.hd, col, n, k_base + n, s_idx, s_w, s_kp, stash_row, crow, acc);
    }
    const auto store_out = [&](int64_t tok) {
        float* o = out + tok * p.hd + col;
        if (p.out_vec && VEC % 4 == 0) {
#pragma unroll
            for (int e = 0; e < VEC; e += 4)
                store_stream(reinterpret_cast<float4*>(o + e), make_float4(acc[e], acc[e + 1], acc[e + 2], acc[e + 3]));
        } else {
#pragma unroll
            for (int e = 0; e < VEC; ++e) store_stream(o + e, acc[e]);
        }
    };
    if (lane_on) store_out(t);
    if constexpr (LIVE) {
        // this block's share of the padding tokens: +0 outputs and, for a full stash,
        // zero stash rows, tpb tokens at a time in the same lane layout
        if (vi >= p.vpr) return;
#pragma unroll
        for (int e = 0; e < VEC; ++e) acc[e] = 0.0f;
        for (int64_t j0 = pad_begin; j0 < pad_end; j0 += tpb) {
            if (j0 + g >= pad_end) break;
            const int64_t tp = m.pad_token(j0 + g);
            store_out(tp);
            if (!CMP && p.stash != nullptr && op == 0) {
                E* row = static_cast<E*>(p.stash) + tp * p.width0 * p.hd;
                V zero;
                __builtin_memset(&zero, 0, VB);
                for (int n = 0; n < p.width0; ++n) store_stream(reinterpret_cast<V*>(row + int64_t(n) * p.hd + col), zero);
            }
        }
    }
}

// Pair layout, for launches without a stash and rows of at least 9 lane-vectors
// (lane groups of 16, 32 or 64 lanes): each group takes one (token, operand,
// slice) pair, the live pairs first (operand 0's, then operand 1's, each in the
// order of the live tokens and in whole wavefronts), then runs of kPadPairs padding pairs, whose
// outputs are +0. A pair's entries are taken in ascending batches of kFB: lane l
// of the group requests the slot and weight of entry l mod kFB of the next batch
// before this batch's rows, and the group passes them round by cross-lane moves
// that need no LDS round trip (DPP row broadcasts for 16-lane groups, which are
// DPP rows; reads of one lane into a scalar register for 32- and 64-lane
// groups), so each batch costs one memory round trip and the slots never pass
// through LDS; with no staging and no stash the kernel keeps few registers, so
// eight wavefronts per SIMD (more rows) are in flight. The same lanes, vectors
// and fused multiply-add chain as the token-order layout: the same bits.
constexpr int kFB = 8;
constexpr int kPadPairs = 8;

// Lane I of its group's value of a register, for lane groups of LPR lanes: a DPP
// row broadcast for 16-lane groups (a DPP row is 16 lanes), the lane read into a
// scalar register for 64-lane groups, and for 32-lane groups both halves' lanes
// read and each half taking its own; 16-, 32- or 64-bit values.
template <int LPR, int I> __device__ __forceinline__ uint32_t row_lane(uint32_t v) {
    if constexpr (LPR == 16) {
        return uint32_t(__builtin_amdgcn_update_dpp(0, int(v), 0x150 + I, 0xf, 0xf, false));
    } else if constexpr (LPR == 64) {
        return uint32_t(__builtin_amdgcn_readlane(int(v), I));
    } else {
        const uint32_t lo = uint32_t(__builtin_amdgcn_readlane(int(v), I));
        const uint32_t hi = uint32_t(__builtin_amdgcn_readlane(int(v), 32 + I));
        return (threadIdx.x & 32) ? hi : lo;
    }
}
template <int LPR, int I, typename T> __device__ __forceinline__ T bcast(T v) {
    if constexpr (sizeof(T) == 8) {
        const uint64_t x = uint64_t(v);
        const uint64_t lo = row_lane<LPR, I>(uint32_t(x)), hi = row_lane<LPR, I>(uint32_t(x >> 32));
        return T(lo | (hi << 32));
    } else if constexpr (sizeof(T) == 4) {
        uint32_t x;
        __builtin_memcpy(&x, &v, 4);
        x = row_lane<LPR, I>(x);
        T r;
        __builtin_memcpy(&r, &x, 4);
        return r;
    } else {
        return T(row_lane<LPR, I>(uint32_t(v)));
    }
}

// f(integral_constant<int, i>) for i = 0 .. N - 1, each i a constant expression
template <typename F, int... I> __device__ __forceinline__ void static_for_(F&& f, std::integer_sequence<int, I...>) {
    (f(std::integral_constant<int, I>{}), ...);
}
template <int N, typename F> __device__ __forceinline__ void static_for(F&& f) {
    static_for_(f, std::make_integer_sequence<int, N>{});
}

// Live pair index i -> (the pair's (token, slice) index k, operand): with two
// operands, operand 0's pairs take the first run = ceil(n / gpw) * gpw indices
// (whole wavefronts) and operand 1's the next run, so the operand is uniform over a
// wavefront; indices k >= n (the live tokens times the slices) name no pair (the
// end of a run). Operand-major, not interleaved by wavefront: the wavefronts in
// flight then store rows of one output that follow one another, never the same
// token's rows of both outputs at once. Two outputs allocated back to back lie a
// power of two apart when the token count is a power of two, and there such
// paired stores collide in the memory: 32768 tokens of 512-byte output rows (the
// outputs 16 MiB apart) took 204 us interleaved and 186 us operand-major, and
// with the interleaved order a shift of one output by 512 B to 64 KiB did not
// help where a shift by 1 MiB did.
__device__ __forceinline__ int64_t operand_pair(int64_t i, int64_t run, int& op) {
    op = i >= run ? 1 : 0;
    return op ? i - run : i;
}

// Token of live index j < before(chunks): position j - before(c) of the last
// chunk c with before(c) <= j, found by the LPR lanes of one group, which share j.
// Each step splits the remaining chunks into LPR parts of step chunks, lane l
// tests whether part l + 1 starts at or below j, and since the prefix never
// decreases the lanes that pass are lanes 0 .. n - 1, so their count n (a ballot)
// names the part that holds j. A probe past the remaining range fails (j lies
// before it), so each step keeps a whole part: 512 chunks take 3 dependent LDS
// reads (16 lanes) or 2 (32 and 64) before the last, against 9 for a binary search.
template <int LPR>
__device__ __forceinline__ int64_t group_live_at(const LiveMap& m, int64_t j, int lane) {
    if (m.pref == nullptr) return m.live_token(j);
    const int shift = int(threadIdx.x & 63) & ~(LPR - 1);  // the group's first lane in the wavefront
    int32_t lo = 0, n = int32_t(m.chunks);
    while (n > 1) {  // the same steps for every group (they depend on the chunk count only)
        const int32_t step = (n + LPR - 1) / LPR;
        const int32_t probe = lo + (lane + 1) * step;
        const bool pass = probe < m.chunks && m.pref[probe] <= j;
        uint64_t b = __ballot(pass) >> shift;
        if (LPR < 64) b &= (uint64_t(1) << LPR) - 1;
        lo += int32_t(__popcll(b)) * step;
        n = step;
    }
    return int64_t(lo) * m.chunk + (j - m.pref[lo]);
}

// One pair's entries [0, width): see the pair layout above. Entries past the
// width repeat entry width - 1 (the same row) and feed no sum. lane_row: this
// lane's vector of bank row 0; row_bytes: a row's bytes.
template <typename E, int VB, int LPR, typename IdxT, typename WT>
__device__ __forceinline__ void pair_sum(const char* lane_row, uint32_t row_bytes, const IdxT* idx, const WT* wts,
                                         int width, int lane, float (&acc)[VB / sizeof(E)]) {
    using V = typename RawVec<VB>::T;
    constexpr int VEC = VB / int(sizeof(E));
    using U = std::conditional_t<sizeof(IdxT) == 8, uint64_t, uint32_t>;  // slots are >= 0
    const int e0 = lane % kFB < width ? lane % kFB : width - 1;
    const IdxT ms0 = idx[e0];
    WT mw = wts[e0];
    opaque(mw);  // waited for here, with the slot, not at the loop's top
    U sl[kFB];
    static_for<kFB>([&](auto i) { sl[i] = U(bcast<LPR, i>(ms0)); });
    for (int n0 = 0; n0 < width; n0 += kFB) {
        // the next batch's slot and weight (this batch's again past the end)
        const int nx = n0 + kFB < width ? n0 + kFB : n0;
        const int e = nx + lane % kFB < width ? nx + lane % kFB : width - 1;
        const IdxT ms_next = idx[e];
        const WT mw_next = wts[e];
        V r[kFB];
#pragma unroll
        for (int i = 0; i < kFB; ++i) {
            r[i] = load_stream(reinterpret_cast<const V*>(lane_row + uint64_t(sl[i]) * row_bytes));
            // every row load issued before any row is used, each address formed just
            // before its load (eight addresses are not held at once)
            asm volatile("" ::: "memory");
        }
        const WT wcur = mw;
        mw = mw_next;
        static_for<kFB>([&](auto i) {
            const bool use = n0 + i < width;
            const float x = value_of<WT>(bcast<LPR, i>(wcur));
            E el[VEC];
            __builtin_memcpy(el, &r[i], VB);
#pragma unroll
            for (int k = 0; k < VEC; ++k) {
                const float term = __builtin_fmaf(x, widen(el[k]), acc[k]);
                acc[k] = use ? term : acc[k];
            }
        });
        static_for<kFB>([&](auto i) { sl[i] = U(bcast<LPR, i>(ms_next)); });
    }
}

// One work unit (a live pair or a padding run) per lane group; the host sizes the
// grid for the most units any liveness can give, and groups past the launch's
// units exit after the block's scan of the per-chunk counts.
template <typename E, int VB, int NOPS, int LPR, typename IdxT, typename WT>
__global__ __launch_bounds__(kThreads) void sdm_gather_pair_kernel(const GatherParams p) {
    constexpr int VEC = VB / int(sizeof(E));
    extern __shared__ __align__(16) char s_raw[];
    const int tid = threadIdx.x;
    const int lane = tid & (p.lpr - 1);
    const int groups = kThreads / p.lpr;
    const int slices = (p.vpr + p.lpr - 1) / p.lpr;

    LiveMap m;
    m.chunks = p.tokens / p.chunk;
    m.chunk = p.chunk;
    m.v = 0;
    m.pref = nullptr;
    if (p.chunk_valid != nullptr) {
        // exclusive prefix of the clamped per-chunk counts (runs of chunks per
        // thread, scanned by DPP within a wavefront and through LDS across them)
        int32_t* s_pref = reinterpret_cast<int32_t*>(s_raw);
        const int64_t per = (m.chunks + kThreads - 1) / kThreads, c0 = tid * per;
        int32_t run = 0;
        for (int64_t c = c0; c < c0 + per && c < m.chunks; ++c) {
            const int32_t v = p.chunk_valid[c];
            const int32_t n = v < 0 ? 0 : (v > p.chunk ? int32_t(p.chunk) : v);
            s_pref[c] = n;  // the clamped count, until this thread's pass below
            run += n;
        }
        const int wl = tid & 63, wave = tid >> 6;
        const int32_t x = wave_inclusive_sum(run);
        int32_t* s_wave = s_pref + m.chunks + 1;  // [kThreads / 64] wavefront totals
        if (wl == 63) s_wave[wave] = x;
        __syncthreads();
        int32_t acc = x - run;
        for (int w = 0; w < wave; ++w) acc += s_wave[w];
        for (int64_t c = c0; c < c0 + per && c < m.chunks; ++c) {
            const int32_t n = s_pref[c];
            s_pref[c] = acc;
            acc += n;
        }
        if (tid == kThreads - 1) s_pref[m.chunks] = acc;
        __syncthreads();
        m.pref = s_pref;
    } else {
        m.v = p.valid < p.chunk ? p.valid : p.chunk;
    }
    const int64_t live = m.before(m.chunks), pads = p.tokens - live;
    const int gpw = 64 / p.lpr;
    // live pair indices: with two operands, one run per operand, each rounded up to
    // whole wavefronts
    const int64_t live_ks = live * slices;
    const int64_t live_run = (live_ks + gpw - 1) / gpw * gpw;  // one operand's live pairs, whole wavefronts
    const int64_t live_pairs = NOPS == 2 ? 2 * live_run : live_ks;
    const int64_t pad_pairs = pads * NOPS * slices, pad_runs = (pad_pairs + kPadPairs - 1) / kPadPairs;
    const int64_t u = int64_t(blockIdx.x) * groups + tid / p.lpr;
    if (u >= live_pairs + pad_runs) return;
    const E* bank = static_cast<const E*>(p.bank);

    const auto store_out = [&](float* o, const float (&a)[VEC]) {
        if (p.out_vec && VEC % 4 == 0) {
#pragma unroll
            for (int e = 0; e < VEC; e += 4)
                store_stream(reinterpret_cast<float4*>(o + e), make_float4(a[e], a[e + 1], a[e + 2], a[e + 3]));
        } else {
#pragma unroll
            for (int e = 0; e < VEC; ++e) store_stream(o + e, a[e]);
        }
    };
    float acc[VEC];
#pragma unroll
    for (int e = 0; e < VEC; ++e) acc[e] = 0.0f;
    if (u < live_pairs) {
        int op = 0;
        const int64_t k = NOPS == 2 ? operand_pair(u, live_run, op) : u;
        if (k >= live_ks) return;
        op = __builtin_amdgcn_readfirstlane(op);  // uniform over the wavefront (whole runs)
        const int64_t t = group_live_at<LPR>(m, k / slices, lane);
        const int vi = int(k % slices) * p.lpr + lane;
        const int64_t col = int64_t(vi < p.vpr ? vi : p.vpr - 1) * VEC;
        const int width = op == 0 ? p.width0 : p.width1;
        const IdxT* idx = static_cast<const IdxT*>(op == 0 ? p.idx0 : p.idx1) + t * width;
        const WT* wts = static_cast<const WT*>(op == 0 ? p.w0 : p.w1) + t * width;
        const char* lane_row = reinterpret_cast<const char*>(bank + col);
        const uint32_t row_bytes = uint32_t(p.hd * int64_t(sizeof(E)));
        pair_sum<E, VB, LPR>(lane_row, row_bytes, idx, wts, width, lane, acc);
        if (vi < p.vpr) store_out((op == 0 ? p.out0 : p.out1) + t * p.hd + col, acc);
    } else {
        // a run of padding pairs: operand-major, then token, then slice
        const int64_t i0 = (u - live_pairs) * kPadPairs;
        for (int64_t i = i0; i < i0 + kPadPairs && i < pad_pairs; ++i) {
            const int op = NOPS == 2 ? int(i / (pads * slices)) : 0;
            const int64_t k = i - op * pads * slices;
            const int64_t t = m.pad_token(k / slices);
            const int vi = int(k % slices) * p.lpr + lane;
            if (vi < p.vpr) store_out((op == 0 ? p.out0 : p.out1) + t * p.hd + int64_t(vi) * VEC, acc);
        }
    }
}

template <typename E, int VB, int NOPS, int LPR, typename IdxT, typename WT>
hipError_t launch_pair_lpr(const GatherParams& p, hipStream_t stream) {
    // the live pairs of every token live, rounded up to whole runs, plus gpw: the
    // most work units a launch can hold (a padding run of kPadPairs pairs stands
    // for fewer live pairs than it replaces, but a last run of live pairs rounded
    // up can leave up to ceil((gpw - 1) / 4) padding runs beyond that count)
    const int64_t groups = kThreads / p.lpr, gpw = 64 / p.lpr, ks = p.tokens * ((p.vpr + p.lpr - 1) / p.lpr);
    const int64_t pairs = NOPS == 2 ? (ks + gpw - 1) / gpw * (2 * gpw) : ks;
    const int64_t blocks = (pairs + gpw + groups - 1) / groups;
    const size_t lds = p.chunk_valid ? size_t(p.tokens / p.chunk + 1 + kThreads / 64) * 4 : 0;
    hipLaunchKernelGGL((sdm_gather_pair_kernel<E, VB, NOPS, LPR, IdxT, WT>), dim3(unsigned(blocks)), dim3(kThreads),
                       lds, stream, p);
    return hipGetLastError();
}

// Lane groups of 16, 32 or 64 lanes, each its own kernel (registers allocated for
// its own broadcasts).
template <typename E, int VB, int NOPS, typename IdxT, typename WT>
hipError_t launch_pair_typed(const GatherParams& p, hipStream_t stream) {
    if (p.lpr == 16) return launch_pair_lpr<E, VB, NOPS, 16, IdxT, WT>(p, stream);
    if (p.lpr == 32) return launch_pair_lpr<E, VB, NOPS, 32, IdxT, WT>(p, stream);
    return launch_pair_lpr<E, VB, NOPS, 64, IdxT, WT>(p, stream);
}

template <typename E, int VB, int NOPS>
hipError_t launch_pair(const GatherParams& p, hipStream_t stream) {
    if (p.idx64)
        return p.w_bf16 ? launch_pair_typed<E, VB, NOPS, int64_t, uint16_t>(p, stream)
                        : launch_pair_typed<E, VB, NOPS, int64_t, float>(p, stream);
    return p.w_bf16 ? launch_pair_typed<E, VB, NOPS, int32_t, uint16_t>(p, stream)
                    : launch_pair_typed<E, VB, NOPS, int32_t, float>(p, stream);
}

template <typename E, int VB, int NOPS, bool CMP, bool LIVE, typename IdxT, typename WT>
hipError_t launch_typed(const GatherParams& p, const GatherGeometry& geo, hipStream_t stream) {
    // the live-token layout may need one more token block (its live and its padding
    // tokens each end in a partial block)
    const int64_t blocks = (p.tokens + geo.tokens_per_block - 1) / geo.tokens_per_block + (LIVE ? 1 : 0);
    const dim3 grid(unsigned(blocks), unsigned(geo.slices));
    const dim3 block(kThreads);
    size_t lds = size_t(kStageEntries) * (sizeof(IdxT) + sizeof(WT) + (CMP ? sizeof(int32_t) : 0));
    if (LIVE) lds += size_t(kThreads) * 8 + (p.chunk_valid ? size_t(p.tokens / p.chunk + 1 + kThreads / 64) * 4 : 0);
    hipLaunchKernelGGL((sdm_gather_kernel<E, VB, NOPS, CMP, LIVE, IdxT, WT>), grid, block, lds, stream, p);
    return hipGetLastError();
}

template <typename E, int VB, int NOPS, bool CMP, bool LIVE>
hipError_t launch_live(const GatherParams& p, const GatherGeometry& geo, hipStream_t stream) {
    if (p.idx64)
        return p.w_bf16 ? launch_typed<E, VB, NOPS, CMP, LIVE, int64_t, uint16_t>(p, geo, stream)
                        : launch_typed<E, VB, NOPS, CMP, LIVE, int64_t, float>(p, geo, stream);
    return p.w_bf16 ? launch_typed<E, VB, NOPS, CMP, LIVE, int32_t, uint16_t>(p, geo, stream)
                    : launch_typed<E, VB, NOPS, CMP, LIVE, int32_t, float>(p, geo, stream);
}

// The live-token layout is used where there is padding to separate (per-chunk
// counts over at most kLiveMaxChunks chunks, or a scalar valid below the chunk)
// and no full stash: with a full stash, padding tokens write whole zero stash
// rows, work the token order already spreads over the launch (measured: the
// live-token layout gains nothing there).
template <typename E, int VB, int NOPS, bool CMP>
hipError_t launch_ops(const GatherParams& p, const GatherGeometry& geo, hipStream_t stream) {
    if constexpr (!CMP) {
        if (p.stash == nullptr && p.lpr >= 16 && (p.chunk_valid == nullptr || p.tokens / p.chunk <= kLiveMaxChunks))
            return launch_pair<E, VB, NOPS>(p, stream);
    }
    const bool full_stash = p.stash != nullptr && !CMP;
    const bool live = !full_stash && (p.chunk_valid != nullptr ? p.tokens / p.chunk <= kLiveMaxChunks
                                                                : p.valid < p.chunk);
    return live ? launch_live<E, VB, NOPS, CMP, true>(p, geo, stream)
                : launch_live<E, VB, NOPS, CMP, false>(p, geo, stream);
}

template <typename E, int VB>
hipError_t launch_vb(const GatherParams& p, const GatherGeometry& geo, bool two, hipStream_t stream) {
    if (p.kpos != nullptr)
        return two ? launch_ops<E, VB, 2, true>(p, geo, stream) : launch_ops<E, VB, 1, true>(p, geo, stream);
    return two ? launch_ops<E, VB, 2, false>(p, geo, stream) : launch_ops<E, VB, 1, false>(p, geo, stream);
}

int pow2_ceil(int64_t x) {
    int p = 1;
    while (p < x) p <<= 1;
    return p;
}

}  // namespace

GatherGeometry gather_geometry(int es, int64_t hd, uintptr_t bank_addr, uintptr_t stash_addr, bool two) {
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
    g.tokens_per_block = kThreads / g.lpr / (two ? 2 : 1);
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
