// Internal declarations of the libsdm HIP path: launch parameter blocks, the
// element helpers the kernels share, and the launchers the C ABI calls.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace sdm {

constexpr int kMaxWidth = 256;

// ------------------------------------------------------------------ elements
// A bank element is kept as its raw bits: uint16_t for bfloat16, float for float32.
template <int VB> struct RawVec;
template <> struct RawVec<16> { using T = uint4; };
template <> struct RawVec<8> { using T = uint2; };
template <> struct RawVec<4> { using T = uint32_t; };
template <> struct RawVec<2> { using T = uint16_t; };

// Stores of data the kernel writes once and never reads back (outputs, the
// stash): marked non-temporal so the lines are not kept in the caches, which
// leaves their capacity to the random row reads sharing the memory system.
typedef uint32_t StreamU32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t StreamU32x2 __attribute__((ext_vector_type(2)));
__device__ __forceinline__ void store_stream(uint4* p, uint4 v) {
    const StreamU32x4 w = {v.x, v.y, v.z, v.w};
    __builtin_nontemporal_store(w, reinterpret_cast<StreamU32x4*>(p));
}
__device__ __forceinline__ void store_stream(uint2* p, uint2 v) {
    const StreamU32x2 w = {v.x, v.y};
    __builtin_nontemporal_store(w, reinterpret_cast<StreamU32x2*>(p));
}
__device__ __forceinline__ void store_stream(uint32_t* p, uint32_t v) { __builtin_nontemporal_store(v, p); }
__device__ __forceinline__ void store_stream(uint16_t* p, uint16_t v) { __builtin_nontemporal_store(v, p); }
__device__ __forceinline__ void store_stream(float* p, float v) { __builtin_nontemporal_store(v, p); }
__device__ __forceinline__ void store_stream(float4* p, float4 v) {
    store_stream(reinterpret_cast<uint4*>(p),
                 make_uint4(__float_as_uint(v.x), __float_as_uint(v.y), __float_as_uint(v.z), __float_as_uint(v.w)));
}

// Loads of rows read once and not written (the gather's): non-temporal, so they
// do not displace lines the caches can still use.
__device__ __forceinline__ uint4 load_stream(const uint4* p) {
    const StreamU32x4 w = __builtin_nontemporal_load(reinterpret_cast<const StreamU32x4*>(p));
    return make_uint4(w.x, w.y, w.z, w.w);
}
__device__ __forceinline__ uint2 load_stream(const uint2* p) {
    const StreamU32x2 w = __builtin_nontemporal_load(reinterpret_cast<const StreamU32x2*>(p));
    return make_uint2(w.x, w.y);
}
__device__ __forceinline__ uint32_t load_stream(const uint32_t* p) { return __builtin_nontemporal_load(p); }
__device__ __forceinline__ uint16_t load_stream(const uint16_t* p) { return __builtin_nontemporal_load(p); }

__device__ __forceinline__ float widen(uint16_t b) { return __uint_as_float(uint32_t(b) << 16); }
__device__ __forceinline__ float widen(float f) { return f; }

// float32 -> bfloat16 bits, round to nearest even, NaN kept a NaN with its quiet
// bit set: gfx950's packed conversion (two values per instruction). sdm_round_bf16
// exposes it, and a GPU test compares it, bit for bit, with the oracle's
// bit-level rounding on every one of the 2^32 float32 inputs (denormals and NaN
// payloads included).
typedef __bf16 Bf16x2 __attribute__((ext_vector_type(2)));
typedef float F32x2 __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t to_bf16x2_rne(float lo, float hi) {
    const F32x2 f = {lo, hi};
    const Bf16x2 h = __builtin_convertvector(f, Bf16x2);
    uint32_t u;
    __builtin_memcpy(&u, &h, 4);
    return u;
}
__device__ __forceinline__ uint16_t to_bf16_rne(float f) { return uint16_t(to_bf16x2_rne(f, 0.0f)); }

// Make a register's contents opaque to the optimiser (no instruction is
// emitted): values derived from it before this point are not reused after it.
__device__ __forceinline__ void opaque(uint4& v) {
    asm volatile("" : "+v"(v.x), "+v"(v.y), "+v"(v.z), "+v"(v.w));
}
__device__ __forceinline__ void opaque(uint2& v) { asm volatile("" : "+v"(v.x), "+v"(v.y)); }
__device__ __forceinline__ void opaque(uint32_t& v) { asm volatile("" : "+v"(v)); }
__device__ __forceinline__ void opaque(float& v) { asm volatile("" : "+v"(v)); }
__device__ __forceinline__ void opaque(uint16_t& v) {
    uint32_t w = v;
    asm volatile("" : "+v"(w));
    v = uint16_t(w);
}

template <typename E> __device__ __forceinline__ E narrow(float f);
template <> __device__ __forceinline__ uint16_t narrow<uint16_t>(float f) { return to_bf16_rne(f); }
template <> __device__ __forceinline__ float narrow<float>(float f) { return f; }

// VEC float32 results as one vector of bank elements (pairs converted together).
template <typename E, int VB> struct Pack;
template <int VB> struct Pack<float, VB> {
    static __device__ __forceinline__ typename RawVec<VB>::T of(const float (&r)[VB / 4]) {
        typename RawVec<VB>::T o;
        __builtin_memcpy(&o, r, VB);
        return o;
    }
};
template <int VB> struct Pack<uint16_t, VB> {
    static __device__ __forceinline__ typename RawVec<VB>::T of(const float (&r)[VB / 2]) {
        typename RawVec<VB>::T o;
        if constexpr (VB == 2) {
            o = to_bf16_rne(r[0]);
        } else {
            uint32_t w[VB / 4];
#pragma unroll
            for (int i = 0; i < VB / 4; ++i) w[i] = to_bf16x2_rne(r[2 * i], r[2 * i + 1]);
            __builtin_memcpy(&o, w, VB);
        }
        return o;
    }
};

// Round a float32 to the bank element type and widen it back.
template <typename E> __device__ __forceinline__ float to_bank(float f) { return widen(narrow<E>(f)); }

// A slot of an int32 (idx_bytes = 4) or int64 (8) array, with no branch on the
// type: two 32-bit loads, at the same address for int32, always both consumed
// (through a mask), so the compiler cannot move one of them under a branch and
// wait for it there.
__device__ __forceinline__ int64_t slot_at(const void* base, int64_t i, int idx_bytes) {
    const char* q = static_cast<const char*>(base) + i * idx_bytes;
    const uint32_t lo = *reinterpret_cast<const uint32_t*>(q);
    const uint32_t hi = *reinterpret_cast<const uint32_t*>(q + (idx_bytes - 4));
    const uint32_t wide = 0u - uint32_t(idx_bytes == 8);  // all ones for int64
    const uint32_t sign = uint32_t(int32_t(lo) >> 31);    // sign extension of an int32
    return int64_t((uint64_t((hi & wide) | (sign & ~wide)) << 32) | lo);
}

// A float32 (val_bytes = 4) or bfloat16 (2) value as float32, with no branch on
// the type: two 16-bit loads (little-endian halves), at the same address for
// bfloat16, whose bits are the high half of a float32; both always consumed.
__device__ __forceinline__ float value_at(const void* base, int64_t i, int val_bytes) {
    const char* q = static_cast<const char*>(base) + i * val_bytes;
    const uint32_t hi = *reinterpret_cast<const uint16_t*>(q + (val_bytes - 2));
    const uint32_t lo = *reinterpret_cast<const uint16_t*>(q);
    const uint32_t keep = 0u - uint32_t(val_bytes == 4);  // all ones for float32
    return __uint_as_float((hi << 16) | (lo & keep));
}

// A value or weight given as float32 or bfloat16 (raw bits), as float32.
template <typename T> __device__ __forceinline__ float value_of(T x);
template <> __device__ __forceinline__ float value_of<float>(float x) { return x; }
template <> __device__ __forceinline__ float value_of<uint16_t>(uint16_t x) { return widen(x); }

// ------------------------------------------------------------------ decode
struct DecodeParams {
    void* bank;
    const void* k_idx;
    const void* q_idx;
    const void* k_val;
    const void* v;
    const void* q_val;
    const float* beta;
    const float* g;
    void* readings;
    int64_t hd;
    int64_t streams;  // streams per step (the per-step stride of every input)
    int steps;        // tokens per stream in this call (1 for sdm_decode_step)
    int W, R, G;
    int vpr;  // vectors per row
    int lpr;  // lanes per row group: a power of two <= 32
    int rg;   // row groups
    int k_bytes, q_bytes, val_bytes;  // element sizes of k_idx, q_idx and the values
};

// Which decode kernel runs: one step, or the compact or wide multi-step loop.
constexpr int kLoopSingle = 0;
constexpr int kLoopCompact = 1;
constexpr int kLoopWide = 2;

struct DecodeGeometry {
    int vb;      // bytes per vector load: 16, 8, 4 or 2
    int vpr;     // vectors per row
    int lpr;     // lanes per row group
    int slices;  // column slices (grid y)
    int rg;      // row groups: fixes the summation order
    int jn;      // rows per lane per phase: 1, 2, 4 or 8
    int threads; // lpr * rg
    int loop;    // kLoopSingle, kLoopCompact or kLoopWide
    size_t lds;  // dynamic LDS bytes
};

// steps > 1 picks a multi-step loop: the wide one where the grid leaves at most
// two waves on each SIMD of `cus` compute units (and a workgroup has at most
// 256 threads), else the compact one. force_loop (kLoopCompact or kLoopWide,
// or -1 for none) overrides that choice where the wide loop can run.
DecodeGeometry decode_geometry(int es, int64_t hd, int W, int R, uintptr_t bank_addr, int64_t steps,
                               int64_t streams, int cus, int force_loop);
hipError_t launch_decode(const DecodeParams& p, const DecodeGeometry& geo, bool bf16, hipStream_t stream);

// ------------------------------------------------------------------ gather
struct GatherParams {
    const void* bank;
    void* stash;
    const void* idx0;
    const void* w0;
    float* out0;
    const void* idx1;
    const void* w1;
    float* out1;
    const int32_t* chunk_valid;
    const int32_t* kpos;  // NULL, or operand 0's compact-stash positions [tokens, width0]
    int64_t hd, tokens, chunk, valid;
    int width0, width1;
    int vpr;  // vectors per row
    int lpr;  // lanes per (token, operand) pair: a power of two <= 64
    int idx64, w_bf16;
    int out_vec;  // outputs aligned for whole-vector float stores
};

struct GatherGeometry {
    int vb;
    int vpr;
    int lpr;
    int slices;
    int tokens_per_block;
    int threads;
};

GatherGeometry gather_geometry(int es, int64_t hd, uintptr_t bank_addr, uintptr_t stash_addr, bool two);
hipError_t launch_gather(const GatherParams& p, const GatherGeometry& geo, bool bf16, bool two,
                         hipStream_t stream);

// ------------------------------------------------------------------ conversion
hipError_t launch_round_bf16(const float* in, uint16_t* out, int64_t n, hipStream_t stream);

}  // namespace sdm
