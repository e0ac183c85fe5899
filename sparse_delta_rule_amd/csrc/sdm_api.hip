// The libsdm C ABI: argument checks, error reporting and kernel launches.
//
// The checks follow the argument contracts the pages state for the decode
// step (page "sparse_delta_memory/decode.py", sdm_decode_step) and the token
// gather (page "sparse_delta_memory/cuda/gather_cuda.py", token_gather and its
// host checks), reported as status codes with a thread-local message instead of
// exceptions. Everything cheap is checked on the host before the first HIP call.

#include <algorithm>
#include <atomic>
#include <cstdarg>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <string>
#include <unordered_map>
#include <vector>

#include "../../include/sdm.h"
#include "sdm_kernels.h"

namespace {

constexpr int kMaxDevices = 64;  // devices whose compute-unit count is cached

thread_local std::string g_last_error;

int fail(int code, const char* fmt, ...) {
    char buf[512];
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(buf, sizeof buf, fmt, ap);
    va_end(ap);
    g_last_error = buf;
    return code;
}

int ok() {
    g_last_error.clear();
    return SDM_OK;
}

int elem_size(int dtype) {
    switch (dtype) {
        case SDM_F32: return 4;
        case SDM_BF16: return 2;
        case SDM_I32: return 4;
        case SDM_I64: return 8;
        default: return 0;
    }
}

bool aligned(const void* p, int bytes) { return reinterpret_cast<uintptr_t>(p) % uintptr_t(bytes) == 0; }

// Half-open byte ranges [a, a + na) and [b, b + nb) intersect.
bool overlap(const void* a, int64_t na, const void* b, int64_t nb) {
    if (a == nullptr || b == nullptr || na <= 0 || nb <= 0) return false;
    const uintptr_t x = reinterpret_cast<uintptr_t>(a), y = reinterpret_cast<uintptr_t>(b);
    return x < y + uintptr_t(nb) && y < x + uintptr_t(na);
}

// a * b * c fits in int64 (all non-negative).
bool mul_fits(int64_t a, int64_t b, int64_t c = 1) {
    const int64_t lim = INT64_MAX;
    if (a == 0 || b == 0 || c == 0) return true;
    if (a > lim / b) return false;
    return a * b <= lim / c;
}

bool debug_validate() {
    static const int on = [] {
        const char* e = std::getenv("SDM_DEBUG_VALIDATE");
        return (e != nullptr && e[0] != '\0' && std::strcmp(e, "0") != 0) ? 1 : 0;
    }();
    return on != 0;
}

// Compute units of the current device, queried once per device.
int device_cus(int* cus) {
    static std::atomic<int> cache[kMaxDevices];  // 0: not queried yet
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return fail(SDM_E_HIP, "hipGetDevice failed: %s", hipGetErrorString(e));
    int v = dev >= 0 && dev < kMaxDevices ? cache[dev].load(std::memory_order_relaxed) : 0;
    if (v <= 0) {
        e = hipDeviceGetAttribute(&v, hipDeviceAttributeMultiprocessorCount, dev);
        if (e != hipSuccess || v <= 0)
            return fail(SDM_E_HIP, "cannot query the compute units of device %d: %s", dev, hipGetErrorString(e));
        if (dev >= 0 && dev < kMaxDevices) cache[dev].store(v, std::memory_order_relaxed);
    }
    *cus = v;
    return SDM_OK;
}

// SDM_STEPS_LOOP=compact|wide pins the multi-step loop; read on every call.
int forced_loop(int* loop) {
    const char* e = std::getenv("SDM_STEPS_LOOP");
    *loop = -1;
    if (e == nullptr || e[0] == '\0') return SDM_OK;
    if (std::strcmp(e, "compact") == 0) {
        *loop = sdm::kLoopCompact;
        return SDM_OK;
    }
    if (std::strcmp(e, "wide") == 0) {
        *loop = sdm::kLoopWide;
        return SDM_OK;
    }
    return fail(SDM_E_RANGE, "SDM_STEPS_LOOP is '%s'; expected 'compact' or 'wide'", e);
}

int check_device_ptr(const void* p, const char* name) {
    hipPointerAttribute_t attr;
    hipError_t e = hipPointerGetAttributes(&attr, p);
    if (e != hipSuccess) {
        (void)hipGetLastError();
        return fail(SDM_E_DEVICE, "%s is not a HIP device pointer (%s)", name, hipGetErrorString(e));
    }
    if (attr.type != hipMemoryTypeDevice && attr.type != hipMemoryTypeManaged)
        return fail(SDM_E_DEVICE, "%s is not device memory", name);
    return SDM_OK;
}

// Copy a device slot list to the host as int64.
int fetch_slots(const void* dev, int dtype, int64_t n, std::vector<int64_t>& out, hipStream_t stream,
                const char* name) {
    out.assign(size_t(n), 0);
    if (n == 0) return SDM_OK;
    hipError_t e;
    if (dtype == SDM_I64) {
        e = hipMemcpyAsync(out.data(), dev, size_t(n) * 8, hipMemcpyDeviceToHost, stream);
        if (e == hipSuccess) e = hipStreamSynchronize(stream);
    } else {
        std::vector<int32_t> tmp(static_cast<size_t>(n));
        e = hipMemcpyAsync(tmp.data(), dev, size_t(n) * 4, hipMemcpyDeviceToHost, stream);
        if (e == hipSuccess) e = hipStreamSynchronize(stream);
        if (e == hipSuccess)
            for (int64_t i = 0; i < n; ++i) out[size_t(i)] = tmp[size_t(i)];
    }
    if (e != hipSuccess) return fail(SDM_E_HIP, "copying %s to the host: %s", name, hipGetErrorString(e));
    return SDM_OK;
}

// The slot preconditions of a decode call, over all of its tokens: every slot in
// [0, num_slots), a stream's W write slots of a token distinct, and every slot
// touched (written or read) by one stream only, across all tokens, since the
// tokens of different streams run in no fixed order relative to one another.
int validate_decode_slots(int64_t num_slots, int64_t steps, int64_t streams, int W, int R, const void* k_idx,
                          int kd, const void* q_idx, int qd, hipStream_t stream) {
    std::vector<int64_t> k, q;
    int rc = fetch_slots(k_idx, kd, steps * streams * W, k, stream, "k_idx");
    if (rc != SDM_OK) return rc;
    rc = fetch_slots(q_idx, qd, steps * streams * R, q, stream, "q_idx");
    if (rc != SDM_OK) return rc;
    std::unordered_map<int64_t, int64_t> owner;
    owner.reserve(size_t(streams) * size_t(W + R));
    for (int64_t t = 0; t < steps; ++t) {
        for (int64_t s = 0; s < streams; ++s) {
            const int64_t* ks = k.data() + (t * streams + s) * W;
            const int64_t* qs = q.data() + (t * streams + s) * R;
            for (int w = 0; w < W; ++w) {
                if (ks[w] < 0 || ks[w] >= num_slots)
                    return fail(SDM_E_RANGE, "token %lld: k_idx[%lld, %d] = %lld outside [0, %lld)", (long long)t,
                                (long long)s, w, (long long)ks[w], (long long)num_slots);
                for (int u = 0; u < w; ++u)
                    if (ks[u] == ks[w])
                        return fail(SDM_E_RANGE, "token %lld: stream %lld writes slot %lld twice", (long long)t,
                                    (long long)s, (long long)ks[w]);
            }
            for (int r = 0; r < R; ++r)
                if (qs[r] < 0 || qs[r] >= num_slots)
                    return fail(SDM_E_RANGE, "token %lld: q_idx[%lld, %d] = %lld outside [0, %lld)", (long long)t,
                                (long long)s, r, (long long)qs[r], (long long)num_slots);
            for (int i = 0; i < W + R; ++i) {
                const int64_t x = i < W ? ks[i] : qs[i - W];
                auto it = owner.emplace(x, s);
                if (!it.second && it.first->second != s)
                    return fail(SDM_E_RANGE, "token %lld: slot %lld is used by streams %lld and %lld", (long long)t,
                                (long long)x, (long long)it.first->second, (long long)s);
            }
        }
    }
    return SDM_OK;
}

// The gather's slot preconditions over `rows` rows of its slot arrays: the
// per-chunk counts in [0, chunk], and the slots of every live row in
// [0, num_slots), row i being live when i mod chunk is below chunk i / chunk's
// count (chunk_valid), else below valid. A padding row is never read, so its
// slots may hold anything. A plan passes valid = chunk: its windows can make
// any row live.
int validate_gather_slots(int64_t num_slots, int64_t rows, int64_t chunk, int64_t valid, const int32_t* chunk_valid,
                          const void* idx0, int width0, const void* idx1, int width1, int idx_dtype,
                          hipStream_t stream) {
    std::vector<int32_t> cv;
    if (chunk_valid != nullptr) {
        const int64_t chunks = rows / chunk;
        cv.resize(static_cast<size_t>(chunks));
        hipError_t e = hipMemcpyAsync(cv.data(), chunk_valid, size_t(chunks) * 4, hipMemcpyDeviceToHost, stream);
        if (e == hipSuccess) e = hipStreamSynchronize(stream);
        if (e != hipSuccess) return fail(SDM_E_HIP, "copying chunk_valid: %s", hipGetErrorString(e));
        for (int64_t c = 0; c < chunks; ++c)
            if (cv[size_t(c)] < 0 || cv[size_t(c)] > chunk)
                return fail(SDM_E_RANGE, "chunk_valid[%lld] = %d outside [0, %lld]", (long long)c, cv[size_t(c)],
                            (long long)chunk);
    }
    const struct { const void* idx; int width; const char* name; } ops[] = {{idx0, width0, "idx0"},
                                                                           {idx1, width1, "idx1"}};
    for (const auto& op : ops) {
        if (op.idx == nullptr) continue;
        std::vector<int64_t> v;
        int rc = fetch_slots(op.idx, idx_dtype, rows * op.width, v, stream, op.name);
        if (rc != SDM_OK) return rc;
        for (int64_t i = 0; i < rows; ++i) {
            const int64_t limit = chunk_valid != nullptr ? int64_t(cv[size_t(i / chunk)]) : valid;
            if (i % chunk >= limit) continue;
            for (int n = 0; n < op.width; ++n) {
                const int64_t x = v[size_t(i * op.width + n)];
                if (x < 0 || x >= num_slots)
                    return fail(SDM_E_RANGE, "%s[%lld, %d] = %lld outside [0, %lld)", op.name, (long long)i, n,
                                (long long)x, (long long)num_slots);
            }
        }
    }
    return SDM_OK;
}

// Compact-stash positions: each below chunk * width0, and live entries of one
// chunk that name one position name one slot.
int validate_compact_positions(int64_t tokens, int64_t chunk, int64_t valid, const int32_t* chunk_valid,
                               const void* idx0, int width0, int idx_dtype, const int32_t* kpos,
                               hipStream_t stream) {
    std::vector<int64_t> slots;
    int rc = fetch_slots(idx0, idx_dtype, tokens * width0, slots, stream, "idx0");
    if (rc != SDM_OK) return rc;
    const int64_t n = tokens * width0, chunks = tokens / chunk, crow = chunk * width0;
    std::vector<int32_t> kp(static_cast<size_t>(n)), cv(static_cast<size_t>(chunk_valid ? chunks : 0));
    hipError_t e = hipMemcpyAsync(kp.data(), kpos, size_t(n) * 4, hipMemcpyDeviceToHost, stream);
    if (e == hipSuccess && chunk_valid != nullptr)
        e = hipMemcpyAsync(cv.data(), chunk_valid, size_t(chunks) * 4, hipMemcpyDeviceToHost, stream);
    if (e == hipSuccess) e = hipStreamSynchronize(stream);
    if (e != hipSuccess) return fail(SDM_E_HIP, "copying kpos: %s", hipGetErrorString(e));
    std::vector<int64_t> owner(static_cast<size_t>(crow));
    for (int64_t c = 0; c < chunks; ++c) {
        std::fill(owner.begin(), owner.end(), int64_t(-1));
        const int64_t limit = chunk_valid ? int64_t(cv[size_t(c)]) : valid;
        for (int64_t t = c * chunk; t < c * chunk + limit && t < (c + 1) * chunk; ++t)
            for (int j = 0; j < width0; ++j) {
                const int64_t i = t * width0 + j, p = kp[size_t(i)];
                if (p < 0) continue;
                if (p >= crow)
                    return fail(SDM_E_RANGE, "kpos[%lld, %d] = %lld outside [-1, %lld)", (long long)t, j, (long long)p,
                                (long long)crow);
                if (owner[size_t(p)] >= 0 && owner[size_t(p)] != slots[size_t(i)])
                    return fail(SDM_E_RANGE, "chunk %lld: position %lld is named by slots %lld and %lld", (long long)c,
                                (long long)p, (long long)owner[size_t(p)], (long long)slots[size_t(i)]);
                owner[size_t(p)] = slots[size_t(i)];
            }
    }
    return SDM_OK;
}

}  // namespace

extern "C" {

const char* sdm_last_error(void) { return g_last_error.c_str(); }

int sdm_abi_version(void) { return SDM_ABI_VERSION; }

int sdm_round_bf16(const float* in, uint16_t* out, int64_t n, void* hip_stream) {
    if (n < 0) return fail(SDM_E_SHAPE, "sdm_round_bf16: n = %lld < 0", (long long)n);
    if (n == 0) return ok();
    if (in == nullptr || out == nullptr) return fail(SDM_E_NULL, "sdm_round_bf16: in and out are required");
    if (!aligned(in, 8) || !aligned(out, 4))
        return fail(SDM_E_ALIGN, "sdm_round_bf16: in must be 8-byte and out 4-byte aligned");
    if (!mul_fits(n, 1, 4)) return fail(SDM_E_SHAPE, "sdm_round_bf16: n overflows 64-bit byte counts");
    if (overlap(in, n * 4, out, n * 2)) return fail(SDM_E_OVERLAP, "sdm_round_bf16: in and out overlap");
    hipError_t e = sdm::launch_round_bf16(in, out, n, static_cast<hipStream_t>(hip_stream));
    if (e != hipSuccess) return fail(SDM_E_HIP, "sdm_round_bf16: launch failed: %s", hipGetErrorString(e));
    return ok();
}

}  // extern "C"

namespace {

// Shared by sdm_decode_step (steps = 1, per-step arrays) and sdm_decode_steps.
int decode_call(const char* fn, void* bank, int bank_dtype, int64_t num_slots, int64_t head_dim, int64_t steps,
                int64_t streams, int32_t W, int32_t R, int32_t G, const void* k_idx, int k_idx_dtype,
                const void* k_val, const void* v, const void* q_val, int val_dtype, const float* beta,
                const float* g, const void* q_idx, int q_idx_dtype, void* readings, void* hip_stream) {
    if (bank_dtype != SDM_F32 && bank_dtype != SDM_BF16)
        return fail(SDM_E_DTYPE, "%s: bank must be float32 or bfloat16 (dtype %d)", fn, bank_dtype);
    if (val_dtype != SDM_F32 && val_dtype != SDM_BF16)
        return fail(SDM_E_DTYPE, "%s: k_val, v, q_val must be float32 or bfloat16 (dtype %d)", fn, val_dtype);
    if ((k_idx_dtype != SDM_I32 && k_idx_dtype != SDM_I64) || (q_idx_dtype != SDM_I32 && q_idx_dtype != SDM_I64))
        return fail(SDM_E_DTYPE, "%s: k_idx and q_idx must be int32 or int64 (dtypes %d, %d)", fn, k_idx_dtype,
                    q_idx_dtype);
    if (num_slots < 1 || head_dim < 1)
        return fail(SDM_E_SHAPE, "%s: empty bank [%lld, %lld]: num_slots and head_dim must both be positive", fn,
                    (long long)num_slots, (long long)head_dim);
    if (head_dim > SDM_MAX_ROW_BYTES / (bank_dtype == SDM_BF16 ? 2 : 4))
        return fail(SDM_E_RANGE, "%s: head_dim %lld: a bank row would exceed %lld bytes", fn, (long long)head_dim,
                    (long long)SDM_MAX_ROW_BYTES);
    if (streams < 0) return fail(SDM_E_SHAPE, "%s: streams = %lld < 0", fn, (long long)streams);
    if (steps < 0) return fail(SDM_E_SHAPE, "%s: steps = %lld < 0", fn, (long long)steps);
    if (W < 1 || W > SDM_MAX_WIDTH || R < 1 || R > SDM_MAX_WIDTH)
        return fail(SDM_E_RANGE, "%s: W=%d, R=%d: each width must lie in 1..%d", fn, W, R, SDM_MAX_WIDTH);
    if (G != 1 && G != W) return fail(SDM_E_SHAPE, "%s: G must be 1 or W=%d, got %d", fn, W, G);
    const int es = elem_size(bank_dtype);
    if (!mul_fits(num_slots, head_dim, es) || !mul_fits(steps, streams, head_dim * es) ||
        !mul_fits(steps, streams, SDM_MAX_WIDTH * 8))
        return fail(SDM_E_SHAPE, "%s: sizes overflow 64-bit byte counts", fn);
    if (streams > 0x7fffffffLL)
        return fail(SDM_E_SHAPE, "%s: at most 2^31-1 streams per call, got %lld", fn, (long long)streams);
    if (steps > 0x7fffffffLL) return fail(SDM_E_SHAPE, "%s: at most 2^31-1 steps per call", fn);
    if (streams == 0 || steps == 0) return ok();
    const struct { const void* p; const char* name; } req[] = {
        {bank, "bank"}, {k_idx, "k_idx"}, {k_val, "k_val"}, {v, "v"}, {q_val, "q_val"},
        {beta, "beta"}, {g, "g"}, {q_idx, "q_idx"}, {readings, "readings"}};
    for (const auto& r : req)
        if (r.p == nullptr) return fail(SDM_E_NULL, "%s: %s is NULL", fn, r.name);
    const int vs = elem_size(val_dtype);
    if (!aligned(bank, es) || !aligned(readings, es) || !aligned(k_idx, elem_size(k_idx_dtype)) ||
        !aligned(q_idx, elem_size(q_idx_dtype)) || !aligned(k_val, vs) || !aligned(v, vs) || !aligned(q_val, vs) ||
        !aligned(beta, 4) || !aligned(g, 4))
        return fail(SDM_E_ALIGN, "%s: a pointer is not aligned to its element size", fn);
    if (overlap(readings, steps * streams * head_dim * es, bank, num_slots * head_dim * es))
        return fail(SDM_E_OVERLAP, "%s: readings overlap the bank", fn);

    hipStream_t stream = static_cast<hipStream_t>(hip_stream);
    if (debug_validate()) {
        for (const auto& r : req) {
            int rc = check_device_ptr(r.p, r.name);
            if (rc != SDM_OK) return rc;
        }
        int rc = validate_decode_slots(num_slots, steps, streams, W, R, k_idx, k_idx_dtype, q_idx, q_idx_dtype, stream);
        if (rc != SDM_OK) return rc;
    }

    int cus = 0, force = -1;
    if (steps > 1) {
        int rc = device_cus(&cus);
        if (rc == SDM_OK) rc = forced_loop(&force);
        if (rc != SDM_OK) return rc;
    }
    const sdm::DecodeGeometry geo =
        sdm::decode_geometry(es, head_dim, W, R, reinterpret_cast<uintptr_t>(bank), steps, streams, cus, force);
    if (geo.slices > 65535)
        return fail(SDM_E_SHAPE, "%s: head_dim %lld needs %d column slices (max 65535)", fn, (long long)head_dim,
                    geo.slices);
    sdm::DecodeParams p{};
    p.bank = bank;
    p.k_idx = k_idx;
    p.q_idx = q_idx;
    p.k_val = k_val;
    p.v = v;
    p.q_val = q_val;
    p.beta = beta;
    p.g = g;
    p.readings = readings;
    p.hd = head_dim;
    p.streams = streams;
    p.steps = int(steps);
    p.W = W;
    p.R = R;
    p.G = G;
    p.vpr = geo.vpr;
    p.lpr = geo.lpr;
    p.rg = geo.rg;
    p.k_bytes = elem_size(k_idx_dtype);
    p.q_bytes = elem_size(q_idx_dtype);
    p.val_bytes = vs;
    hipError_t e = sdm::launch_decode(p, geo, bank_dtype == SDM_BF16, stream);
    if (e != hipSuccess) return fail(SDM_E_HIP, "%s: launch failed: %s", fn, hipGetErrorString(e));
    return ok();
}

}  // namespace

extern "C" {

int sdm_decode_step(void* bank, int bank_dtype, int64_t num_slots, int64_t head_dim, int64_t streams,
                    int32_t W, int32_t R, int32_t G, const void* k_idx, int k_idx_dtype, const void* k_val,
                    const void* v, const void* q_val, int val_dtype, const float* beta, const float* g,
                    const void* q_idx, int q_idx_dtype, void* readings, void* hip_stream) {
    return decode_call("sdm_decode_step", bank, bank_dtype, num_slots, head_dim, 1, streams, W, R, G, k_idx,
                       k_idx_dtype, k_val, v, q_val, val_dtype, beta, g, q_idx, q_idx_dtype, readings, hip_stream);
}

int sdm_decode_steps(void* bank, int bank_dtype, int64_t num_slots, int64_t head_dim, int64_t steps,
                     int64_t streams, int32_t W, int32_t R, int32_t G, const void* k_idx, int k_idx_dtype,
                     const void* k_val, const void* v, const void* q_val, int val_dtype, const float* beta,
                     const float* g, const void* q_idx, int q_idx_dtype, void* readings, void* hip_stream) {
    return decode_call("sdm_decode_steps", bank, bank_dtype, num_slots, head_dim, steps, streams, W, R, G, k_idx,
                       k_idx_dtype, k_val, v, q_val, val_dtype, beta, g, q_idx, q_idx_dtype, readings, hip_stream);
}

}  // extern "C"

namespace {

// A checked gather launch: its parameter block and geometry; run == false when there
// is nothing to launch (tokens == 0).
struct GatherLaunch {
    sdm::GatherParams p;
    sdm::GatherGeometry geo;
    int two, bf16, run;
};

// Every check of a gather call, then its launch parameters. index_rows: the rows of
// idx and w the call may read (tokens for a call, more for a plan), which the
// SDM_DEBUG_VALIDATE slot checks cover.
int gather_prepare(const char* fn, const void* bank, int bank_dtype, int64_t num_slots, int64_t head_dim,
                   int64_t tokens, int64_t chunk, int64_t valid, const int32_t* chunk_valid, int idx_dtype,
                   int w_dtype, const void* idx0, const void* w0, int32_t width0, float* out0, void* stash,
                   const int32_t* kpos, const void* idx1, const void* w1, int32_t width1, float* out1,
                   int64_t index_rows, hipStream_t stream, GatherLaunch* out) {
    out->run = 0;
    if (bank_dtype != SDM_F32 && bank_dtype != SDM_BF16)
        return fail(SDM_E_DTYPE, "%s: bank must be float32 or bfloat16 (dtype %d)", fn, bank_dtype);
    if (idx_dtype != SDM_I32 && idx_dtype != SDM_I64)
        return fail(SDM_E_DTYPE, "%s: indices must be int32 or int64 (dtype %d)", fn, idx_dtype);
    if (w_dtype != SDM_F32 && w_dtype != SDM_BF16)
        return fail(SDM_E_DTYPE, "%s: weights must be float32 or bfloat16 (dtype %d)", fn, w_dtype);
    if (num_slots < 1 || head_dim < 1)
        return fail(SDM_E_SHAPE, "%s: empty bank [%lld, %lld]: num_slots and head_dim must both be positive", fn,
                    (long long)num_slots, (long long)head_dim);
    if (head_dim > SDM_MAX_ROW_BYTES / (bank_dtype == SDM_BF16 ? 2 : 4))
        return fail(SDM_E_RANGE, "%s: head_dim %lld: a bank row would exceed %lld bytes", fn, (long long)head_dim,
                    (long long)SDM_MAX_ROW_BYTES);
    if (tokens < 0 || chunk < 1 || tokens % chunk != 0 || valid < 0 || valid > chunk)
        return fail(SDM_E_SHAPE, "%s: tokens must be a whole number of chunks and valid lie in [0, chunk]: tokens=%lld "
                    "chunk=%lld valid=%lld", fn, (long long)tokens, (long long)chunk, (long long)valid);
    if (width0 < 1 || width0 > SDM_MAX_WIDTH)
        return fail(SDM_E_RANGE, "%s: width0 must be in 1..%d, got %d", fn, SDM_MAX_WIDTH, width0);
    const bool two = idx1 != nullptr || w1 != nullptr || out1 != nullptr || width1 != 0;
    if (two) {
        if (idx1 == nullptr || w1 == nullptr || out1 == nullptr)
            return fail(SDM_E_NULL, "%s: operand 1 is given in part: pass idx1, w1 and out1 all, or none", fn);
        if (width1 < 1 || width1 > SDM_MAX_WIDTH)
            return fail(SDM_E_RANGE, "%s: width1 must be in 1..%d, got %d", fn, SDM_MAX_WIDTH, width1);
    }
    const int es = elem_size(bank_dtype);
    if (!mul_fits(num_slots, head_dim, es) || !mul_fits(tokens, SDM_MAX_WIDTH, head_dim * 8))
        return fail(SDM_E_SHAPE, "%s: sizes overflow 64-bit byte counts", fn);
    if (!mul_fits(index_rows, SDM_MAX_WIDTH, 8)) return fail(SDM_E_SHAPE, "%s: sizes overflow 64-bit byte counts", fn);
    if (tokens == 0) return ok();
    if (bank == nullptr || idx0 == nullptr || w0 == nullptr || out0 == nullptr)
        return fail(SDM_E_NULL, "%s: bank, idx0, w0 and out0 are required", fn);
    const int is = elem_size(idx_dtype), ws = elem_size(w_dtype);
    if (!aligned(bank, es) || !aligned(idx0, is) || !aligned(w0, ws) || !aligned(out0, 4) ||
        (stash != nullptr && !aligned(stash, es)) || !aligned(chunk_valid, 4) || !aligned(kpos, 4) ||
        (two && (!aligned(idx1, is) || !aligned(w1, ws) || !aligned(out1, 4))))
        return fail(SDM_E_ALIGN, "%s: a pointer is not aligned to its element size", fn);
    const int64_t bank_bytes = num_slots * head_dim * es;
    const int64_t out_bytes = tokens * head_dim * 4;
    const int64_t stash_bytes = stash != nullptr ? tokens * width0 * head_dim * es : 0;
    if (overlap(out0, out_bytes, bank, bank_bytes) || overlap(stash, stash_bytes, bank, bank_bytes) ||
        (two && overlap(out1, out_bytes, bank, bank_bytes)))
        return fail(SDM_E_OVERLAP, "%s: the stash or an output shares memory with the bank", fn);
    if (overlap(out0, out_bytes, stash, stash_bytes) || (two && (overlap(out1, out_bytes, stash, stash_bytes) ||
                                                                 overlap(out0, out_bytes, out1, out_bytes))))
        return fail(SDM_E_OVERLAP, "%s: the stash and the outputs share memory", fn);

    if (debug_validate()) {
        const void* ptrs[] = {bank, idx0, w0, out0, stash, chunk_valid, kpos, idx1, w1, out1};
        const char* names[] = {"bank", "idx0", "w0", "out0", "stash", "chunk_valid", "kpos", "idx1", "w1", "out1"};
        for (int i = 0; i < 10; ++i) {
            if (ptrs[i] == nullptr) continue;
            int rc = check_device_ptr(ptrs[i], names[i]);
            if (rc != SDM_OK) return rc;
        }
        int rc = validate_gather_slots(num_slots, index_rows, chunk, valid, chunk_valid, idx0, width0,
                                       two ? idx1 : nullptr, width1, idx_dtype, stream);
        if (rc == SDM_OK && kpos != nullptr)
            rc = validate_compact_positions(tokens, chunk, valid, chunk_valid, idx0, width0, idx_dtype, kpos, stream);
        if (rc != SDM_OK) return rc;
    }

    const sdm::GatherGeometry geo = sdm::gather_geometry(es, head_dim, reinterpret_cast<uintptr_t>(bank),
                                                         reinterpret_cast<uintptr_t>(stash), two);
    const int64_t blocks = (tokens + geo.tokens_per_block - 1) / geo.tokens_per_block;
    if (blocks > 0x7fffffffLL || geo.slices > 65535)
        return fail(SDM_E_SHAPE, "%s: %lld tokens x %d column slices exceed the grid", fn, (long long)tokens,
                    geo.slices);
    sdm::GatherParams& p = out->p;
    p = sdm::GatherParams{};
    p.bank = bank;
    p.stash = stash;
    p.idx0 = idx0;
    p.w0 = w0;
    p.out0 = out0;
    p.idx1 = two ? idx1 : nullptr;
    p.w1 = two ? w1 : nullptr;
    p.out1 = two ? out1 : nullptr;
    p.chunk_valid = chunk_valid;
    p.kpos = kpos;
    p.hd = head_dim;
    p.tokens = tokens;
    p.chunk = chunk;
    p.valid = valid;
    p.width0 = width0;
    p.width1 = two ? width1 : 0;
    p.vpr = geo.vpr;
    p.lpr = geo.lpr;
    p.idx64 = idx_dtype == SDM_I64;
    p.w_bf16 = w_dtype == SDM_BF16;
    p.out_vec = aligned(out0, 16) && (!two || aligned(out1, 16));
    out->geo = geo;
    out->two = two;
    out->bf16 = bank_dtype == SDM_BF16;
    out->run = 1;
    return SDM_OK;
}

// Shared by sdm_gather (kpos NULL) and sdm_gather_compact.
int gather_call(const char* fn, const void* bank, int bank_dtype, int64_t num_slots, int64_t head_dim,
                int64_t tokens, int64_t chunk, int64_t valid, const int32_t* chunk_valid, int idx_dtype, int w_dtype,
                const void* idx0, const void* w0, int32_t width0, float* out0, void* stash, const int32_t* kpos,
                const void* idx1, const void* w1, int32_t width1, float* out1, void* hip_stream) {
    hipStream_t stream = static_cast<hipStream_t>(hip_stream);
    GatherLaunch g;
    int rc = gather_prepare(fn, bank, bank_dtype, num_slots, head_dim, tokens, chunk, valid, chunk_valid, idx_dtype,
                            w_dtype, idx0, w0, width0, out0, stash, kpos, idx1, w1, width1, out1, tokens, stream, &g);
    if (rc != SDM_OK || !g.run) return rc == SDM_OK ? ok() : rc;
    hipError_t e = sdm::launch_gather(g.p, g.geo, g.bf16 != 0, g.two != 0, stream);
    if (e != hipSuccess) return fail(SDM_E_HIP, "%s: launch failed: %s", fn, hipGetErrorString(e));
    return ok();
}

// The contents of an sdm_gather_plan: a checked launch, the offsets a step moves
// the slot and weight pointers by, and the bounds a step is checked against.
constexpr uint64_t kPlanMagic = 0x314e414c50534453ull;  // "SDSPLAN1"
struct PlanImpl {
    uint64_t magic;
    GatherLaunch g;
    int64_t row0_max;
    int64_t chunk;  // valid's bound, also for a plan with nothing to launch
    int64_t idx_row0, w_row0, idx_row1, w_row1;  // bytes per token row of idx0, w0, idx1, w1
    int device;
};
static_assert(sizeof(PlanImpl) <= sizeof(sdm_gather_plan), "sdm_gather_plan is too small");
static_assert(alignof(PlanImpl) <= alignof(sdm_gather_plan), "sdm_gather_plan is under-aligned");

}  // namespace

extern "C" {

int sdm_gather(const void* bank, int bank_dtype, int64_t num_slots, int64_t head_dim, int64_t tokens, int64_t chunk,
               int64_t valid, const int32_t* chunk_valid, int idx_dtype, int w_dtype, const void* idx0,
               const void* w0, int32_t width0, float* out0, void* stash, const void* idx1, const void* w1,
               int32_t width1, float* out1, void* hip_stream) {
    return gather_call("sdm_gather", bank, bank_dtype, num_slots, head_dim, tokens, chunk, valid, chunk_valid,
                       idx_dtype, w_dtype, idx0, w0, width0, out0, stash, nullptr, idx1, w1, width1, out1, hip_stream);
}

int sdm_gather_compact(const void* bank, int bank_dtype, int64_t num_slots, int64_t head_dim, int64_t tokens,
                       int64_t chunk, int64_t valid, const int32_t* chunk_valid, int idx_dtype, int w_dtype,
                       const void* idx0, const void* w0, int32_t width0, float* out0, void* stash, const int32_t* kpos,
                       const void* idx1, const void* w1, int32_t width1, float* out1, void* hip_stream) {
    if (tokens > 0 && (stash == nullptr || kpos == nullptr))
        return fail(SDM_E_NULL, "sdm_gather_compact: stash and kpos are required");
    return gather_call("sdm_gather_compact", bank, bank_dtype, num_slots, head_dim, tokens, chunk, valid,
                       chunk_valid, idx_dtype, w_dtype, idx0, w0, width0, out0, stash, kpos, idx1, w1, width1, out1,
                       hip_stream);
}

int sdm_gather_plan_init(sdm_gather_plan* plan, const void* bank, int bank_dtype, int64_t num_slots,
                         int64_t head_dim, int64_t tokens, int64_t chunk, int64_t row0_max, int idx_dtype, int w_dtype,
                         const void* idx0, const void* w0, int32_t width0, float* out0, const void* idx1,
                         const void* w1, int32_t width1, float* out1) {
    const char* fn = "sdm_gather_plan_init";
    if (plan == nullptr) return fail(SDM_E_NULL, "%s: plan is NULL", fn);
    std::memset(plan, 0, sizeof *plan);
    if (row0_max < 0) return fail(SDM_E_SHAPE, "%s: row0_max = %lld < 0", fn, (long long)row0_max);
    if (tokens >= 0 && row0_max > INT64_MAX - tokens)
        return fail(SDM_E_SHAPE, "%s: row0_max + tokens overflows", fn);
    PlanImpl pl{};
    // Checked at the largest valid; every step's valid is checked against the chunk.
    int rc = gather_prepare(fn, bank, bank_dtype, num_slots, head_dim, tokens, chunk, chunk, nullptr, idx_dtype,
                            w_dtype, idx0, w0, width0, out0, nullptr, nullptr, idx1, w1, width1, out1,
                            tokens >= 0 ? row0_max + tokens : 0, nullptr, &pl.g);
    if (rc != SDM_OK) return rc;
    if (pl.g.run) {
        const hipError_t e = hipGetDevice(&pl.device);
        if (e != hipSuccess) return fail(SDM_E_HIP, "%s: hipGetDevice failed: %s", fn, hipGetErrorString(e));
    }
    const int is = elem_size(idx_dtype), ws = elem_size(w_dtype);
    pl.row0_max = row0_max;
    pl.chunk = chunk;
    pl.idx_row0 = int64_t(width0) * is;
    pl.w_row0 = int64_t(width0) * ws;
    pl.idx_row1 = pl.g.two ? int64_t(width1) * is : 0;
    pl.w_row1 = pl.g.two ? int64_t(width1) * ws : 0;
    pl.magic = kPlanMagic;
    std::memcpy(plan, &pl, sizeof pl);
    return ok();
}

int sdm_gather_plan_launch(const sdm_gather_plan* plan, int64_t row0, int64_t valid, void* hip_stream) {
    const char* fn = "sdm_gather_plan_launch";
    if (plan == nullptr) return fail(SDM_E_NULL, "%s: plan is NULL", fn);
    PlanImpl pl;
    std::memcpy(&pl, plan, sizeof pl);
    if (pl.magic != kPlanMagic) return fail(SDM_E_SHAPE, "%s: not an initialised gather plan", fn);
    if (row0 < 0 || row0 > pl.row0_max)
        return fail(SDM_E_RANGE, "%s: row0 = %lld outside [0, %lld]", fn, (long long)row0, (long long)pl.row0_max);
    if (valid < 0 || valid > pl.chunk)
        return fail(SDM_E_RANGE, "%s: valid = %lld outside [0, %lld]", fn, (long long)valid, (long long)pl.chunk);
    if (!pl.g.run) return ok();
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return fail(SDM_E_HIP, "%s: hipGetDevice failed: %s", fn, hipGetErrorString(e));
    if (dev != pl.device)
        return fail(SDM_E_DEVICE, "%s: the plan is for device %d, the current device is %d", fn, pl.device, dev);
    sdm::GatherParams p = pl.g.p;
    p.idx0 = static_cast<const char*>(p.idx0) + row0 * pl.idx_row0;
    p.w0 = static_cast<const char*>(p.w0) + row0 * pl.w_row0;
    if (pl.g.two) {
        p.idx1 = static_cast<const char*>(p.idx1) + row0 * pl.idx_row1;
        p.w1 = static_cast<const char*>(p.w1) + row0 * pl.w_row1;
    }
    p.valid = valid;
    e = sdm::launch_gather(p, pl.g.geo, pl.g.bf16 != 0, pl.g.two != 0, static_cast<hipStream_t>(hip_stream));
    if (e != hipSuccess) return fail(SDM_E_HIP, "%s: launch failed: %s", fn, hipGetErrorString(e));
    return ok();
}

}  // extern "C"
