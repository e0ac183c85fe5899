/*
 * libsdm: the sparse-delta-memory (SDM) decode step and token gather on an
 * AMD Instinct MI355X (gfx950), behind a plain C ABI.
 *
 * Every pointer argument of a compute call is a DEVICE pointer to a contiguous,
 * row-major array that the caller owns; the library allocates nothing, keeps
 * no state between calls and only enqueues work on `hip_stream` (a
 * hipStream_t; NULL = the null stream), so calls may be captured in a HIP
 * graph. Results are ready when that stream reaches them. The cheap argument
 * checks run on the host before any HIP call; a failing call enqueues nothing
 * and returns one of the status codes below, with a message for
 * sdm_last_error() on the calling thread.
 *
 * Setting the environment variable SDM_DEBUG_VALIDATE=1 adds checks that need
 * the slot lists on the host (bounds, distinct write slots, private stream
 * ranges, per-chunk valid counts): each call then copies them from the device
 * and synchronises `hip_stream`. Without it those preconditions are not
 * checked, and a call that breaks them has undefined results.
 */
#ifndef SDM_H
#define SDM_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define SDM_ABI_VERSION 3 /* 2: adds sdm_gather_compact and the gather plan; 3: sdm_round_bf16 */
#define SDM_MAX_WIDTH 256 /* largest W, R and gather width */
#define SDM_MAX_ROW_BYTES (1LL << 30) /* largest bank row, head_dim x element size, in bytes */

/* Element types (sdm_dtype). */
enum {
    SDM_F32 = 0,  /* IEEE float32 */
    SDM_BF16 = 1, /* bfloat16: the high 16 bits of a float32 */
    SDM_I32 = 2,
    SDM_I64 = 3
};

/* Status codes (sdm_status). */
enum {
    SDM_OK = 0,
    SDM_E_DTYPE = 1,   /* an element type outside the ones an argument accepts */
    SDM_E_SHAPE = 2,   /* a size that is negative, zero where one is needed, or inconsistent */
    SDM_E_RANGE = 3,   /* a width outside 1..SDM_MAX_WIDTH, a bank row above SDM_MAX_ROW_BYTES,
                          a count outside its range, or a slot-list precondition broken
                          (SDM_DEBUG_VALIDATE only) */
    SDM_E_ALIGN = 4,   /* a pointer not aligned to its element size */
    SDM_E_OVERLAP = 5, /* an output overlapping the bank or another output */
    SDM_E_NULL = 6,    /* a required pointer is NULL (or operand 1 given in part) */
    SDM_E_DEVICE = 7,  /* no HIP device, or a pointer that is not device memory
                          (SDM_DEBUG_VALIDATE only) */
    SDM_E_HIP = 8      /* the HIP runtime reported an error; see sdm_last_error() */
};

/*
 * sdm_decode_step: advance every stream by one token, then read the bank back.
 *
 * Operation (page "sparse_delta_memory/decode.py", docstring of
 * sdm_decode_step; prior art: _sdm_decode_kernel on the same page). For each
 * stream s, with d[w] = exp(g[s, G == 1 ? 0 : w]):
 *     retrieved = sum_w k_val[s,w] d[w] bank[k_idx[s,w]]
 *     delta_v   = beta[s] (v[s] - retrieved)
 *     bank[k_idx[s,w]] = d[w] bank[k_idx[s,w]] + k_val[s,w] delta_v   for each w
 *     readings[s] = sum_r q_val[s,r] bank[q_idx[s,r]]                  after the writes
 * Only the W written rows change (decay is applied to them alone). k_val, v and
 * q_val are rounded to the bank dtype (round to nearest even) before use; beta
 * and g are float32; arithmetic is float32; rows are stored and readings
 * returned in the bank dtype (rounded to nearest even). d[w] is the float32
 * nearest to exp(g) (computed in double).
 *
 * Summation order (fixed, a function of W and R only): with
 *     RG = min(32, next_pow2(ceil(max(W, R) / 4)))
 * each column's retrieved is ((0 + p_0) + p_1) + ... + p_{RG-1}, where p_j is
 * the fused multiply-add chain over w = j, j + RG, j + 2 RG, ... ascending,
 * starting from +0, of (k_val[w] d[w]) * row_w (the product k_val[w] d[w]
 * rounded to float32 first); readings use the same scheme over r with q_val.
 * Each new row element is fma(k_val[w], delta_v, row * d[w]) with row * d[w]
 * rounded first, and delta_v = beta * (v - retrieved) with two roundings.
 * Results do not depend on the GPU's size or on which other streams are in the
 * call.
 *
 * Arguments:
 *   bank        [num_slots, head_dim] of bank_dtype (SDM_F32 or SDM_BF16);
 *               read and written in place.
 *   num_slots   >= 1. head_dim >= 1, a row of at most SDM_MAX_ROW_BYTES.
 *   streams     >= 0; 0 enqueues nothing and returns SDM_OK.
 *   W, R        write and read widths, 1..SDM_MAX_WIDTH.
 *   G           1 (one gate per stream) or W (one gate per write).
 *   k_idx       [streams, W] absolute bank rows, SDM_I32 or SDM_I64 (k_idx_dtype).
 *   k_val       [streams, W], v [streams, head_dim], q_val [streams, R], all of
 *               val_dtype (SDM_F32 or SDM_BF16).
 *   beta        [streams] float32.  g [streams, G] float32.
 *   q_idx       [streams, R] absolute bank rows, SDM_I32 or SDM_I64 (q_idx_dtype;
 *               may differ from k_idx_dtype).
 *   readings    [streams, head_dim] of bank_dtype, written; must not overlap bank.
 * Preconditions (checked only under SDM_DEBUG_VALIDATE): every slot is in
 * [0, num_slots); a stream's W write slots are distinct; the slots a stream
 * touches (written or read) belong to no other stream of the call. Read slots
 * may repeat (each occurrence adds its term) and may coincide with write slots
 * (the read sees the new row).
 * Errors: SDM_E_DTYPE, SDM_E_SHAPE, SDM_E_RANGE, SDM_E_NULL, SDM_E_ALIGN,
 * SDM_E_OVERLAP (readings and bank overlap), SDM_E_HIP (launch failure).
 */
int sdm_decode_step(void* bank, int bank_dtype, int64_t num_slots, int64_t head_dim,
                    int64_t streams, int32_t W, int32_t R, int32_t G,
                    const void* k_idx, int k_idx_dtype,
                    const void* k_val, const void* v, const void* q_val, int val_dtype,
                    const float* beta, const float* g,
                    const void* q_idx, int q_idx_dtype,
                    void* readings, void* hip_stream);

/*
 * sdm_decode_steps: advance every stream by `steps` tokens in one call.
 *
 * Operation: exactly `steps` successive sdm_decode_step calls (same results,
 * bit for bit), token t of every stream before token t + 1; the pages' decode
 * step is the single-token case of this multi-token recurrence (page
 * "sparse_delta_memory/decode.py", docstring of sdm_decode_step). One launch
 * keeps each stream's workgroup resident across its tokens and overlaps a
 * token's reads with the next token's row loads, for workloads where a single
 * step is too small to cover launch and memory latency.
 *
 * Arguments: as sdm_decode_step, each per-token array gaining a leading
 * [steps] axis (token-major, contiguous): k_idx, k_val [steps, streams, W];
 * v [steps, streams, head_dim]; beta [steps, streams]; g [steps, streams, G];
 * q_idx, q_val [steps, streams, R]; readings [steps, streams, head_dim] (must not
 * overlap the bank). steps >= 0; steps == 0 or streams == 0 enqueues nothing.
 * The preconditions apply to every token (slots of one stream stay private to
 * it across all tokens of the call). Errors: as sdm_decode_step; SDM_E_HIP also
 * when the device's compute-unit count cannot be queried, SDM_E_RANGE for an
 * unknown SDM_STEPS_LOOP value.
 *
 * The library runs one of two loops, with identical results: a wide one (every
 * row of a token in flight at once per wave) where the grid leaves at most two
 * waves on each SIMD, a compact one (fewer registers, more workgroups per CU)
 * otherwise. The environment variable SDM_STEPS_LOOP=wide or =compact, read on
 * every call, pins that choice (wide only where a stream's workgroup has at
 * most 256 threads); it exists for testing and tuning.
 */
int sdm_decode_steps(void* bank, int bank_dtype, int64_t num_slots, int64_t head_dim,
                     int64_t steps, int64_t streams, int32_t W, int32_t R, int32_t G,
                     const void* k_idx, int k_idx_dtype,
                     const void* k_val, const void* v, const void* q_val, int val_dtype,
                     const float* beta, const float* g,
                     const void* q_idx, int q_idx_dtype,
                     void* readings, void* hip_stream);

/*
 * sdm_gather: per-token weighted sums of bank rows, with a raw copy of the rows.
 *
 * Operation (page "sparse_delta_memory/cuda/gather_cuda.py", module docstring;
 * prior art: token_gather_kernel on the same page). For each token t of the
 * call and each operand o (operand 1 is optional):
 *     out_o[t]    = sum_n w_o[t,n] bank[idx_o[t,n]]      (float32 accumulation)
 *     stash[t, n] = bank[idx_0[t,n]]                     (raw bits, n < width0)
 * Token t is padding when (t mod chunk) >= limit, where limit = chunk_valid[t /
 * chunk] if chunk_valid is given, else valid: a padding token reads no slot or
 * weight and writes +0.0 outputs and all-zero stash rows. Weights are used as
 * given (a bfloat16 weight is widened exactly, not rounded to the bank dtype).
 *
 * Summation order (fixed): each output element is one fused multiply-add
 * chain over n = 0, 1, ..., width-1 ascending, starting from +0 (the "groups =
 * 1" order of the pages); it depends on nothing but the inputs.
 *
 * Arguments:
 *   bank         [num_slots, head_dim] of bank_dtype (SDM_F32 or SDM_BF16); read only;
 *                num_slots, head_dim >= 1, a row of at most SDM_MAX_ROW_BYTES.
 *   tokens       >= 0, a multiple of chunk; 0 enqueues nothing and returns SDM_OK.
 *   chunk        >= 1.  valid in [0, chunk].
 *   chunk_valid  NULL, or [tokens / chunk] int32 on the device, each in [0, chunk]
 *                (checked only under SDM_DEBUG_VALIDATE); overrides valid.
 *   idx_dtype    SDM_I32 or SDM_I64, for both operands.  w_dtype SDM_F32 or SDM_BF16.
 *   idx0, w0     [tokens, width0]; width0 in 1..SDM_MAX_WIDTH.  out0 [tokens, head_dim] float32.
 *   stash        NULL (no copy), or [tokens, width0, head_dim] of bank_dtype.
 *   idx1, w1, out1, width1: the second operand, like the first; all NULL with
 *                width1 = 0 for one operand, or all given with width1 in 1..SDM_MAX_WIDTH.
 * Slots of live tokens must lie in [0, num_slots) (checked only under
 * SDM_DEBUG_VALIDATE); a padding token's slots and weights are never read and may
 * hold anything.
 * Outputs and stash must not overlap the bank or one another (SDM_E_OVERLAP).
 * Errors: SDM_E_DTYPE, SDM_E_SHAPE, SDM_E_RANGE, SDM_E_NULL, SDM_E_ALIGN,
 * SDM_E_OVERLAP, SDM_E_HIP.
 */
int sdm_gather(const void* bank, int bank_dtype, int64_t num_slots, int64_t head_dim,
               int64_t tokens, int64_t chunk, int64_t valid, const int32_t* chunk_valid,
               int idx_dtype, int w_dtype,
               const void* idx0, const void* w0, int32_t width0, float* out0, void* stash,
               const void* idx1, const void* w1, int32_t width1, float* out1,
               void* hip_stream);

/*
 * sdm_gather_compact: sdm_gather with a compact stash.
 *
 * Operation (page "sparse_delta_memory/cuda/gather_cuda.py": the kernel's
 * snapshot addressing when a position map is passed, and the checks that
 * token_gather_dc makes of that map). Outputs exactly as sdm_gather. The stash
 * is one block of chunk * width0 rows per chunk, [tokens / chunk, chunk * width0,
 * head_dim] in the bank dtype (as many bytes as sdm_gather's stash): entry n of a
 * live token t with p = kpos[t, n] >= 0 copies the raw row bank[idx0[t, n]] to
 * row p of the block of chunk t / chunk. Entries with a negative position and
 * every entry of a padding token copy nothing, and rows that no entry names keep
 * their contents (nothing is zeroed). On the pages the map gives each entry the
 * first position of its slot in its chunk's sorted list of slots, so the block
 * holds each distinct row once and entries with one slot share a position.
 *
 * Arguments: as sdm_gather, with
 *   stash   required: [tokens / chunk, chunk * width0, head_dim] of bank_dtype.
 *   kpos    required: [tokens, width0] int32 on the device.
 * Preconditions (checked only under SDM_DEBUG_VALIDATE, with sdm_gather's): every
 * position is below chunk * width0 (a position at or past it stores nothing);
 * live entries of one chunk that name one position name one slot (otherwise
 * which row lands there is not defined).
 * Errors: as sdm_gather; SDM_E_NULL when tokens > 0 and stash or kpos is NULL.
 */
int sdm_gather_compact(const void* bank, int bank_dtype, int64_t num_slots, int64_t head_dim,
                       int64_t tokens, int64_t chunk, int64_t valid, const int32_t* chunk_valid,
                       int idx_dtype, int w_dtype,
                       const void* idx0, const void* w0, int32_t width0, float* out0,
                       void* stash, const int32_t* kpos,
                       const void* idx1, const void* w1, int32_t width1, float* out1,
                       void* hip_stream);

/*
 * sdm_gather_plan_init / sdm_gather_plan_launch: one gather checked once and
 * launched many times, each launch on another window of slot rows.
 *
 * Operation (page "sparse_delta_memory/cuda/gather_cuda.py": the plan and step
 * functions that follow token_gather_dc, which check a launch once at the
 * largest row offset a step will use and then launch it per step with the row
 * offset and valid replaced). sdm_gather_plan_init runs every check of
 * sdm_gather, without a stash or per-chunk counts, for `tokens` tokens whose
 * slots and weights are rows [row0, row0 + tokens) of idx0 and w0 (and idx1, w1)
 * for any row0 in [0, row0_max], and stores the launch in *plan. Then
 *     sdm_gather_plan_launch(plan, row0, valid, hip_stream)
 * gives, bit for bit, what
 *     sdm_gather(bank, ..., tokens, chunk, valid, NULL, idx_dtype, w_dtype,
 *                idx0 + row0 * width0, w0 + row0 * width0, width0, out0, NULL,
 *                idx1 + row0 * width1, w1 + row0 * width1, width1, out1, hip_stream)
 * gives (pointer steps in elements), checking only the plan, row0, valid and
 * that the current device is the plan's. Every launch writes the same out0 and
 * out1; padding is (t mod chunk) >= valid with t counted from the launch's
 * first token, as in sdm_gather.
 *
 * The plan is a plain caller-owned struct (the library allocates nothing). It
 * holds raw device pointers, so the caller keeps every array it names alive and
 * in place while using the plan; a copy of the struct is the same plan. Launches
 * are asynchronous on hip_stream and may be captured in a HIP graph (a captured
 * launch keeps the row0 and valid it was captured with).
 *
 * Arguments of sdm_gather_plan_init: as sdm_gather without valid, chunk_valid
 * and stash, and
 *   plan       where the plan is stored (zeroed first, so a failed init leaves
 *              no usable plan).
 *   row0_max   >= 0: idx0 and w0 (idx1 and w1) hold row0_max + tokens rows.
 * Under SDM_DEBUG_VALIDATE init checks the slots of all row0_max + tokens rows
 * (copying them on the null stream).
 * Errors of init: as sdm_gather; SDM_E_NULL for a NULL plan; SDM_E_HIP when the
 * current device cannot be queried. Errors of launch: SDM_E_NULL (NULL plan),
 * SDM_E_SHAPE (not an initialised plan), SDM_E_RANGE (row0 outside
 * [0, row0_max] or valid outside [0, chunk]), SDM_E_DEVICE (the current device
 * is not the plan's), SDM_E_HIP (launch failure).
 */
typedef struct {
    uint64_t opaque[48];
} sdm_gather_plan;

int sdm_gather_plan_init(sdm_gather_plan* plan, const void* bank, int bank_dtype, int64_t num_slots,
                         int64_t head_dim, int64_t tokens, int64_t chunk, int64_t row0_max,
                         int idx_dtype, int w_dtype,
                         const void* idx0, const void* w0, int32_t width0, float* out0,
                         const void* idx1, const void* w1, int32_t width1, float* out1);

int sdm_gather_plan_launch(const sdm_gather_plan* plan, int64_t row0, int64_t valid, void* hip_stream);

/* Message of the last failing call on this thread ("" if none). The pointer stays
 * valid until the next libsdm call on the same thread. */
const char* sdm_last_error(void);

/* SDM_ABI_VERSION of the library. */
int sdm_abi_version(void);

/*
 * sdm_round_bf16: out[i] = the bfloat16 bits of in[i], rounded as every kernel of
 * this library rounds a float32 it stores in a bfloat16 bank or returns as a
 * bfloat16 reading: to nearest, ties to even, denormals kept, a NaN kept a NaN
 * with its sign and its high payload bits and the quiet bit set (page
 * "sparse_delta_memory/decode.py": the decode kernel's casts to the bank dtype).
 * Exposed so that the conversion can be checked on its own against a reference.
 * in: [n] float32 (8-byte aligned), out: [n] bfloat16 bits (4-byte aligned),
 * device pointers owned by the caller, not overlapping. Asynchronous on
 * hip_stream. Errors: SDM_E_SHAPE (n < 0), SDM_E_NULL, SDM_E_ALIGN,
 * SDM_E_OVERLAP, SDM_E_HIP.
 */
int sdm_round_bf16(const float* in, uint16_t* out, int64_t n, void* hip_stream);

#ifdef __cplusplus
}
#endif

#endif /* SDM_H */
