/*
 * libsdm_ceiling: reference access patterns over a bank of rows, for measuring
 * what random rows allow on this device. They are the yardstick that the
 * decode's and the gather's fractions of the HBM peak are read against: not
 * part of the method, and no step of the decode or the gather calls them.
 *
 * Each pattern is one kernel launch over n units, every row touched as 16-byte
 * vectors by consecutive lanes (the layout the decode and gather kernels use),
 * with several units' loads in flight per lane group before any is used:
 *
 *   SDM_CEIL_READ    unit i reads row rows[i]; every loaded 32-bit word is
 *                    XOR-folded into a per-thread word written to sink
 *                    (sink holds sdm_ceiling_sink_words() words).
 *   SDM_CEIL_STASH   unit i reads row rows[i] and stores it to stash row i
 *                    (non-temporal stores: a stream written once).
 *   SDM_CEIL_RMW     unit i reads row rows[i] and writes it back in place with
 *                    every 32-bit word XORed with 0x00010001 (rows[] must hold
 *                    distinct rows, or writes race).
 *   SDM_CEIL_MIX     unit i does SDM_CEIL_RMW on rows[2i] and SDM_CEIL_READ on
 *                    rows[2i + 1]: two row reads and one row write per unit, the
 *                    decode's mix (W rows read and written, R rows read). The
 *                    rows[2i] must be distinct from one another and from every
 *                    rows[2j + 1].
 *
 * sdm_ceiling_copy copies `bytes` bytes (a multiple of 16, both pointers
 * 16-byte aligned) from src to dst with 16-byte loads and stores: a plain
 * streaming copy (nontemporal != 0: non-temporal loads and stores).
 *
 * All pointers are device pointers owned by the caller; rows[] is int64 in
 * [0, num_rows); row_bytes is a multiple of 16 between 16 and 1024. Work is
 * enqueued on hip_stream (NULL = the null stream). Returns 0, or a nonzero
 * status (2: a size out of range, 6: a NULL pointer, 8: a HIP error) with a
 * message for sdm_ceiling_last_error() on the calling thread.
 */
#ifndef SDM_CEILING_H
#define SDM_CEILING_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum { SDM_CEIL_READ = 0, SDM_CEIL_STASH = 1, SDM_CEIL_RMW = 2, SDM_CEIL_MIX = 3 };

int sdm_ceiling_rows(int mode, void* bank, int64_t num_rows, int64_t row_bytes, const int64_t* rows, int64_t n,
                     void* stash, uint32_t* sink, void* hip_stream);

/* Words the sink of SDM_CEIL_READ and SDM_CEIL_MIX must hold (one per thread of
   the largest grid a launch uses). */
int64_t sdm_ceiling_sink_words(void);

int sdm_ceiling_copy(void* dst, const void* src, int64_t bytes, int nontemporal, void* hip_stream);

const char* sdm_ceiling_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* SDM_CEILING_H */
