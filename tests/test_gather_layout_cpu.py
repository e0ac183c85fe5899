"""The gather kernels' index arithmetic, restated and checked on the CPU: every
mapping from a workgroup or lane group to its work is a bijection onto the work,
and the pair layout's grid holds every unit any liveness can give. Each function
below restates one formula of sparse_delta_rule_amd/csrc/sdm_gather.hip (named in
its docstring); the constants are read from that source."""

import os
import re

import numpy as np
import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = open(os.path.join(ROOT, "sparse_delta_rule_amd", "csrc", "sdm_gather.hip")).read()


def _const(name):
    return int(re.search(rf"constexpr int {name} = (\d+);", SRC).group(1))


THREADS, PAD_PAIRS, FB = _const("kThreads"), _const("kPadPairs"), _const("kFB")


def cdiv(a, b):
    return -(-a // b)


def xcd_share(i, n):
    """sdm_gather_kernel's token order: workgroup i (run on XCD i mod 8) takes a pair
    of a contiguous eighth of the n (token block, slice) pairs, each XCD walking its
    eighth from its own starting point."""
    q, r, x, k = n // 8, n % 8, i % 8, i // 8
    sz = q + (1 if x < r else 0)
    return x * q + min(x, r) + (k + x * (sz // 8 + 1)) % sz


@pytest.mark.parametrize("n", list(range(1, 70)) + [255, 256, 257, 4096, 4097, 8191])
def test_xcd_share_is_a_bijection(n):
    assert sorted(xcd_share(i, n) for i in range(n)) == list(range(n))


def test_xcd_walks_at_equal_progress_are_not_a_power_of_two_apart():
    # c3: 4096 token blocks of 8 tokens; the eight XCDs' blocks at the same step of
    # their walks (the stash rows they store at about the same time)
    n = 4096
    for k in range(0, n // 8, 37):
        pos = [xcd_share(x + 8 * k, n) for x in range(8)]
        for a in range(8):
            for b in range(a + 1, 8):
                gap = abs(pos[a] - pos[b])
                assert gap & (gap - 1) != 0, (k, a, b, gap)


def test_xcd_share_gives_each_xcd_a_contiguous_run():
    n = 1000
    for x in range(8):
        got = sorted(xcd_share(i, n) for i in range(x, n, 8))
        assert got == list(range(got[0], got[0] + len(got)))


def operand_pair(i, run):
    """sdm_gather_pair_kernel: live pair index -> (token-slice index, operand), operand 0's
    run of indices first."""
    op = 1 if i >= run else 0
    return (i - run if op else i), op


@pytest.mark.parametrize("gpw", [1, 2, 4])
@pytest.mark.parametrize("live_ks", [0, 1, 3, 4, 5, 63, 64, 65, 1000])
def test_operand_pairs_cover_each_pair_once_with_one_operand_per_wavefront(gpw, live_ks):
    run = cdiv(live_ks, gpw) * gpw
    live_pairs = 2 * run
    seen = [operand_pair(i, run) for i in range(live_pairs)]
    named = [s for s in seen if s[0] < live_ks]
    assert sorted(named) == sorted((k, op) for k in range(live_ks) for op in (0, 1))
    for w0 in range(0, live_pairs, gpw):  # a wavefront's groups: gpw consecutive indices
        assert len({seen[i][1] for i in range(w0, w0 + gpw)}) == 1


@pytest.mark.parametrize("gpw", [1, 2, 4])
def test_operand_pairs_never_hold_one_token_of_both_operands_in_a_window(gpw):
    # operand-major: a window of consecutive indices (the wavefronts in flight) shorter
    # than one operand's run never holds one token's pairs of both operands
    live_ks = 5000
    run = cdiv(live_ks, gpw) * gpw
    window = 1024
    for w0 in range(0, 2 * run - window, 97):
        got = [operand_pair(i, run) for i in range(w0, w0 + window)]
        assert not {k for k, op in got if op == 0} & {k for k, op in got if op == 1}, w0


def pair_units(tokens, live, slices, nops, gpw):
    """sdm_gather_pair_kernel: live pairs (whole runs for two operands) plus runs of
    kPadPairs padding pairs."""
    live_ks = live * slices
    live_pairs = 2 * cdiv(live_ks, gpw) * gpw if nops == 2 else live_ks
    return live_pairs + cdiv((tokens - live) * nops * slices, PAD_PAIRS)


def pair_grid_units(tokens, slices, nops, lpr):
    """launch_pair_lpr: the grid, in lane-group units."""
    groups, gpw, ks = THREADS // lpr, 64 // lpr, tokens * slices
    pairs = cdiv(ks, gpw) * 2 * gpw if nops == 2 else ks
    return cdiv(pairs + gpw, groups) * groups


def test_the_restated_formulas_are_the_kernels():
    """Each restated formula, as it stands in the kernel source."""
    for line in ("const int64_t blocks = (pairs + gpw + groups - 1) / groups;",
                 "const int64_t live_run = (live_ks + gpw - 1) / gpw * gpw;",
                 "const int64_t live_pairs = NOPS == 2 ? 2 * live_run : live_ks;",
                 "pad_runs = (pad_pairs + kPadPairs - 1) / kPadPairs;",
                 "const int64_t q = n / 8, r = n % 8, x = i % 8, k = i / 8;",
                 "const int64_t sz = q + (x < r ? 1 : 0);",
                 "const int64_t j = x * q + (x < r ? x : r) + (k + x * (sz / 8 + 1)) % sz;",
                 "op = i >= run ? 1 : 0;",
                 "return op ? i - run : i;"):
        assert line in SRC, line


@pytest.mark.parametrize("nops", [1, 2])
@pytest.mark.parametrize("slices", [1, 2, 3])
@pytest.mark.parametrize("lpr", [16, 32, 64])
def test_pair_grid_holds_every_liveness(nops, slices, lpr):
    gpw = 64 // lpr
    for tokens in list(range(1, 300)) + [32767, 32768]:
        cap = pair_grid_units(tokens, slices, nops, lpr)
        lives = range(tokens + 1) if tokens < 300 else list(range(60)) + list(range(tokens - 60, tokens + 1))
        for live in lives:
            assert pair_units(tokens, live, slices, nops, gpw) <= cap, (tokens, live)


def test_pair_batches_fit_a_group():
    # lane l of a group (16 lanes or more) loads entry l mod kFB of each batch: a
    # batch fits the smallest group
    assert 1 <= FB <= 16 and 16 % FB == 0
    assert re.search(r"p\.lpr >= 16 &&", SRC), "the pair layout takes groups of 16 lanes or more"


class LiveMap:
    """LiveMap: the live and padding tokens of a launch from its per-chunk counts
    (live_at, a bisection, is the reference that group_live_at is checked against)."""

    def __init__(self, counts, chunk):
        self.chunk = chunk
        self.pref = np.concatenate([[0], np.cumsum(np.clip(counts, 0, chunk))])
        self.chunks = len(counts)

    def live_at(self, j):
        lo, hi = 0, self.chunks - 1
        while lo < hi:
            mid = (lo + hi + 1) // 2
            if self.pref[mid] <= j:
                lo = mid
            else:
                hi = mid - 1
        return lo * self.chunk + (j - self.pref[lo])

    def pad_token(self, j):
        lo, hi = 0, self.chunks - 1
        while lo < hi:
            mid = (lo + hi + 1) // 2
            if mid * self.chunk - self.pref[mid] <= j:
                lo = mid
            else:
                hi = mid - 1
        c = lo
        return c * self.chunk + (self.pref[c + 1] - self.pref[c]) + (j - (c * self.chunk - self.pref[c]))


@pytest.mark.parametrize("seed", range(6))
def test_live_map_lists_the_live_and_the_padding_tokens(seed):
    rng = np.random.default_rng(seed)
    chunk = int(rng.integers(1, 70))
    chunks = int(rng.integers(1, 40))
    counts = rng.integers(-3, chunk + 4, chunks)  # out-of-range counts are clamped
    m = LiveMap(counts, chunk)
    t = np.arange(chunks * chunk)
    live = t % chunk < np.clip(counts, 0, chunk)[t // chunk]
    assert [m.live_at(j) for j in range(int(m.pref[-1]))] == list(t[live])
    assert [m.pad_token(j) for j in range(chunks * chunk - int(m.pref[-1]))] == list(t[~live])


def wave_inclusive_sum(x):
    """wave_inclusive_sum: DPP row_shr 1, 2, 4, 8 within rows of 16 lanes (a source
    outside the row gives 0), then the earlier rows' totals from lanes 15, 31, 47."""
    x = list(x)
    for d in (1, 2, 4, 8):
        x = [x[i] + (x[i - d] if i % 16 >= d else 0) for i in range(64)]
    r0 = x[15]
    r1 = r0 + x[31]
    r2 = r1 + x[47]
    return [x[i] + (0, r0, r1, r2)[i // 16] for i in range(64)]


def test_wave_inclusive_sum_is_the_prefix_sum():
    rng = np.random.default_rng(5)
    for _ in range(200):
        x = rng.integers(0, 1 << 16, 64).tolist()
        assert wave_inclusive_sum(x) == np.cumsum(x).tolist()
    assert wave_inclusive_sum([1] * 64) == list(range(1, 65))


def group_live_at(pref, chunks, chunk, j, lpr):
    """group_live_at: the group's lanes split the remaining chunks into lpr parts a
    step; the count of lanes whose part starts at or below j names the part."""
    lo, n = 0, chunks
    while n > 1:
        step = -(-n // lpr)
        passed = [lo + (lane + 1) * step < chunks and pref[lo + (lane + 1) * step] <= j for lane in range(lpr)]
        assert passed == sorted(passed, reverse=True)  # lanes 0 .. count - 1 pass
        lo += sum(passed) * step
        n = step
    return lo * chunk + (j - pref[lo])


@pytest.mark.parametrize("lpr", [16, 32, 64])
def test_group_live_at_is_the_live_token_map(lpr):
    rng = np.random.default_rng(lpr)
    chunk = 64
    shapes = [1, 2, 3, 15, 16, 17, 63, 64, 65, 255, 256, 257, 512, 1000, 4096]
    for chunks in shapes:
        for kind in ("uniform", "sparse", "ones", "full"):
            if kind == "uniform":
                counts = rng.integers(0, chunk + 1, chunks)
            elif kind == "sparse":  # mostly empty chunks: long runs of equal prefix values
                counts = np.where(rng.random(chunks) < 0.05, rng.integers(1, chunk + 1, chunks), 0)
            elif kind == "ones":
                counts = np.ones(chunks, dtype=np.int64)
            else:
                counts = np.full(chunks, chunk)
            lm = LiveMap(counts, chunk)
            live = int(lm.pref[-1])
            js = range(live) if live <= 3000 else sorted(set(rng.integers(0, live, 3000).tolist()) | {0, live - 1})
            for j in js:
                assert group_live_at(lm.pref, chunks, chunk, j, lpr) == lm.live_at(j), (chunks, kind, j)


def test_the_scan_and_search_restatements_are_the_kernels():
    for line in ("x += __builtin_amdgcn_update_dpp(0, x, 0x111, 0xf, 0xf, false);  // row_shr:1",
                 "x += __builtin_amdgcn_update_dpp(0, x, 0x112, 0xf, 0xf, false);  // row_shr:2",
                 "x += __builtin_amdgcn_update_dpp(0, x, 0x114, 0xf, 0xf, false);  // row_shr:4",
                 "x += __builtin_amdgcn_update_dpp(0, x, 0x118, 0xf, 0xf, false);  // row_shr:8",
                 "return x + (row == 0 ? 0 : row == 1 ? r0 : row == 2 ? r1 : r2);",
                 "const int32_t step = (n + LPR - 1) / LPR;",
                 "const int32_t probe = lo + (lane + 1) * step;",
                 "const bool pass = probe < m.chunks && m.pref[probe] <= j;",
                 "lo += int32_t(__popcll(b)) * step;",
                 "return int64_t(lo) * m.chunk + (j - m.pref[lo]);"):
        assert line in SRC, line
    assert SRC.count("wave_inclusive_sum(run)") == 2  # both kernels' scans
    assert "__shfl_up" not in SRC
