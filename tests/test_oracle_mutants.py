"""The oracle's pins against deliberately broken copies of the oracle.

Each mutant is sdm_oracle.c with one plausible mistake planted (a dropped term,
a wrong sign or index, a skipped rounding, another order, an off-by-one in the
padding or the stash); it is compiled into a temporary directory and the pin
tests (tests/test_oracle_*.py) run against it through SDM_ORACLE_LIBRARY. Every
mutant must fail at least one pin, and the unmodified source, built the same
way, must pass them all. Mistakes are planted only in copies of the oracle, on
the CPU; nothing here touches the HIP library.
"""

import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "oracle", "sdm_oracle.c")
PINS = ["tests/test_oracle_decode.py", "tests/test_oracle_gather.py", "tests/test_oracle_bf16.py"]

# The float32 path's delta_v line, with the line before it (the float64 brute
# force has the same delta_v line).
DV32 = "float vc = round_to_bank(v[s * hd + c], bank_bf16);\n            dv[c] = b * (vc - retrieved);"

# name: [(text in sdm_oracle.c, replacement), ...]; each text occurs exactly once.
MUTANTS = {
    "decode: no decay": [("d[w] = (float)exp((double)g[s * G + (G == 1 ? 0 : w)]);", "d[w] = 1.0f;")],
    "decode: gate of the stream for every write": [
        ("d[w] = (float)exp((double)g[s * G + (G == 1 ? 0 : w)]);", "d[w] = (float)exp((double)g[s * G]);")],
    "decode: delta sign flipped": [(DV32, DV32.replace("(vc - retrieved)", "(retrieved - vc)"))],
    "decode: beta dropped": [(DV32, DV32.replace("b * (vc - retrieved);", "(vc - retrieved); (void)b;"))],
    "decode: delta_v one rounding": [
        (DV32, DV32.replace("b * (vc - retrieved);", "(float)((double)b * ((double)vc - (double)retrieved));"))],
    "decode: k_val not rounded to the bank dtype": [
        ("kv[w] = round_to_bank(k_val[s * W + w], bank_bf16);", "kv[w] = k_val[s * W + w];")],
    "decode: q_val not rounded to the bank dtype": [
        ("qv[r] = round_to_bank(q_val[s * R + r], bank_bf16);", "qv[r] = q_val[s * R + r];")],
    "decode: v not rounded to the bank dtype": [
        ("float vc = round_to_bank(v[s * hd + c], bank_bf16);", "float vc = v[s * hd + c];")],
    "decode: unfused update": [("fmaf(kv[w], dv[c], decayed)", "kv[w] * dv[c] + decayed")],
    "decode: k_val times a rounded d*row": [
        ("coef[w] = kv[w] * d[w];", "coef[w] = kv[w];"),
        ("for (int64_t c = 0; c < hd; ++c) rows[w * hd + c] = bank_load(bank, bank_bf16, hd, ks[w], c);",
         "for (int64_t c = 0; c < hd; ++c) rows[w * hd + c] = bank_load(bank, bank_bf16, hd, ks[w], c) * d[w];")],
    "decode: writes dropped (reads see the old rows)": [
        ("bank_store_f32(bank, bank_bf16, hd, ks[w], c, fmaf(kv[w], dv[c], decayed));", "(void)decayed;")],
    "decode: column stride 1 in the retrieval": [
        ("grouped_dot(coef, rows + c, hd, W, groups)", "grouped_dot(coef, rows + c, 1, W, groups)")],
    "sums: group order reversed": [
        ("for (int g = 0; g < groups; ++g) {\n        float p = 0.0f;",
         "for (int g = groups - 1; g >= 0; --g) {\n        float p = 0.0f;")],
    "sums: descending chains": [
        ("for (int i = g; i < n; i += groups) p = fmaf(a[i], x[(int64_t)i * stride], p);",
         "for (int i = g + (n - 1 - g) / groups * groups; i >= g; i -= groups) "
         "p = fmaf(a[i], x[(int64_t)i * stride], p);")],
    "bf16: truncation": [
        ("if (low > 0x8000u || (low == 0x8000u && (keep & 1u))) keep += 1u;", "(void)low;")],
    "bf16: ties rounded up": [("(low == 0x8000u && (keep & 1u))", "(low == 0x8000u)")],
    "bf16: NaN not kept quiet": [("return (uint16_t)((u >> 16) | 0x0040u);", "return (uint16_t)(u >> 16);")],
    "gather: padding test shifted": [("return (t % chunk) < lim;", "return (t % chunk) <= lim;")],
    "gather: stash copies the next entry's row": [
        ("memcpy(row, (const unsigned char*)bank + (size_t)(idx0[t * width0 + n] * hd * es), (size_t)(hd * es));",
         "memcpy(row, (const unsigned char*)bank + (size_t)(idx0[t * width0 + (n + 1) % width0] * hd * es), "
         "(size_t)(hd * es));")],
    "gather: weights of the next token": [
        ("grouped_dot(w + t * width, rows + c, hd, width, groups)",
         "grouped_dot(w + (t + 1) % tokens * width, rows + c, hd, width, groups)")],
    "gather: compact stash one position on": [
        ("memcpy((unsigned char*)stash + (size_t)((k * crow + p) * hd * es),",
         "memcpy((unsigned char*)stash + (size_t)((k * crow + (p + 1) % crow) * hd * es),")],
    "gather: padding outputs -0": [("for (int64_t c = 0; c < hd; ++c) out[t * hd + c] = 0.0f;",
                                    "for (int64_t c = 0; c < hd; ++c) out[t * hd + c] = -0.0f;")],
    "gather: padding stash rows not zero": [("else memset(row, 0, (size_t)(hd * es));",
                                             "else memset(row, 0xff, (size_t)(hd * es));")],
    "compact stash: padding tokens stored too": [
        ("            if (!token_live(t, chunk, valid, chunk_valid)) continue;\n            for (int n = 0; n < width0;",
         "            for (int n = 0; n < width0;")],
    "brute force: decode decay dropped": [("d[w] = exp((double)g[s * G + (G == 1 ? 0 : w)]);", "d[w] = 1.0;")],
    "brute force: decode delta sign flipped": [("dv[c] = b * (vc - retrieved);\n            dvmag",
                                                "dv[c] = b * (retrieved - vc);\n            dvmag")],
    "brute force: gather weight dropped": [
        ("double x = (double)w[t * width + n] * (double)bank_load(bank, bank_bf16, hd, idx[t * width + n], c);",
         "double x = (double)bank_load(bank, bank_bf16, hd, idx[t * width + n], c);")],
}


def _build(src_text: str, out_dir: str) -> str:
    c = os.path.join(out_dir, "sdm_oracle.c")
    so = os.path.join(out_dir, "libsdm_oracle.so")
    with open(c, "w") as f:
        f.write(src_text)
    subprocess.run(["gcc", "-O2", "-ffp-contract=off", "-fno-fast-math", "-std=c11", "-fPIC", "-shared", "-o", so,
                    c, "-lm"], check=True, capture_output=True)
    return so


def _pins_pass(so: str) -> bool:
    env = dict(os.environ, SDM_ORACLE_LIBRARY=so)
    r = subprocess.run([sys.executable, "-m", "pytest", *PINS, "-x", "-q", "-p", "no:cacheprovider", "-m", "not gpu"],
                       cwd=ROOT, env=env, capture_output=True, text=True, timeout=600)
    return r.returncode == 0


def _mutated(src: str, edits) -> str:
    for old, new in edits:
        assert src.count(old) == 1, f"mutation text occurs {src.count(old)} times: {old[:60]!r}"
        src = src.replace(old, new)
    return src


def test_every_mutant_fails_a_pin(tmp_path):
    with open(SRC) as f:
        src = f.read()
    jobs = {"unmodified": src}
    for name, edits in MUTANTS.items():
        jobs[name] = _mutated(src, edits)
    dirs = {}
    for i, (name, text) in enumerate(jobs.items()):
        d = tmp_path / f"m{i}"
        d.mkdir()
        dirs[name] = _build(text, str(d))
    workers = max(1, min(8, len(os.sched_getaffinity(0))))
    with ThreadPoolExecutor(max_workers=workers) as ex:
        passed = dict(zip(dirs, ex.map(_pins_pass, dirs.values())))
    assert passed["unmodified"], "the pins fail on the unmodified oracle built this way"
    survivors = [name for name, ok in passed.items() if name != "unmodified" and ok]
    assert not survivors, f"mutants that pass every pin: {survivors}"
