"""Mutation check of the oracle's pins (CPU only).

Each entry below plants one plausible mistake in a copy of oracle/oracle.c (a
wrong rounding, a dropped term, a wrong order, sign, index, offset or
modulus), builds that copy, and runs the pin tests of tests/test_oracle.py
that concern the mutated function against it.  Every planted mistake must
make at least one of those pins fail; a mistake that survives means the
pins do not tie the oracle to the pages there.  The shipped oracle itself is
not touched.
"""
import concurrent.futures
import os
import subprocess
import sys

import oracle

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

BF16 = "bf16"
ONE = "1stage"
TWO = "2stage and not fused"
FUSED = "fused and not 2stage and not lamport"
LL = "ll_pack or wire or round_trip or decode or unaligned"
LAMPORT = "lamport"
FUSED2 = "fused_2stage"
FIFO = "fifo"

# (name, text in oracle.c (must occur exactly once), replacement, pin selector)
MUTATIONS = [
    ("bf16: ties not to even", "u += 0x7FFFu + lsb;", "u += 0x7FFFu;", BF16),
    ("bf16: truncation", "u += 0x7FFFu + lsb;", "u += 0u * lsb;", BF16),
    ("bf16: ties away from zero", "u += 0x7FFFu + lsb;", "u += 0x8000u + 0u * lsb;", BF16),
    ("bf16: NaN not kept quiet",
     "if ((u & 0x7F800000u) == 0x7F800000u && (u & 0x007FFFFFu) != 0)", "if (0)", BF16),
    ("bf16 from f64: one bit too few", "int qexp = e - 8;", "int qexp = e - 7;", BF16),
    ("bf16 from f64: floor instead of nearest",
     "double q = nearbyint(ldexp(a, -qexp));", "double q = floor(ldexp(a, -qexp));", BF16),
    ("bf16 from f64: denormal spacing",
     "if (qexp < -133)\n        qexp = -133;", "if (qexp < -126)\n        qexp = -126;", BF16),
    ("1stage: accumulator from +0.0",
     "float acc = orc_bf16_to_f32(x[0][j]);\n        for (int r = 1; r < W; ++r)\n"
     "            acc = acc + orc_bf16_to_f32(x[r][j]);\n        out[j]",
     "float acc = 0.0f;\n        for (int r = 0; r < W; ++r)\n"
     "            acc = acc + orc_bf16_to_f32(x[r][j]);\n        out[j]", ONE),
    ("1stage: reversed order",
     "float acc = orc_bf16_to_f32(x[0][j]);\n        for (int r = 1; r < W; ++r)\n"
     "            acc = acc + orc_bf16_to_f32(x[r][j]);\n        out[j]",
     "float acc = orc_bf16_to_f32(x[W - 1][j]);\n        for (int r = W - 2; r >= 0; --r)\n"
     "            acc = acc + orc_bf16_to_f32(x[r][j]);\n        out[j]", ONE),
    ("1stage: last rank dropped",
     "float acc = orc_bf16_to_f32(x[0][j]);\n        for (int r = 1; r < W; ++r)\n"
     "            acc = acc + orc_bf16_to_f32(x[r][j]);\n        out[j]",
     "float acc = orc_bf16_to_f32(x[0][j]);\n        for (int r = 1; r < W - 1; ++r)\n"
     "            acc = acc + orc_bf16_to_f32(x[r][j]);\n        out[j]", ONE),
    ("1stage: rounding every partial sum",
     "for (int r = 1; r < W; ++r)\n            acc = acc + orc_bf16_to_f32(x[r][j]);\n"
     "        out[j]",
     "for (int r = 1; r < W; ++r)\n            acc = orc_bf16_to_f32(orc_bf16_rne("
     "acc + orc_bf16_to_f32(x[r][j])));\n        out[j]", ONE),
    ("2stage: no rotation",
     "int r = rank_order ? i : (s + i) % W;", "int r = i; (void)rank_order;", TWO),
    ("2stage: rotation the wrong way",
     "int r = rank_order ? i : (s + i) % W;", "int r = rank_order ? i : (s - i + W) % W;", TWO),
    ("2stage: owner's value not first",
     "int first = rank_order ? 0 : s;", "int first = 0;", TWO),
    ("2stage: remainder dropped",
     "*last = (s == W - 1) ? packs : *first + part;", "*last = *first + part;", TWO),
    ("fused: eps outside the root",
     "double rms = 1.0 / sqrt(ss / (double)N + eps);",
     "double rms = 1.0 / (sqrt(ss / (double)N) + eps);", FUSED),
    ("fused: mean over N - 1",
     "double rms = 1.0 / sqrt(ss / (double)N + eps);",
     "double rms = 1.0 / sqrt(ss / (double)(N - 1) + eps);", FUSED),
    ("fused: residual not added",
     "float h = a + orc_bf16_to_f32(residual[row + j]);", "float h = a;", FUSED),
    ("fused: weight not applied",
     "* rms) * (double)orc_bf16_to_f32(weight[j]);", "* rms) * 1.0;", FUSED),
    ("fused: weight reversed",
     "* rms) * (double)orc_bf16_to_f32(weight[j]);",
     "* rms) * (double)orc_bf16_to_f32(weight[N - 1 - j]);", FUSED),
    ("fused: rms not inverted",
     "double rms = 1.0 / sqrt(ss / (double)N + eps);",
     "double rms = sqrt(ss / (double)N + eps);", FUSED),
    ("LL: flag = step", "uint32_t flag = (uint32_t)(k + 1);", "uint32_t flag = (uint32_t)k;", LL),
    ("LL: data halves swapped",
     "put_u32le(line + 0, get_u32le(data));     /* data1 */",
     "put_u32le(line + 0, get_u32le(data + 4)); /* data1 */", LL),
    ("LL: slot modulo 7",
     "return (int64_t)(k % 8u) * step_lines + i % step_lines;",
     "return (int64_t)(k % 7u) * step_lines + i % step_lines;", LL),
    ("LL: one flag checked", "if (f1 != expect || f2 != expect) {", "if (f1 != expect) {", LL),
    ("LL: last partial line dropped",
     "int64_t orc_ll_lines(int64_t n) { return (4 * n + 7) / 8; }",
     "int64_t orc_ll_lines(int64_t n) { return (4 * n) / 8; }", LL),
    ("LL128: flag in word 14", "put_u64le(line + 120, k + 1);\n    }",
     "put_u64le(line + 112, k + 1);\n    }", LL),
    ("LL128: 128 payload bytes per line",
     "line[b] = payload_byte(src, nbytes, 120 * l + b);",
     "line[b] = payload_byte(src, nbytes, 128 * l + b);", LL),
    ("LL128: flag not checked", "if (get_u64le(line + 120) != k + 1) {", "if (0) {", LL),
    ("Lamport: high half not scrubbed", "if (hi == 0x8000u)\n        hi = 0;", "", LAMPORT),
    ("Lamport: halves swapped",
     "return (uint32_t)lo | ((uint32_t)hi << 16);",
     "return (uint32_t)hi | ((uint32_t)lo << 16);", LAMPORT),
    ("Lamport: two regions",
     "const int64_t region = (int64_t)(flag % 3u);\n    for (int p = 0; p < W; ++p) {",
     "const int64_t region = (int64_t)(flag % 2u);\n    for (int p = 0; p < W; ++p) {", LAMPORT),
    ("Lamport: push into the reader's slot",
     "uint32_t *slot = comms[p] + (region * W + rank) * words;",
     "uint32_t *slot = comms[p] + (region * W + p) * words;", LAMPORT),
    ("Lamport: reset of the wrong region",
     "const int64_t stale = (region + 2) % 3;",
     "const int64_t stale = (region + 1) % 3;", LAMPORT),
    ("Lamport: bad words instead of chunks", "bad += any;", "bad += 4 * any;", LAMPORT),
    ("Lamport: flag wraps at 2^32",
     "return flag + 1u >= ORC_LAMPORT_FLAG_PERIOD ? 0u : flag + 1u;", "return flag + 1u;",
     LAMPORT),
    ("Lamport: reader takes flags past the period",
     "if (flag >= ORC_LAMPORT_FLAG_PERIOD)\n        return -1;", "", LAMPORT),
    ("two-shot: no rotation",
     "xs[i] = x[rank_order ? i : (s + i) % W] + m0 * N;", "xs[i] = x[i] + m0 * N;", FUSED2),
    ("two-shot: no row offset",
     "xs[i] = x[rank_order ? i : (s + i) % W] + m0 * N;",
     "xs[i] = x[rank_order ? i : (s + i) % W];", FUSED2),
    ("two-shot: remainder rows dropped",
     "*last = (s == W - 1) ? M : *first + part;", "*last = *first + part;", FUSED2),
    ("two-shot: staged outputs swapped",
     "residual_out[m0 * N + q] = stage[q];\n            norm_out[m0 * N + q] = stage[rows * N + q];",
     "norm_out[m0 * N + q] = stage[q];\n            residual_out[m0 * N + q] = stage[rows * N + q];",
     FUSED2),
    ("stream: local addend ignored", "out[e] = local ? local[e] + v : v;",
     "out[e] = v + 0.0f * (local ? local[e] : 0.0f);", FIFO),
    ("stream: global step numbers",
     "const uint64_t k = first_step + (uint64_t)(g - s0);",
     "const uint64_t k = first_step + (uint64_t)g;", FIFO),
    ("stream: LL128 flag in word 14", "put_u64le(slot + 128 * l + 120, k + 1);",
     "put_u64le(slot + 128 * l + 112, k + 1);", FIFO),
    ("stream: LL flag = step",
     "put_u32le(slot + 16 * i + 4, (uint32_t)(k + 1));",
     "put_u32le(slot + 16 * i + 4, (uint32_t)k);", FIFO),
    ("stream: channels take ceil(T / channels) steps each",
     "const int64_t s0 = (int64_t)c * T / channels, s1 = (int64_t)(c + 1) * T / channels;",
     "const int64_t cs = (T + channels - 1) / channels;\n"
     "        const int64_t s0 = c * cs < T ? c * cs : T, s1 = (c + 1) * cs < T ? (c + 1) * cs : T;",
     FIFO),
]


def _source():
    with open(oracle.SRC) as f:
        return f.read()


def test_every_mutation_applies_exactly_once():
    src = _source()
    for name, old, _new, _sel in MUTATIONS:
        assert src.count(old) == 1, f"{name}: the text to mutate occurs {src.count(old)} times"


def _run_one(args):
    idx, (name, old, new, sel), src, tmpdir = args
    mutated = src.replace(old, new, 1)
    c_path = os.path.join(tmpdir, f"m{idx}.c")
    so_path = os.path.join(tmpdir, f"liboracle_m{idx}.so")
    with open(c_path, "w") as f:
        f.write(mutated)
    b = subprocess.run(["gcc", *oracle.CFLAGS, "-o", so_path, c_path, "-lm"],
                       capture_output=True, text=True)
    if b.returncode != 0:
        return name, "build failed: " + b.stderr[-500:]
    env = dict(os.environ)
    env["ORACLE_LIB"] = so_path
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-x", "-p", "no:cacheprovider",
                        "-k", sel, os.path.join(ROOT, "tests", "test_oracle.py")],
                       cwd=ROOT, env=env, capture_output=True, text=True, timeout=600)
    if r.returncode == 1:          # a pin failed: the mutation is caught
        return name, None
    if r.returncode == 0:
        return name, "survived"
    return name, f"pytest ended with status {r.returncode}: " + (r.stdout + r.stderr)[-500:]


def test_every_planted_mistake_fails_a_pin(tmp_path):
    src = _source()
    jobs = [(i, m, src, str(tmp_path)) for i, m in enumerate(MUTATIONS)]
    workers = max(1, min(4, os.cpu_count() or 1))
    with concurrent.futures.ThreadPoolExecutor(workers) as pool:
        results = list(pool.map(_run_one, jobs))
    bad = [f"{name}: {why}" for name, why in results if why is not None]
    assert not bad, "mutations not caught by the pins:\n" + "\n".join(bad)
