"""The pins are strong enough to catch plausible mistakes in the oracle.

Each case below plants one mistake in a copy of oracle/qkv_oracle.c (on the
CPU, in a temporary directory), builds it, points the oracle module at it and
runs the CPU pin tests until one fails.  Every planted mistake must be caught;
the unmodified source must pass the same battery."""
import ctypes
import inspect
import os
import subprocess
import sys
import tempfile
from concurrent.futures import ThreadPoolExecutor
from pathlib import Path

import pytest

import oracle
import test_oracle_formats as T_FMT
import test_oracle_mxfp8 as T_MX
import test_oracle_op as T_OP
import test_oracle_row as T_ROW
import test_oracle_store_gather as T_SG

SRC = os.path.join(os.path.dirname(oracle.__file__), "qkv_oracle.c")

# Pin tests in increasing cost, so that a mutant is usually caught within
# milliseconds.  The slow strided cross-checks against torch's casts come last.
SLOW = {"test_bf16_matches_torch_cast_on_strided_patterns"}
# The exhaustive sweeps (billions of patterns) run once, directly, in
# test_oracle_formats.py; the battery leaves them out.
EXHAUSTIVE = {"test_e4m3_matches_torch_cast_on_every_in_range_pattern",
              "test_ue8m0_definition_on_every_positive_pattern",
              "test_ue8m0_byte_on_every_pattern"}


def _expand(name, fn):
    """The test as zero-argument calls, one per parametrize case."""
    marks = [m for m in getattr(fn, "pytestmark", []) if m.name == "parametrize"]
    if not marks:
        return [(name, fn)]
    argnames, values = marks[0].args[0], marks[0].args[1]
    single = "," not in argnames if isinstance(argnames, str) else len(argnames) == 1
    calls = []
    for v in values:
        args = (v,) if single else tuple(v)
        calls.append(("%s[%s]" % (name, v), lambda fn=fn, args=args: fn(*args)))
    return calls


def battery():
    tests = []
    for mod in (T_FMT, T_ROW, T_OP, T_SG, T_MX):
        for name, fn in inspect.getmembers(mod, inspect.isfunction):
            if name.startswith("test_") and fn.__module__ == mod.__name__ and name not in EXHAUSTIVE:
                for n, call in _expand(name, fn):
                    tests.append((name in SLOW, n, call))
    tests.sort(key=lambda t: t[0])
    return [(n, f) for _, n, f in tests]


# (name, text in the source, replacement): one plausible mistake each.
MUTANTS = [
    ("bf16 ties to odd", "r = ((lo >> 16) & 1u) ? hi : lo;", "r = ((lo >> 16) & 1u) ? lo : hi;"),
    ("bf16 truncates", "if (below < above)\n        r = lo;", "if (1)\n        r = lo;"),
    ("e4m3 bias 8 (fnuz)", "int biased = ex + 7;", "int biased = ex + 8;"),
    ("e4m3 truncates", "double q = nearbyint((2.0 * f - 1.0) * 8.0);",
     "double q = floor((2.0 * f - 1.0) * 8.0);"),
    ("e4m3 subnormal step 2^-10", "double m = nearbyint(a * 512.0);", "double m = nearbyint(a * 1024.0);"),
    ("e4m3 saturates at 240", "if (biased > 15 || (biased == 15 && q == 7.0))",
     "if (biased > 14 || (biased == 14 && q == 7.0))"),
    ("e4m3 decode bias", "v = ldexp(1.0 + m / 8.0, e - 7);", "v = ldexp(1.0 + m / 8.0, e - 8);"),
    ("ue8m0 boundary off by one", "while (a <= ldexp(448.0, e - 1))", "while (a < ldexp(448.0, e - 1))"),
    ("ue8m0 against 256", "while (a > ldexp(448.0, e))\n        e += 1;\n    while (a <= ldexp(448.0, e - 1))",
     "while (a > ldexp(256.0, e))\n        e += 1;\n    while (a <= ldexp(256.0, e - 1))"),
    ("ue8m0 lower clamp -126", "if (e < -127)\n        e = -127;", "if (e < -126)\n        e = -126;"),
    ("sum of squares drops a term",
     "for (int l = 0; l < 64; ++l) {\n        float acc = 0.0f;\n        for (int k = 0; k < 8; ++k) {",
     "for (int l = 0; l < 64; ++l) {\n        float acc = 0.0f;\n        for (int k = 0; k < 7; ++k) {"),
    ("sum of squares sequential",
     "for (int n = 64; n > 1; n /= 2)\n        for (int i = 0; i < n / 2; ++i)\n            c[i] = c[2 * i] + c[2 * i + 1];",
     "for (int i = 1; i < 64; ++i)\n        c[0] = c[0] + c[i];"),
    ("sum of squares pairs (l, l+32) first",
     "for (int n = 64; n > 1; n /= 2)\n        for (int i = 0; i < n / 2; ++i)\n            c[i] = c[2 * i] + c[2 * i + 1];",
     "for (int n = 64; n > 1; n /= 2)\n        for (int i = 0; i < n / 2; ++i)\n            c[i] = c[i] + c[i + n / 2];"),
    ("mean over 448 dims", "float mean_sq = sum_sq / 512.0f;", "float mean_sq = sum_sq / 448.0f;"),
    ("eps outside the root", "float v = mean_sq + eps;\n    float r = sqrtf(v);\n    return 1.0f / r;",
     "float v = mean_sq;\n    float r = sqrtf(v) + eps;\n    return 1.0f / r;"),
    ("gemma 1+w", "y[j] = w ? t * orc_bf16_to_f32(w[j]) : t;",
     "y[j] = w ? t * (1.0f + orc_bf16_to_f32(w[j])) : t;"),
    ("weight index reversed", "y[j] = w ? t * orc_bf16_to_f32(w[j]) : t;",
     "y[j] = w ? t * orc_bf16_to_f32(w[511 - j]) : t;"),
    ("rope sign", "z[ORC_NOPE_DIM + 2 * i] = fmaf(a, c, -bs);", "z[ORC_NOPE_DIM + 2 * i] = fmaf(a, c, bs);"),
    ("rope cos/sin swapped", "float c = cs[i];\n        float sn = cs[ORC_NPAIR + i];",
     "float sn = cs[i];\n        float c = cs[ORC_NPAIR + i];"),
    ("rope without fma", "z[ORC_NOPE_DIM + 2 * i] = fmaf(a, c, -bs);", "z[ORC_NOPE_DIM + 2 * i] = a * c - bs;"),
    ("rope fma on the sine product", "z[ORC_NOPE_DIM + 2 * i] = fmaf(a, c, -bs);",
     "z[ORC_NOPE_DIM + 2 * i] = fmaf(-b, sn, a * c);"),
    ("rope second output without fma", "z[ORC_NOPE_DIM + 2 * i + 1] = fmaf(a, sn, bc);",
     "z[ORC_NOPE_DIM + 2 * i + 1] = a * sn + bc;"),
    ("rope second output fma on the cosine product", "z[ORC_NOPE_DIM + 2 * i + 1] = fmaf(a, sn, bc);",
     "z[ORC_NOPE_DIM + 2 * i + 1] = fmaf(b, c, a * sn);"),
    ("norm weight before inv", "y[j] = w ? t * orc_bf16_to_f32(w[j]) : t;",
     "y[j] = w ? (orc_bf16_to_f32(x[j]) * orc_bf16_to_f32(w[j])) * inv : t;"),
    ("norm inv times weight first", "y[j] = w ? t * orc_bf16_to_f32(w[j]) : t;",
     "y[j] = w ? orc_bf16_to_f32(x[j]) * (inv * orc_bf16_to_f32(w[j])) : t;"),
    ("rope half-split pairs", "float a = y[ORC_NOPE_DIM + 2 * i];\n        float b = y[ORC_NOPE_DIM + 2 * i + 1];",
     "float a = y[ORC_NOPE_DIM + i];\n        float b = y[ORC_NOPE_DIM + 32 + i];"),
    ("scale byte bias 128", "return (uint8_t)(e + 127);", "return (uint8_t)(e + 128);"),
    ("pad byte not zero", "scale[ORC_NQBLOCK] = 0;", "scale[ORC_NQBLOCK] = 0xff;"),
    ("interleaved slot records", "*data_off = base + s * ORC_SLOT_DATA;", "*data_off = base + s * ORC_SLOT_BYTES;"),
    ("capacity slot written", "if (slot < 0 || block_size <= 0 || slot >= num_blocks * (int64_t)block_size)",
     "if (slot < 0 || block_size <= 0 || slot > num_blocks * (int64_t)block_size)"),
    ("rope bytes big-endian", "data[ORC_NOPE_DIM + 2 * j] = (uint8_t)(h & 0xff);\n        data[ORC_NOPE_DIM + 2 * j + 1] = (uint8_t)(h >> 8);",
     "data[ORC_NOPE_DIM + 2 * j] = (uint8_t)(h >> 8);\n        data[ORC_NOPE_DIM + 2 * j + 1] = (uint8_t)(h & 0xff);"),
    ("quantized from the wrong block", "scale[b] = orc_quant_block(y + b * ORC_QBLOCK, data + b * ORC_QBLOCK);",
     "scale[b] = orc_quant_block(y + (b ^ 1) * ORC_QBLOCK, data + b * ORC_QBLOCK);"),
    ("kv codes from bf16-rounded values", "codes[j] = orc_f32_to_e4m3(y[j] * inv_scale);",
     "codes[j] = orc_f32_to_e4m3(orc_bf16_to_f32(orc_f32_to_bf16(y[j])) * inv_scale);"),
    ("kv amax from bf16-rounded values", "amax = fmaxf(amax, fabsf(y[j]));",
     "amax = fmaxf(amax, fabsf(orc_bf16_to_f32(orc_f32_to_bf16(y[j]))));"),
    ("rope table row of position + 1", "const float *cs = cos_sin + positions[t] * 64;",
     "const float *cs = cos_sin + ((positions[t] + 1) % max_position) * 64;"),
    ("q weight ignored", "orc_row(q_in + row, q_w, eps, cs, y, z, NULL);", "orc_row(q_in + row, NULL, eps, cs, y, z, NULL);"),
    ("q takes the kv weight", "orc_row(q_in + row, q_w, eps, cs, y, z, NULL);",
     "orc_row(q_in + row, kv_w, eps, cs, y, z, NULL);"),
    ("kv weight ignored", "orc_row(kv + t * ORC_HEAD_DIM, kv_w, eps, cs, y, z, NULL);",
     "orc_row(kv + t * ORC_HEAD_DIM, NULL, eps, cs, y, z, NULL);"),
    ("kv row of the next token", "orc_row(kv + t * ORC_HEAD_DIM, kv_w, eps, cs, y, z, NULL);",
     "orc_row(kv + ((t + 1) % num_tokens) * ORC_HEAD_DIM, kv_w, eps, cs, y, z, NULL);"),
    ("inverse root in double", "    float r = sqrtf(v);\n    return 1.0f / r;", "    return (float)(1.0 / sqrt((double)v));"),
    ("eps doubled", "float v = mean_sq + eps;", "float v = mean_sq + 2.0f * eps;"),
    ("mean over 511", "float mean_sq = sum_sq / 512.0f;", "float mean_sq = sum_sq / 511.0f;"),
    ("e4m3 ties away from zero", "double q = nearbyint((2.0 * f - 1.0) * 8.0);", "double q = round((2.0 * f - 1.0) * 8.0);"),
    ("e4m3 subnormal ties away from zero", "double m = nearbyint(a * 512.0);", "double m = round(a * 512.0);"),
    ("only slot -1 skips", "if (slot < 0 || block_size <= 0 || slot >= num_blocks * (int64_t)block_size)",
     "if (slot == -1 || block_size <= 0 || slot >= num_blocks * (int64_t)block_size)"),
    ("scale records reversed", "scale[b] = orc_quant_block(y + b * ORC_QBLOCK, data + b * ORC_QBLOCK);",
     "scale[ORC_NQBLOCK - 1 - b] = orc_quant_block(y + b * ORC_QBLOCK, data + b * ORC_QBLOCK);"),
    ("q output unrotated", "q_out[row + j] = orc_f32_to_bf16(z[j]);", "q_out[row + j] = orc_f32_to_bf16(y[j]);"),
    ("kv rope bytes unrotated", "uint16_t h = orc_f32_to_bf16(z[ORC_NOPE_DIM + j]);\n        data[ORC_NOPE_DIM + 2 * j]",
     "uint16_t h = orc_f32_to_bf16(y[ORC_NOPE_DIM + j]);\n        data[ORC_NOPE_DIM + 2 * j]"),
    ("bf16 store at the fp8 slot stride", "uint8_t *data = cache + slot * 1024;", "uint8_t *data = cache + slot * 584;"),
    ("gather rope from the nope bytes",
     "(uint16_t)(data[ORC_NOPE_DIM + 2 * j] | (data[ORC_NOPE_DIM + 2 * j + 1] << 8)));",
     "(uint16_t)(data[2 * j] | (data[2 * j + 1] << 8)));"),
    ("gather scale of the next block", "(int)scale[j / ORC_QBLOCK] - 127", "(int)scale[(j / ORC_QBLOCK + 1) % 7] - 127"),
    ("cos/sin table interleaved", "float c = cs[i];\n        float sn = cs[ORC_NPAIR + i];",
     "float c = cs[2 * i];\n        float sn = cs[2 * i + 1];"),
    ("rope dims weighted after the rotation",
     "        y[j] = w ? t * orc_bf16_to_f32(w[j]) : t;\n        z[j] = y[j];",
     "        y[j] = (w && j < ORC_NOPE_DIM) ? t * orc_bf16_to_f32(w[j]) : t;\n        z[j] = y[j];"),
    ("bf16 store unrotated", "insert_bf16_slot(z, cache, slot_mapping[t]);", "insert_bf16_slot(y, cache, slot_mapping[t]);"),
    ("gather exponent bias", "(int)scale[j / ORC_QBLOCK] - 127", "(int)scale[j / ORC_QBLOCK] - 128"),
    ("mxfp8 byte of a power of two bumped", "while (b > 0 && a <= ldexp(1.0, b - 1 - 127))  /* the least such b, not below 0 */\n        b -= 1;",
     "while (0)\n        b -= 1;"),
    ("mxfp8 byte rounded down", "b += 127;                                      /* so a <= 2^(b - 127) holds */",
     "b += 126;"),
    ("mxfp8 byte capped at 255", "return b > 254 ? 254u : (uint32_t)b;", "return b > 255 ? 255u : (uint32_t)b;"),
    ("mxfp8 byte negative wraps", "if (b < 0)\n        b = 0;\n    return b > 254", "if (b < -1000)\n        b = 0;\n    return b > 254"),
    ("mxfp8 inverse of 254 kept", "if (byte == 0 || byte >= 254)", "if (byte == 0 || byte >= 255)"),
    ("mxfp8 plain weight", "float g1 = orc_bf16_to_f32(gamma[j]) + 1.0f;", "float g1 = orc_bf16_to_f32(gamma[j]);"),
    ("mxfp8 no bf16 rounding before quant", "normed[j] = orc_bf16_to_f32(orc_f32_to_bf16(t * g1));",
     "normed[j] = t * g1;"),
    ("mxfp8 swizzle row stride", "(row % 32) * 16 + ((row % 128) / 32) * 4", "(row % 32) * 4 + ((row % 128) / 32) * 128"),
    ("mxfp8 padding rows kept", "scale_out[orc_mxfp8_scale_offset(r, b, padded_cols)] = 0;",
     "scale_out[orc_mxfp8_scale_offset(r, b, padded_cols)] = scale_out[orc_mxfp8_scale_offset(r, b, padded_cols)];"),
    ("mxfp8 odd element dropped", "if (nc % 2)\n            c[half] = c[nc - 1];", "if (nc % 2)\n            c[half] = 0.0f;"),
    ("mxfp8 residual ignored", "float sum = orc_bf16_to_f32(xr[j]) + orc_bf16_to_f32(residual[r * hidden + j]);",
     "float sum = orc_bf16_to_f32(xr[j]);"),
    ("mxfp8 eps outside the root", "float inv = 1.0f / sqrtf(mean_sq + eps);", "float inv = 1.0f / (sqrtf(mean_sq) + eps);"),
    ("mxfp8 norm scales the binary32 residual sum", "float t = orc_bf16_to_f32(pre[j]) * inv;",
     "float t = (residual ? orc_bf16_to_f32(xr[j]) + orc_bf16_to_f32(residual[r * hidden + j])\n"
     "                                 : orc_bf16_to_f32(pre[j])) * inv;"),
    ("mxfp8 weight before inv",
     "float t = orc_bf16_to_f32(pre[j]) * inv;\n            normed[j] = orc_bf16_to_f32(orc_f32_to_bf16(t * g1));",
     "float t = orc_bf16_to_f32(pre[j]) * g1;\n            normed[j] = orc_bf16_to_f32(orc_f32_to_bf16(t * inv));"),
    ("mxfp8 residual output from x", "                residual_out[r * hidden + j] = pre[j];",
     "                residual_out[r * hidden + j] = xr[j];"),
    ("mxfp8 mean over the padded width", "float mean_sq = f32_div(s, (float)hidden);",
     "float mean_sq = f32_div(s, (float)((hidden + 511) / 512 * 512));"),
    ("mxfp8 clamp at 240", "v = fminf(fmaxf(v, -448.0f), 448.0f);", "v = fminf(fmaxf(v, -240.0f), 240.0f);"),
    ("mxfp8 column interleave", "return col % 4 + (col / 4) * 512 +", "return (col / 4) % 4 + (col % 4) * 512 + (col / 16) * 2048 +"),
    ("mxfp8 tile stride of 64 columns", "(row / 128) * 128 * padded_cols;", "(row / 128) * 64 * padded_cols;"),
    ("mxfp8 amax over 31 elements",
     "for (int k = 0; k < 32; ++k)\n                amax = fmaxf(amax, fabsf(normed[32 * b + k]));",
     "for (int k = 0; k < 31; ++k)\n                amax = fmaxf(amax, fabsf(normed[32 * b + k]));"),
    ("mxfp8 scale byte one column over", "scale_out[orc_mxfp8_scale_offset(r, b, padded_cols)] = (uint8_t)byte;",
     "scale_out[orc_mxfp8_scale_offset(r, (b + 1) % cols, padded_cols)] = (uint8_t)byte;"),
    ("mxfp8 block of 16", "uint32_t byte = orc_ue8m0_ceil_byte(amax * inv448);",
     "uint32_t byte = orc_ue8m0_ceil_byte(fmaxf(amax, 0.0f) * inv448 * ((b & 1) ? 1.0f : 1.0f) + 0.0f * normed[0]);\n            amax = 0.0f; for (int k = 0; k < 16; ++k) amax = fmaxf(amax, fabsf(normed[32 * b + k]));\n            byte = orc_ue8m0_ceil_byte(amax * inv448);"),
]


def build_variant(tmp_path, text):
    src = tmp_path / "mut.c"
    src.write_text(text)
    lib = tmp_path / "libmut.so"
    subprocess.run(["gcc", "-O2", "-std=c11", "-ffp-contract=off", "-fno-fast-math", "-fopenmp",
                    "-fPIC", "-shared", str(src), "-o", str(lib), "-lm"], check=True)
    return str(lib)


def first_failure_in_child(lib_path):
    """Run the battery against the library at lib_path in a child process (a
    planted mistake may write out of bounds).  Returns the first failing test,
    "crash: <signal>" if the child died, or None if every pin passed."""
    code = (
        "import ctypes, sys\n"
        "import oracle, test_oracle_mutants as M\n"
        "oracle._lib = oracle.configure(ctypes.CDLL(sys.argv[1]))\n"
        "for slow in (False, True):\n"
        "    for name, fn in M.battery():\n"
        "        if (name.split('[')[0] in M.SLOW) != slow:\n"
        "            continue\n"
        "        try:\n"
        "            fn()\n"
        "        except Exception:\n"
        "            print('FAILED', name); sys.exit(0)\n"
        "print('PASSED')\n")
    here = os.path.dirname(os.path.abspath(__file__))
    env = dict(os.environ)
    env["PYTHONPATH"] = os.pathsep.join([here, os.path.dirname(here), env.get("PYTHONPATH", "")])
    res = subprocess.run([sys.executable, "-c", code, lib_path], capture_output=True, text=True,
                         env=env, timeout=300)
    if res.returncode != 0:
        return "crash: %d" % res.returncode
    last = res.stdout.strip().splitlines()[-1]
    return None if last == "PASSED" else last.split(" ", 1)[1]


def test_unmodified_oracle_passes_the_battery(tmp_path):
    assert first_failure_in_child(build_variant(tmp_path, open(SRC).read())) is None


def _run_mutant(i):
    """Build mutant i in a directory of its own and run the battery on it."""
    name, old, new = MUTANTS[i]
    with tempfile.TemporaryDirectory(prefix="mutant%02d_" % i) as d:
        return first_failure_in_child(build_variant(Path(d), open(SRC).read().replace(old, new)))


_FUTURES = []


def _mutant_result(i):
    """The battery's first failure on mutant i.  Each mutant is a gcc build
    and a child process, so on the first request every mutant is started, a
    few at a time, and each test then waits for its own; under pytest-xdist,
    which already spreads the cases over workers, each case runs alone."""
    if os.environ.get("PYTEST_XDIST_WORKER"):
        return _run_mutant(i)
    if not _FUTURES:
        pool = ThreadPoolExecutor(max(1, min(8, os.cpu_count() or 1)))
        _FUTURES.extend(pool.submit(_run_mutant, k) for k in range(len(MUTANTS)))
        pool.shutdown(wait=False)
    return _FUTURES[i].result()


@pytest.mark.parametrize("i", range(len(MUTANTS)), ids=[m[0] for m in MUTANTS])
def test_planted_mistake_is_caught(i):
    name, old, new = MUTANTS[i]
    assert open(SRC).read().count(old) == 1, "mutation site not found exactly once: %s" % name
    assert _mutant_result(i) is not None, "no pin catches: %s" % name
