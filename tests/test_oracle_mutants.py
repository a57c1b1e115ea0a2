"""Plants one plausible mistake at a time in a copy of the oracle (on the CPU,
in a temporary directory) and checks that the pins in test_oracle_pins.py
catch every one of them.  The real oracle source is never modified."""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "oracle", "oracle.c")

MUTANTS = [
    ("i2s shift order", "*shift = 6 - 2 * (int)(r / 32);", "*shift = 2 * (int)(r / 32);"),
    ("i2s byte index", "*byte = n * (K / 4) + 32 * g + (r % 32);", "*byte = n * (K / 4) + 32 * g + ((r % 32) ^ 1);"),
    ("i2s decode sign", "w[n * K + k] = (int8_t)(code - 1);", "w[n * K + k] = (int8_t)(1 - code);"),
    ("i2s scale dropped", "y[m * nr + i] = scale * acc;", "y[m * nr + i] = acc;"),
    ("i2s operand transposed", "acc += (double)w * (double)x[m * K + k];", "acc += (double)w * (double)x[k * M + m];"),
    ("tq2 code table", "case 0x3: return -1;", "case 0x3: return 1;"),
    ("tq2 element order", "int code = (blocks[66 * blk + e / 4] >> (2 * (e % 4))) & 3;",
     "int code = (blocks[66 * blk + e / 4] >> (6 - 2 * (e % 4))) & 3;"),
    ("tq2 gemv element order", "int w = tq2_value_of((blk[e / 4] >> (2 * (e % 4))) & 3);",
     "int w = tq2_value_of((blk[e / 4] >> (6 - 2 * (e % 4))) & 3);"),
    ("tq2 scale byte order", "double s = orc_f16_to_f64((uint16_t)(blk[64] | (blk[65] << 8)));",
     "double s = orc_f16_to_f64((uint16_t)(blk[65] | (blk[64] << 8)));"),
    ("tq2 i8 token scale dropped", "y[m * nr + i] = (double)s_tok[m] * acc;", "y[m * nr + i] = acc;"),
    ("tq2 i8 block scale dropped", "acc += s * (double)d;", "acc += (double)d;"),
    ("tq2 i8 activation index", "int64_t qv = q[m * K + b * 256 + e];", "int64_t qv = q[m * K + b * 256 + (e ^ 1)];"),
    ("w1 sign", "d += (int64_t)(2 * b - 1) * qv;", "d += (int64_t)(1 - 2 * b) * qv;"),
    ("w1 scale index", "S += orc_f16_to_f64(sc[n * (K / G) + g]) * (double)d;",
     "S += orc_f16_to_f64(sc[n * (K / G)]) * (double)d;"),
    ("w1 bit order", "int b = (bits[n * (K / 32) + k / 32] >> (k % 32)) & 1;",
     "int b = (bits[n * (K / 32) + k / 32] >> (31 - k % 32)) & 1;"),
    ("bf16 tie rule", "return (lo & 1u) ? hi : lo;", "return (lo & 1u) ? lo : hi;"),
    ("bf16 nearest", "if (dl < dh) return lo;", "if (dl > dh) return lo;"),
    ("quantize rounding", "float r = rintf(v);", "float r = truncf(v);"),
    ("quantize scale", "volatile float sv = a / 127.0f;", "volatile float sv = a / 128.0f;"),
    ("i8 epilogue operand", "volatile float t = (float)acc * s_tok[m];", "volatile float t = (float)acc * s_w;"),
    ("f16 rounding", "double m = rint(ldexp(v, 10 - e));", "double m = floor(ldexp(v, 10 - e));"),
    ("from_dense mean", "sc[n * (K / G) + g] = orc_f64_to_f16(s / (double)G);",
     "sc[n * (K / G) + g] = orc_f64_to_f16(s / (double)(G - 1));"),
]


@pytest.mark.parametrize("name,before,after", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_pins_catch_mutant(tmp_path, name, before, after):
    src = open(SRC).read()
    assert src.count(before) >= 1, name
    mut = tmp_path / "oracle_mut.c"
    mut.write_text(src.replace(before, after, 1))
    so = tmp_path / "liboracle_mut.so"
    import oracle
    subprocess.check_call(["gcc", *oracle.GCC_FLAGS, "-o", str(so), str(mut), "-lm"])
    env = dict(os.environ, ORACLE_LIB_OVERRIDE=str(so))
    r = subprocess.run([sys.executable, "-m", "pytest", "-x", "-q", "-p", "no:cacheprovider",
                        os.path.join(ROOT, "tests", "test_oracle_pins.py")],
                       cwd=ROOT, env=env, capture_output=True, text=True, timeout=600)
    assert r.returncode != 0, "mutant '%s' survived the pins" % name
