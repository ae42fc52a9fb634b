"""Plant plausible mistakes in copies of the oracle and check that the pins catch each.

Every mutant is a one-place textual change of oracle.c (a transposed operand, a
dropped term, a wrong sign or index, a wrong constant, a wrong rounding rule),
compiled on the CPU into a temporary library. The mutant passes if no pin fails,
which would mean the pins cannot tell that mistake from the real oracle.
"""
import os
import subprocess
import sys

import pytest

from oracle import oracle as oracle_mod

# (name, text to replace, replacement, which occurrence (0-based))
MUTANTS = [
    ("V transposed in vtx", "acc += elem(th->V, dt, i * r + k)", "acc += elem(th->V, dt, k * d_in + i)", 0),
    ("U transposed", "elem(th->U, dt, o * r + k) * vtx[k]", "elem(th->U, dt, k * d_out + o) * vtx[k]", 0),
    ("W0 transposed", "elem(th->W0, dt, o * d_in + i) * elem(x, dt, x0 + i)", "elem(th->W0, dt, i * d_out + o) * elem(x, dt, x0 + i)", 0),
    ("x stride d_out", "const int64_t x0 = t * d_in;", "const int64_t x0 = t * d_out;", 0),
    ("s also scales delta", "y[t * d_out + o] = so * m + delta;", "y[t * d_out + o] = so * (m + delta);", 0),
    ("delta sign", "y[t * d_out + o] = so * m + delta;", "y[t * d_out + o] = so * m - delta;", 0),
    ("s dropped", "y[t * d_out + o] = so * m + delta;", "y[t * d_out + o] = m + delta;", 0),
    ("delta dropped", "y[t * d_out + o] = so * m + delta;", "y[t * d_out + o] = so * m;", 0),
    ("last rank term dropped", "for (int64_t k = 0; k < r; ++k) {\n                double p = elem(th->U, dt, o * r + k) * vtx[k];",
     "for (int64_t k = 0; k < r - 1; ++k) {\n                double p = elem(th->U, dt, o * r + k) * vtx[k];", 0),
    ("last column dropped", "for (int64_t i = 0; i < d_in; ++i) {\n                double p = elem(th->W0",
     "for (int64_t i = 0; i < d_in - 1; ++i) {\n                double p = elem(th->W0", 0),
    ("vtx over last input dropped", "for (int64_t i = 0; i < d_in; ++i)\n                acc +=",
     "for (int64_t i = 1; i < d_in; ++i)\n                acc +=", 0),
    ("s default 0", "double so = th->s ? (double)th->s[o] : 1.0;\n            y[", "double so = th->s ? (double)th->s[o] : 0.0;\n            y[", 0),
    ("bound ignores sign of s", "bound[t * d_out + o] = fabs(so) * m_abs + delta_abs;", "bound[t * d_out + o] = so * m_abs + delta_abs;", 0),
    ("bound signed sum", "m_abs += fabs(p);", "m_abs += p;", 0),
    ("gelu cubic constant", "0.044715 * z * z * z", "0.04715 * z * z * z", 0),
    ("gelu sqrt(pi/2)", "sqrt(2.0 / M_PI)", "sqrt(M_PI / 2.0)", 0),
    ("gelu drops z", "return 0.5 * z * (1.0 + tanh(a));", "return 0.5 * (1.0 + tanh(a));", 0),
    ("gelu of product", "orc_gelu_tanh(g[j]) * u[j]", "orc_gelu_tanh(g[j] * u[j])", 0),
    ("h not rounded to nearest", "((uint16_t *)hr)[j] = orc_bf16_rne(h);",
     "((uint16_t *)hr)[j] = (uint16_t)(orc_bf16_rne(h) + 1);", 0),
    ("up reads gate", "orc_linear(up, T, x, u, NULL)", "orc_linear(gate, T, x, u, NULL)", 0),
    ("rounding ties away from zero", "double n = nearbyint(ldexp(a, -q));", "double n = round(ldexp(a, -q));", 0),
    ("rounding truncates", "double n = nearbyint(ldexp(a, -q));", "double n = trunc(ldexp(a, -q));", 0),
    ("8 fraction bits", "int q = (e - 1) - 7;", "int q = (e - 1) - 8;", 0),
    ("subnormal quantum", "q = -133;", "q = -134;", 0),
    ("overflow saturates", "return sign | 0x7F80;             /* rounds past", "return sign | 0x7F7F;             /* rounds past", 0),
    ("qkv column offset", "col0 += n;", "col0 += q->d_out;", 0),
    ("weff V transposed", "elem(th->V, dt, i * r + k);\n                delta +=", "elem(th->V, dt, k * d_in + i);\n                delta +=", 0),
    ("weff unscaled", "double base = so * elem(th->W0, dt, o * d_in + i);", "double base = elem(th->W0, dt, o * d_in + i);", 0),
    ("rel frob squared", "return sqrt(num) / sqrt(den);", "return num / den;", 0),
    ("rel frob zero norm", "return num == 0.0 ? 0.0 : INFINITY;", "return 0.0;", 0),
    ("f32 read as bf16", "return (double)((const float *)p)[j];",
     "return bf16_value((uint16_t)(((const uint32_t *)p)[j] >> 16));", 0),
    ("f32 h rounded to bf16", "((float *)hr)[j] = (float)h;", "((float *)hr)[j] = (float)bf16_value(orc_bf16_rne(h));", 0),
    ("f32 h rounded down", "((float *)hr)[j] = (float)h;", "((float *)hr)[j] = (float)(h * (1.0 - 0x1p-24));", 0),
    ("f32 x read with the theta's W0 type only", "elem(x, dt, x0 + i);\n            vtx[k]", "elem(x, ORC_BF16, x0 + i);\n            vtx[k]", 0),
]


def _replace_nth(text, old, new, n):
    pos = -1
    for _ in range(n + 1):
        pos = text.find(old, pos + 1)
        assert pos >= 0, f"mutation anchor not found: {old!r}"
    return text[:pos] + new + text[pos + len(old):]


@pytest.mark.parametrize("name,old,new,nth", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_pins_catch_mutant(tmp_path, name, old, new, nth):
    src = open(oracle_mod.SOURCE).read()
    mutated = _replace_nth(src, old, new, nth)
    assert mutated != src
    c = tmp_path / "mutant.c"
    c.write_text(mutated)
    lib = oracle_mod.build(str(c), str(tmp_path / "libmutant.so"))
    # A mutant may index out of bounds, so the pins run in a child process; a
    # crash there also counts as caught.
    here = os.path.dirname(os.path.abspath(__file__))
    code = ("import sys; sys.path[:0] = [%r, %r]; import oracle_pins; "
            "oracle_pins.report(%r)" % (here, os.path.dirname(here), lib))
    proc = subprocess.run([sys.executable, "-c", code], capture_output=True, text=True,
                          timeout=300)
    if proc.returncode != 0:
        return
    failed = [line for line in proc.stdout.splitlines() if line.startswith("FAIL ")]
    assert failed, f"no pin catches the mutant '{name}'"
