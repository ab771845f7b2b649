"""The oracle's pins catch plausible mistakes.

Each case plants one mistake in a copy of ``oracle/moe_oracle.c`` (on the CPU,
in a temporary directory), builds it with gcc, points the oracle binding at the
mutated library and runs the pins of ``test_oracle.py``: at least one of them
must fail.
"""
import ctypes
import inspect
import os
import subprocess
import tempfile

import pytest

import oracle
import test_oracle as pins

SRC = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "oracle", "moe_oracle.c")

MUTATIONS = {
    "nibble order reversed": ("(word >> (4 * (k % 8)))", "(word >> (4 * (7 - k % 8)))"),
    "bias term dropped": ("* (double)oracle_code(m, n, k) + b;", "* (double)oracle_code(m, n, k);"),
    "group index wrong": ("(size_t)(k / m->group);", "(size_t)((k / m->group + 1) % ng);"),
    "scale and bias swapped": ("double s = sb_value(m->s,", "double s = sb_value(m->b,"),
    "tie goes to higher index": ("key > best_key", "key >= best_key"),
    "softmax sign flipped": ("p[e] = exp(l[e] - lmax);", "p[e] = exp(lmax - l[e]);"),
    "no renormalisation": ("/ kept;", "/ 1.0;"),
    "selection on smallest": ("if (best < 0 || key > best_key)", "if (best < 0 || key < best_key)"),
    "logit bias subtracted": ("acc += (double)logit_bias[e];", "acc -= (double)logit_bias[e];"),
    "sigmoid instead of silu": ("return z / (1.0 + exp(-z));", "return 1.0 / (1.0 + exp(-z));"),
    "gate and up swapped": ("a[i] = silu(g) * u;", "a[i] = silu(u) * g;"),
    "down operand transposed": ("acc += Wd[(size_t)o * I + i] * a[i];", "acc += Wd[((size_t)i * H + o) % ((size_t)H * I)] * a[i];"),
    "routing weight ignored": ("acc += w[(size_t)t * k + j] * y_slot", "acc += 1.0 * y_slot"),
    "shared expert dropped": ("* y_shared[(size_t)t * H + h];", "* 0.0 * y_shared[(size_t)t * H + h];"),
    "router row index wrong": ("bf16_bits_value(router[(size_t)e * H + h])", "bf16_bits_value(router[(size_t)((e + 1) % E) * H + h])"),
    "shared gate sign flipped": ("s[t] = 1.0 / (1.0 + exp(-z));", "s[t] = 1.0 / (1.0 + exp(z));"),
    "shared gate ignored": ("(shared_w ? shared_w[t] : 1.0)", "(shared_w ? 1.0 : 1.0)"),
    "q8 router byte order reversed": ("(word >> (8 * (h % 4)))", "(word >> (8 * (3 - h % 4)))"),
    "q8 router ties rounded up": ("(lower == 0x8000u && (upper & 1u))", "(lower == 0x8000u)"),
    "q8 router scale and bias swapped": ("fmaf(sv, (float)q, bv)", "fmaf(bv, (float)q, sv)"),
    "rmsnorm sum instead of mean": ("sqrt(ss / (double)H + eps)", "sqrt(ss + eps)"),
    "rmsnorm eps ignored": ("sqrt(ss / (double)H + eps)", "sqrt(ss / (double)H)"),
    "rmsnorm gamma ignored": ("const double g = gamma ? bf16_bits_value(gamma[h]) : 1.0;", "const double g = 1.0;"),
    "rmsnorm rounds toward zero": ("nearbyint(ldexp(m, 8))", "trunc(ldexp(m, 8))"),
    "gqa group index modulo": ("const int32_t g = h / per_kv;", "const int32_t g = h % Hkv;"),
    "gqa scale ignored": ("p[j] = scale * acc;", "p[j] = acc;"),
    "gqa current row dropped": ("int32_t n = seq_len[b];", "int32_t n = seq_len[b] - 1;"),
    "gqa normaliser dropped": ("o[d] = acc / z;", "o[d] = acc;"),
    "gqa values read from the keys": ("acc += p[j] * bf16_bits_value(vg[", "acc += p[j] * bf16_bits_value(kg["),
    "permute not stable": ("sorted_slot[cursor[idx[s]]++] = s;", "sorted_slot[offsets[idx[s] + 1] - 1 - (cursor[idx[s]]++ - offsets[idx[s]])] = s;"),
}


def _pin_functions():
    fns = []
    for name, fn in inspect.getmembers(pins, inspect.isfunction):
        if not name.startswith("test_") or name.startswith("test_zipf") or name.startswith("test_near_ties"):
            continue
        marks = getattr(fn, "pytestmark", [])
        params = [m for m in marks if m.name == "parametrize"]
        if params:
            argname, values = params[0].args[0], params[0].args[1]
            for v in values:
                fns.append((fn, {argname: v}))
        else:
            fns.append((fn, {}))
    return fns


@pytest.mark.parametrize("name", sorted(MUTATIONS))
def test_mutation_is_caught(name):
    old, new = MUTATIONS[name]
    src = open(SRC).read()
    assert src.count(old) >= 1, "mutation anchor not found: " + old
    with tempfile.TemporaryDirectory() as d:
        cpath = os.path.join(d, "m.c")
        so = os.path.join(d, "libm.so")
        with open(cpath, "w") as f:
            f.write(src.replace(old, new))
        subprocess.check_call(["gcc", "-O1", "-std=c99", "-fPIC", "-shared", "-I" + os.path.dirname(SRC),
                               "-o", so, cpath, "-lm"])
        saved_path, saved_lib = oracle._LIB_PATH, oracle._lib
        oracle._LIB_PATH, oracle._lib = so, None
        failed = []
        try:
            for fn, kw in _pin_functions():
                try:
                    fn(**kw)
                except (AssertionError, Exception):  # noqa: B014 - any failure counts as caught
                    failed.append(fn.__name__)
                    break
        finally:
            oracle._LIB_PATH, oracle._lib = saved_path, saved_lib
            ctypes  # keep import used
    assert failed, "no pin failed for mutation: " + name
