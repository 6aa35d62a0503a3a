"""The pins are strong enough: each plausible mistake planted in a copy of the C++ oracle makes
at least one pin fail.

Each mutant is one textual change to oracle/routed_attention.cpp (a wrong rounding, an
off-by-one window, a wrong divisor, a reversed order or tie-break, a dropped scale, a wrong kv
head, a dropped kappa, a lost running sum), compiled to a temporary library on the CPU; the C++
oracle's Python face is pointed at it and the pins of tests/test_oracle.py run against it.
"""
import inspect
import os
import subprocess

import pytest

import oracle.cpp as CPP
import test_oracle as PINS

MUTANTS = [
    ("kappa keeps 9 bits", "std::max(e - 8, -133)", "std::max(e - 7, -133)"),
    ("kappa truncates", "std::nearbyint((double)x / spacing)", "std::trunc((double)x / spacing)"),
    ("window one token short", "t - W + 1 > 0 ? t - W + 1 : 0", "t - W > 0 ? t - W : 0"),
    ("mean over S + 1", "sum[e] / (float)S", "sum[e] / (float)(S + 1)"),
    ("scores sorted ascending", "return scores[a] > scores[b];", "return scores[a] < scores[b];"),
    ("ties go to the higher index", "return a < b;", "return a > b;"),
    ("one span too few", "const int64_t m = std::min(k, r);", "const int64_t m = std::min(k, r - (r > 0));"),
    ("no 1/sqrt(d)", "z[i] = dot * inv_sqrt_d;", "z[i] = dot;"),
    ("wrong kv head", "const int64_t t = pos[i], g = head[i] / G;", "const int64_t t = pos[i], g = head[i] % hkv;"),
    ("query's own token left out", "for (int64_t p = window_start(t, S, W); p <= t; ++p)",
     "for (int64_t p = window_start(t, S, W); p < t; ++p)"),
    ("no kappa for bf16", "s += q[e] * (double)(is_bf16 ? kappa_bf16(m) : m);", "s += q[e] * (double)m;"),
    ("running sum dropped", "if (p0 == old_len)", "if (p0 == old_len && false)"),
    ("softmax not normalised", "const double w = std::exp(z[i] - zmax) / denom;",
     "const double w = std::exp(z[i] - zmax);"),
]


def _pins():
    """(name, callable) for every pin of the method's steps, with its parameters filled in."""
    out = []
    for name, fn in sorted(vars(PINS).items()):
        if not name.startswith("test_") or not callable(fn):
            continue
        params = list(inspect.signature(fn).parameters)
        if params and params[0] == "impl":
            rest = params[1:]
            if rest == ["chunk"]:
                out += [(name, lambda fn=fn, c=c: fn(CPP, c)) for c in (1, 7, 100)]
            elif rest == ["bf16"]:
                out += [(name, lambda fn=fn, b=b: fn(CPP, b)) for b in (False, True)]
            elif not rest:
                out.append((name, lambda fn=fn: fn(CPP)))
        elif name.startswith("test_cpp_"):
            p = inspect.signature(fn).parameters
            if list(p) == ["bf16"]:
                out += [(name, lambda fn=fn, b=b: fn(b)) for b in (False, True)]
            elif not p:
                out.append((name, fn))
    return out


@pytest.mark.parametrize("what,old,new", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_planted_mistake_fails_a_pin(what, old, new, tmp_path, monkeypatch):
    src = open(CPP.SOURCE).read()
    assert src.count(old) == 1, "the mutation no longer applies: " + old
    cpp = tmp_path / "mutant.cpp"
    cpp.write_text(src.replace(old, new))
    so = tmp_path / "libmutant.so"
    subprocess.check_call(["g++", "-O2", "-std=c++17", "-pthread", "-fPIC", "-shared", str(cpp), "-o", str(so)])
    monkeypatch.setattr(CPP, "LIB_PATH", str(so))
    monkeypatch.setattr(CPP, "_lib", None)
    failed = []
    for name, pin in _pins():
        try:
            pin()
        except AssertionError:
            failed.append(name)
            break
    monkeypatch.setattr(CPP, "_lib", None)
    assert failed, "no pin caught: " + what
