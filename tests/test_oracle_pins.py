"""The fp64 oracle against its pins, and the pins against planted oracle mistakes (CPU only)."""

import os
import types

import pytest

import oracle.attention as real_oracle
from oracle_pins import PINS

ORACLE_SRC = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))),
                          "oracle", "attention.py")


@pytest.mark.parametrize("pin", PINS, ids=[p.__name__ for p in PINS])
def test_oracle_pin(pin):
    pin(real_oracle)


# Plausible mistakes, each planted in a copy of the oracle's source.  Every one
# must make at least one pin fail; otherwise the pins would not protect the
# parity tests from that mistake.
MUTATIONS = [
    ("causal off by one", "vis &= j <= i + o", "vis &= j < i + o"),
    ("top-left causal", "o = s_k - s_q\n    i = np.arange", "o = 0\n    i = np.arange"),
    ("window off by one", "vis &= j >= i + o - window + 1", "vis &= j >= i + o - window"),
    ("scale dropped", "s = scale * (q[bi, h, i0:i1] @ kg.T)", "s = (q[bi, h, i0:i1] @ kg.T)"),
    ("scale squared", "s = scale * (q[bi, h, i0:i1] @ kg.T)", "s = scale * scale * (q[bi, h, i0:i1] @ kg.T)"),
    ("V transposed", "num = e @ vg", "num = e @ vg.T"),
    ("Q K^T transposed", "s = scale * (q[bi, h, i0:i1] @ kg.T)", "s = scale * (kg[i0:i1] @ q[bi, h].T)"),
    ("GQA interleaved mapping", "            g = h // ratio\n            kg = k[bi, g]",
     "            g = h % h_kv\n            kg = k[bi, g]"),
    ("sink scaled", "z = z + np.exp(sig[h] - m_safe)\n                num = e @ vg",
     "z = z + np.exp(scale * sig[h] - m_safe)\n                num = e @ vg"),
    ("sink dropped from Z", "z = z + np.exp(sig[h] - m_safe)\n                num = e @ vg", "z = z\n                num = e @ vg"),
    ("LSE without max", "lse[bi, h, i0:i1] = np.where(nonempty, m_safe + np.log(",
     "lse[bi, h, i0:i1] = np.where(nonempty, 0.0 + np.log("),
    ("not normalised", "num / np.where(nonempty, z, 1.0)[:, None]", "num"),
    ("exp sign flipped", "e = np.exp(s - m_safe[:, None])", "e = np.exp(m_safe[:, None] - s)"),
    ("online: O not rescaled", "acc = alpha[:, None] * acc + p @ v[bi, g, j0:j1]",
     "acc = acc + p @ v[bi, g, j0:j1]"),
    ("online: l not rescaled", "l = alpha * l + p.sum(axis=1)", "l = l + p.sum(axis=1)"),
    ("online: P normalised early", "p = np.exp(s - base[:, None])",
     "p = np.exp(s - base[:, None]); p = p / np.maximum(p.sum(axis=1, keepdims=True), 1e-300)"),
    ("merge without exp", "w = np.where(np.isfinite(l), np.exp(l - m_safe[None]), 0.0)",
     "w = np.where(np.isfinite(l), l - m_safe[None], 0.0)"),
    ("merge LSE without max", "lse = np.where(nonempty, m_safe + np.log(np.where(nonempty, wsum, 1.0)), NEG_INF)",
     "lse = np.where(nonempty, np.log(np.where(nonempty, wsum, 1.0)), NEG_INF)"),
    ("split drops a key", "j1 = min(int(lens[bi]), j0 + split)", "j1 = min(int(lens[bi]), j0 + split - 1)"),
    ("decode window of sequence shifted", "kb = np.transpose(k[s0:s0 + n], (1, 0, 2))[None]",
     "kb = np.transpose(k[s0 + 1:s0 + n + 1], (1, 0, 2))[None]"),
    ("paged: next page read", "out[t0:t0 + n] = cache[int(table[t0 // page_size]), :n]",
     "out[t0:t0 + n] = cache[int(table[t0 // page_size + 1]), :n]"),
    ("paged: slot offset", "out[t0:t0 + n] = cache[int(table[t0 // page_size]), :n]",
     "out[t0:t0 + n] = cache[int(table[t0 // page_size]), 1:n + 1]"),
    ("paged: page index by slot", "out[t0:t0 + n] = cache[int(table[t0 // page_size]), :n]",
     "out[t0:t0 + n] = cache[int(table[t0 % page_size]), :n]"),
    ("fp8: exponent bias 8", "(1.0 + m / 8.0) * np.exp2(e.astype(np.float64) - 7.0)",
     "(1.0 + m / 8.0) * np.exp2(e.astype(np.float64) - 8.0)"),
    ("fp8: subnormals as normals", "np.where(e == 0, m / 8.0 * 2.0 ** -6,", "np.where(e < 0, m / 8.0 * 2.0 ** -6,"),
    ("fp8: sign dropped", "sign = np.where((c >> 7) & 1, -1.0, 1.0)", "sign = np.where((c >> 7) & 1, 1.0, 1.0)"),
    ("fp8: scales swapped", "k = fp8_e4m3_value(np.asarray(k_codes)) * ks[None, :, None]",
     "k = fp8_e4m3_value(np.asarray(k_codes)) * vs[None, :, None]"),
    ("bwd: D from P", "dd = (d_o[bi, h] * o).sum(axis=1)", "dd = (d_o[bi, h] * o).sum(axis=1) * 0.0"),
    ("bwd: dK without scale", "dk[bi, g] += scale * (ds.T @ q[bi, h])", "dk[bi, g] += (ds.T @ q[bi, h])"),
    ("bwd: dV transposed P", "dv[bi, g] += p.T @ d_o[bi, h]", "dv[bi, g] += p[:, :v.shape[2]].T @ d_o[bi, h][:p.shape[1]]"),
    ("bwd: dQ from V", "dq[bi, h] = scale * (ds @ k[bi, g])", "dq[bi, h] = scale * (ds @ v[bi, g])"),
    ("bwd: sink gradient sign", "dsig[h] += (p_sink * (0.0 - dd)).sum()", "dsig[h] += (p_sink * dd).sum()"),
    ("bwd: sink left out of P", "                z = z + np.exp(sig[h] - m_safe)\n            p = num",
     "                z = z\n            p = num"),
    ("flops count 2d per pair", "return 4 * d * pairs * b * h_q", "return 2 * d * pairs * b * h_q"),
]


def _mutant(old, new):
    with open(ORACLE_SRC) as f:
        src = f.read()
    assert src.count(old) == 1, f"mutation anchor not unique or missing: {old!r}"
    mod = types.ModuleType("oracle_mutant")
    exec(compile(src.replace(old, new), "oracle_mutant", "exec"), mod.__dict__)
    return mod


@pytest.mark.parametrize("name,old,new", MUTATIONS, ids=[m[0] for m in MUTATIONS])
def test_pins_catch_planted_mistake(name, old, new):
    mod = _mutant(old, new)
    caught = []
    for pin in PINS:
        try:
            pin(mod)
        except Exception as e:  # AssertionError, or a crash the mistake causes
            caught.append(f"{pin.__name__}: {type(e).__name__}")
    assert caught, f"no pin catches the planted mistake '{name}'"
