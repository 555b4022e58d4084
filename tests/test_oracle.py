"""CPU tests of the float64 oracle against what the pages and mathematics fix.

The pins themselves live in ``oracle_pins.py``.  Each is run on the real
oracle; then one plausible mistake at a time (a dropped term, a wrong sign,
index or operand) is planted in a private copy of the oracle's source, and at
least one pin must fail on every such copy.
"""

from __future__ import annotations

import os
import types

import pytest

import oracle_pins
from oracle import attention_f64

ORACLE_SRC = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))),
                          "oracle", "attention_f64.py")


@pytest.mark.parametrize("pin", oracle_pins.ALL_PINS, ids=lambda f: f.__name__)
def test_oracle_pin(pin):
    pin(attention_f64)


# (description, text in the oracle source, replacement)
MUTANTS = [
    ("scale dropped", "s = scale * (q @ k.T)", "s = (q @ k.T)"),
    ("causal mask top-left aligned", "(rows + (nk - total))", "(rows + 0)"),
    ("causal mask off by one", "np.arange(nk)[None, :] <= (rows", "np.arange(nk)[None, :] < (rows"),
    ("max not subtracted", "e = np.exp(s - m_safe[:, None])", "e = np.exp(s)"),
    ("softmax sum over wrong axis", "l = e.sum(axis=1)", "l = e.sum(axis=1) + e[:, :1].sum(axis=1)"),
    ("LSE in log2", "m_safe + np.log(np.where(empty, 1.0, l))", "m_safe + np.log2(np.where(empty, 1.0, l))"),
    ("LSE without max", "lse = np.where(empty, -np.inf, m_safe + np.log(", "lse = np.where(empty, -np.inf, 0 + np.log("),
    ("GQA heads interleaved", "o[b, h] = p @ v[b, h // g]", "o[b, h] = p @ v[b, h % hkv]"),
    ("GQA heads interleaved (probs)", "attention_probs(q[b, h], k[b, h // g]", "attention_probs(q[b, h], k[b, h % hkv]"),
    ("dS sign of D flipped", "ds = p * (dp - dd[:, None])", "ds = p * (dp + dd[:, None])"),
    ("D term dropped", "ds = p * (dp - dd[:, None])", "ds = p * dp"),
    ("D without O", "dd = (do[b, h] * o).sum(axis=1)", "dd = do[b, h].sum(axis=1)"),
    ("dQ scale dropped", "dq[b, h] = scale * (ds @ kh)", "dq[b, h] = (ds @ kh)"),
    ("dQ from V", "dq[b, h] = scale * (ds @ kh)", "dq[b, h] = scale * (ds @ vh[:, :kh.shape[1]])"),
    ("dK scale dropped", "dk[b, h // g] += scale * (ds.T @ q[b, h])", "dk[b, h // g] += (ds.T @ q[b, h])"),
    ("dK transposed dS", "dk[b, h // g] += scale * (ds.T @ q[b, h])", "dk[b, h // g] += scale * (ds @ q[b, h])"),
    ("dV from dS", "dv[b, h // g] += p.T @ do[b, h]", "dv[b, h // g] += ds.T @ do[b, h]"),
    ("dV not accumulated over group", "dv[b, h // g] += p.T @ do[b, h]", "dv[b, h // g] = p.T @ do[b, h]"),
    ("page slot wrong", "out[:, t:t + n, :] = cache[page, :, :n, :]", "out[:, t:t + n, :] = cache[page, :, bs - n:, :]"),
    ("page index wrong", "page = int(block_table_row[t // bs])", "page = int(block_table_row[(t // bs) // 2])"),
    ("streaming sum not rescaled", "l = l * rescale + float", "l = l + float"),
    ("streaming block sum at old max", "float(np.exp(blk - m_new).sum())", "float(np.exp(blk - max(m, float(blk.max()) - 1.0) + 0 * m_new).sum())"),
    ("merge weights swapped", "return mx, l_a * wa + l_b * wb", "return mx, l_a * wb + l_b * wa"),
    ("prefill mask top-left", "o[b], lse[b] = (x[0] for x in attention_fwd(q[b][None], kb, vb, scale, causal))",
     "o[b], lse[b] = (x[0] for x in attention_fwd(q[b][None], kb[:, :, :nq], vb[:, :, :nq], scale, causal))"),
    ("prefill reads table of sequence 0", "kb = gather_pages(k_cache, block_table[b], n)[None]",
     "kb = gather_pages(k_cache, block_table[0], n)[None]"),
    ("fp8 exponent bias 8", "(1.0 + f / 8.0) * np.exp2(e - 7.0)", "(1.0 + f / 8.0) * np.exp2(e - 8.0)"),
    ("fp8 subnormals without the 2^-6 scale", "(f / 8.0) * 2.0 ** -6", "(f / 8.0) * 2.0 ** -7"),
    ("fp8 V descale dropped", "v = fp8_e4m3_decode(v_codes) * v_descale", "v = fp8_e4m3_decode(v_codes)"),
    ("packed rows without head factor", "    r0 = h * int(cu[b])\n", "    r0 = int(cu[b])\n"),
    ("packed blocks token-major", "return x[r0:r0 + h * n].reshape(1, h, n, x.shape[-1])",
     "return x[r0:r0 + h * n].reshape(1, n, h, x.shape[-1]).transpose(0, 2, 1, 3)"),
    ("packed dK rows at query offsets", "rq, rk = hq * int(cu_q[b]), hkv * int(cu_k[b])",
     "rq, rk = hq * int(cu_q[b]), hkv * int(cu_q[b])"),
]


def _mutant(old: str, new: str) -> types.ModuleType:
    with open(ORACLE_SRC) as f:
        src = f.read()
    assert src.count(old) == 1, f"mutation site not unique or missing: {old!r}"
    mod = types.ModuleType("oracle_mutant")
    exec(compile(src.replace(old, new), "oracle_mutant", "exec"), mod.__dict__)
    return mod


@pytest.mark.parametrize("desc,old,new", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_pins_catch_planted_mistake(desc, old, new):
    mod = _mutant(old, new)
    caught = []
    for pin in oracle_pins.ALL_PINS:
        try:
            pin(mod)
        except Exception as e:  # an assertion or a crash both expose the mistake
            caught.append((pin.__name__, type(e).__name__))
            break
    assert caught, f"no pin fails when the oracle has: {desc}"
