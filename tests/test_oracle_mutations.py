"""Plants plausible mistakes in copies of the oracle (on the CPU) and requires
the pins to catch every one of them: evidence that the pins constrain each
step of the oracle, not just its overall shape."""
import importlib.util
import os
import types

import pytest

from pins import PINS

SRC = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))),
                   "oracle", "mqa_oracle.py")

# (description, text in the oracle, replacement)
MUTANTS = [
    ("exponent bias 8", "2.0 ** (exponent - 10)", "2.0 ** (exponent - 11)"),
    ("subnormal step 2^-10", "mantissa * 2.0 ** -9", "mantissa * 2.0 ** -10"),
    ("fnuz-style NaN at 0x80", "if exponent == 0xF and mantissa == 0x7:",
     "if code == 0x80:"),
    ("sign bit ignored", "sign = -1.0 if (code >> 7) else 1.0", "sign = 1.0"),
    ("scale read big-endian", '"<f4"', '">f4"'),
    ("scale not applied", "x = score * s_b[:nv, None]", "x = score"),
    ("relu after the head sum", "np.maximum(x, 0.0) @ w[b * N + j]", "np.maximum(x @ w[b * N + j], 0.0)"),
    ("no relu", "np.maximum(x, 0.0) @ w[b * N + j]", "x @ w[b * N + j]"),
    ("causal window one short", "ctx - next_n + j + 1, max_model_len", "ctx - next_n + j, max_model_len"),
    ("causal window one long", "ctx - next_n + j + 1, max_model_len", "ctx - next_n + j + 2, max_model_len"),
    ("next_n offset ignored", "ctx - next_n + j + 1, max_model_len", "ctx, max_model_len"),
    ("weights of row b*N", "@ w[b * N + j]", "@ w[b * N]"),
    ("block table ignored", "phys = token_rows(block_tables[b], ctx, bs)",
     "phys = np.arange(ctx, dtype=np.int64)"),
    ("block slot ignored", "* block_size + t % block_size", "* block_size"),
    ("block index by token", "np.asarray(table_row)[t // block_size]", "np.asarray(table_row)[t]"),
    ("block size ignored", "return 1 if kv.ndim == 2 else int(kv.shape[1])", "return 1"),
    ("query of decode row 0 for every row", "score = k_b[:nv] @ qv[b, j].T", "score = k_b[:nv] @ qv[b, 0].T"),
    ("query head/dim transposed", "score = k_b[:nv] @ qv[b, j].T",
     "score = k_b[:nv, :qv.shape[2]] @ qv[b, j][:, :qv.shape[2]]"),
    ("top-k keeps the smallest", "order = np.lexsort((np.arange(values.size), -values))",
     "order = np.lexsort((np.arange(values.size), values))"),
    ("top-k ties to highest position", "order = np.lexsort((np.arange(values.size), -values))",
     "order = np.lexsort((-np.arange(values.size), -values))"),
    ("encode ties away from zero", "((d_hi == d_lo) & (hi_c % 2 == 0))", "(d_hi == d_lo)"),
    ("encode truncates", "take_hi = exact | (d_hi < d_lo) | ((d_hi == d_lo) & (hi_c % 2 == 0))", "take_hi = exact"),
    ("encode saturates", "code = np.where(ax > 464.0, np.uint8(0x7F), code)", "code = code"),
    ("scale maps amax to 240", "scale = np.float32(amax / np.float32(E4M3FN_MAX))", "scale = np.float32(amax / np.float32(240.0))"),
    ("scale multiplies", "scaled = (k32 / scale).astype(np.float32)", "scaled = (k32 * scale).astype(np.float32)"),
    ("write ignores the slot", "rows[slot, :HEAD_DIM] = codes", "rows[i, :HEAD_DIM] = codes"),
    ("prefill window end inclusive", "hi = min(max(int(ke[m]), 0), N)", "hi = min(max(int(ke[m]) + 1, 0), N)"),
    ("prefill window start ignored", "lo = min(max(int(ks[m]), 0), N)", "lo = 0"),
    ("prefill scale not applied", "x = score * scales[lo:hi, None]", "x = score"),
    ("top-k one short", "return np.sort(order[:min(k, values.size)])",
     "return np.sort(order[:min(k, values.size) - 1])"),
]


def _load_mutant(old, new):
    with open(SRC) as f:
        text = f.read()
    assert old in text, f"mutation site not found: {old!r}"
    mod = types.ModuleType("oracle_mutant")
    mod.__file__ = SRC
    exec(compile(text.replace(old, new), SRC + " (mutant)", "exec"), mod.__dict__)
    return mod


def _caught(mod):
    for pin in PINS:
        try:
            pin(mod)
        except Exception:   # an assertion, or the mutant crashing on a pin's input
            return pin.__name__
    return None


@pytest.mark.parametrize("desc,old,new", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_pins_catch_mutant(desc, old, new):
    assert _caught(_load_mutant(old, new)) is not None, f"no pin catches: {desc}"


def test_unmutated_oracle_passes_every_pin():
    with open(SRC) as f:
        text = f.read()
    mod = types.ModuleType("oracle_copy")
    exec(compile(text, SRC, "exec"), mod.__dict__)
    assert _caught(mod) is None


# Sparse MLA decode oracle: planted mistakes must be caught by its own pins.
from pins_mla import MLA_PINS  # noqa: E402

MLA_SRC = os.path.join(os.path.dirname(SRC), "sparse_mla_oracle.py")

MLA_MUTANTS = [
    ("softmax scale dropped", "c = float(np.float32(sm_scale)) * float(np.float32(q_scale))", "c = float(np.float32(q_scale))"),
    ("q scale dropped", "c = float(np.float32(sm_scale)) * float(np.float32(q_scale))", "c = float(np.float32(sm_scale))"),
    ("values not scaled", "out[r] = vs * (p.T @ keys[:, :MLA_V_DIM])", "out[r] = p.T @ keys[:, :MLA_V_DIM]"),
    ("values from the wrong dims", "out[r] = vs * (p.T @ keys[:, :MLA_V_DIM])", "out[r] = vs * (p.T @ keys[:, 64:])"),
    ("softmax over heads", "l = e.sum(axis=0)\n        p = e / l", "l = e.sum(axis=1, keepdims=True)\n        p = e / l"),
    ("maximum not subtracted", "e = np.exp(score - m)\n        l = e.sum(axis=0)\n        p = e / l",
     "e = np.exp(score)\n        l = e.sum(axis=0)\n        p = e / l"),
    ("lse without the maximum", "lse[r] = m + np.log(l)", "lse[r] = np.log(l)"),
    ("padding attended", "pos = idx[r][idx[r] >= 0]\n        if pos.size == 0:\n            continue\n        if pos.max()",
     "pos = idx[r]\n        if pos.size == 0:\n            continue\n        if pos.max()"),
    ("duplicates collapsed", "pos = idx[r][idx[r] >= 0]\n        if pos.size == 0:\n            continue\n        if pos.max()",
     "pos = np.unique(idx[r][idx[r] >= 0])\n        if pos.size == 0:\n            continue\n        if pos.max()"),
    ("block slot ignored", "return entries * block_size + t % block_size", "return entries * block_size"),
    ("request of a row taken modulo", "b = r // next_n\n        pos", "b = r % next_n\n        pos"),
    ("query of row 0 for every row", "score = (keys @ qv[r].T) * c", "score = (keys @ qv[0].T) * c"),
    # the tolerance scale of the GPU tests, B = kv_scale * sum_t p |v_t|
    ("bound: kv_scale dropped", "bound[r] = float(np.float32(kv_scale)) * (p.T @ np.abs(keys[:, :MLA_V_DIM]))",
     "bound[r] = p.T @ np.abs(keys[:, :MLA_V_DIM])"),
    ("bound: absolute value dropped", "bound[r] = float(np.float32(kv_scale)) * (p.T @ np.abs(keys[:, :MLA_V_DIM]))",
     "bound[r] = float(np.float32(kv_scale)) * (p.T @ keys[:, :MLA_V_DIM])"),
    ("bound: probabilities unnormalised", "e = np.exp(score - score.max(axis=0))\n        p = e / e.sum(axis=0)",
     "e = np.exp(score - score.max(axis=0))\n        p = e"),
    ("bound: maximum not subtracted", "e = np.exp(score - score.max(axis=0))\n        p = e / e.sum(axis=0)",
     "e = np.exp(score)\n        p = e / e.sum(axis=0)"),
    ("bound: softmax scale dropped", "c = float(np.float32(sm_scale)) * float(np.float32(q_scale)) * float(np.float32(kv_scale))\n    bound",
     "c = float(np.float32(q_scale)) * float(np.float32(kv_scale))\n    bound"),
    ("bound: values from the wrong dims", "(p.T @ np.abs(keys[:, :MLA_V_DIM]))", "(p.T @ np.abs(keys[:, 64:]))"),
    ("bound: request of a row taken modulo", "tables[r // next_n], S)", "tables[r % next_n], S)"),
    ("bound: scaled by 10", "bound[r] = float(np.float32(kv_scale)) *", "bound[r] = 10.0 * float(np.float32(kv_scale)) *"),
]


def _load_mla_mutant(old, new):
    with open(MLA_SRC) as f:
        text = f.read()
    assert old in text, f"mutation site not found: {old!r}"
    text = text.replace(old, new).replace("from .mqa_oracle import", "from oracle.mqa_oracle import")
    mod = types.ModuleType("mla_oracle_mutant")
    mod.__file__ = MLA_SRC
    exec(compile(text, MLA_SRC + " (mutant)", "exec"), mod.__dict__)
    return mod


def _mla_caught(mod):
    for pin in MLA_PINS:
        try:
            pin(mod)
        except Exception:
            return pin.__name__
    return None


@pytest.mark.parametrize("desc,old,new", MLA_MUTANTS, ids=[m[0] for m in MLA_MUTANTS])
def test_mla_pins_catch_mutant(desc, old, new):
    assert _mla_caught(_load_mla_mutant(old, new)) is not None, f"no pin catches: {desc}"


def test_unmutated_mla_oracle_passes_every_pin():
    assert _mla_caught(_load_mla_mutant("MLA_V_DIM = 512", "MLA_V_DIM = 512")) is None
