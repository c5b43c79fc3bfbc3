"""Plant plausible mistakes in a copy of the oracle (on the CPU) and check that
the pins catch every one of them.  A mutant that survives would mean the pins
do not constrain that part of the oracle."""
import importlib.util
import os
import types

import pytest

import oracle_pins

pytestmark = pytest.mark.cpu

SRC = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))),
                   "oracle", "rkv_oracle.py")

# (name, text in the oracle, replacement)
MUTANTS = [
    ("no 1/sqrt(d) scale", "return (q_rows @ k.T) / math.sqrt(d)", "return (q_rows @ k.T)"),
    ("scale 1/d", "return (q_rows @ k.T) / math.sqrt(d)", "return (q_rows @ k.T) / d"),
    ("softmax over the wrong axis", "p = p / p.sum(axis=1, keepdims=True)",
     "p = p / p.sum(axis=0, keepdims=True)"),
    ("sum instead of mean over rows", "return p.mean(axis=0)", "return p.sum(axis=0)"),
    ("max over the wrong axis", "logits - logits.max(axis=1, keepdims=True)",
     "logits - logits.max()"),
    ("diagonal kept", "off = c.sum(axis=1) - np.diag(c)", "off = c.sum(axis=1)"),
    ("divide by N", "return off / (n - 1)", "return off / n"),
    ("no key normalisation", "return khat @ khat.T", "return k @ k.T"),
    ("norm without sqrt", "norms = np.sqrt((k * k).sum(axis=1))", "norms = (k * k).sum(axis=1)"),
    ("mix sign flipped", "return lam * imp - (1.0 - lam) * red", "return lam * imp + (1.0 - lam) * red"),
    ("lambda roles swapped", "return lam * imp - (1.0 - lam) * red", "return (1.0 - lam) * imp - lam * red"),
    ("ties keep the later position", "order = np.lexsort((pos, -s))", "order = np.lexsort((-pos, -s))"),
    ("ascending score kept", "order = np.lexsort((pos, -s))", "order = np.lexsort((pos, s))"),
    ("window not forced", "chosen = np.sort(order[: budget - window])",
     "chosen = np.sort(order[: budget - window]); cand = n"),
    ("budget excludes window", "chosen = np.sort(order[: budget - window])",
     "chosen = np.sort(order[: budget])"),
    ("free blocks floor", "first = -(-budget // block_size)", "first = budget // block_size"),
    ("trigger strict", "return int(n) >= int(budget) + int(buffer)",
     "return int(n) > int(budget) + int(buffer)"),
    ("rows reversed before the row mean", "return (q_rows @ k.T) / math.sqrt(d)",
     "return (k @ q_rows.T).T[::-1] / math.sqrt(d)"),
    ("GQA heads strided", "qg = q_seq_layer[h * group:(h + 1) * group]",
     "qg = q_seq_layer[h::q_seq_layer.shape[0] // group]"),
    ("transposed Gram operand", "return khat @ khat.T", "return khat.T @ khat"),
    ("gather off by one", "return rows[np.asarray(keep)]", "return rows[np.minimum(np.asarray(keep) + 1, len(rows) - 1)]"),
    ("row-wise redundancy keeps the diagonal", "out.append((row.sum() - row[j]) / (n - 1))",
     "out.append(row.sum() / (n - 1))"),
    ("row-wise redundancy unnormalised", "row = khat @ khat[j]", "row = k @ k[j]"),
    ("shared: max over heads", "return hs.sum(axis=0)", "return hs.max(axis=0)"),
    ("shared: first head only", "return hs.sum(axis=0)", "return hs[0]"),
    ("shared: mean over heads", "return hs.sum(axis=0)", "return hs.mean(axis=0)"),
    ("ring slot t // window", "out[layer0 + i, s, :, int(steps[s]) % window, :] = q_step[i, s]",
     "out[layer0 + i, s, :, (int(steps[s]) // window) % window, :] = q_step[i, s]"),
    ("ring ignores layer0", "out[layer0 + i, s, :, int(steps[s]) % window, :] = q_step[i, s]",
     "out[i, s, :, int(steps[s]) % window, :] = q_step[i, s]"),
    ("ring slot shifted by one", "out[layer0 + i, s, :, int(steps[s]) % window, :] = q_step[i, s]",
     "out[layer0 + i, s, :, (int(steps[s]) + 1) % window, :] = q_step[i, s]"),
    ("bf16 decode without the 16-bit shift", "astype(np.uint32) << np.uint32(16)",
     "astype(np.uint32) << np.uint32(8)"),
    ("bf16 decode with swapped bytes", "w = np.asarray(x, dtype=np.uint16).astype",
     "w = np.asarray(x, dtype=np.uint16).byteswap().astype"),
    ("bf16 decode drops the sign", "w = np.asarray(x, dtype=np.uint16).astype(np.uint32) << np.uint32(16)",
     "w = (np.asarray(x, dtype=np.uint16).astype(np.uint32) & np.uint32(0x7FFF)) << np.uint32(16)"),
    ("f32 decode through half precision", "return np.asarray(x, dtype=np.float32).astype(np.float64)",
     "return np.asarray(x, dtype=np.float32).astype(np.float16).astype(np.float64)"),
    ("step_unit with group 1", "return unit_step(q_group(qd, h, group),",
     "return unit_step(q_group(qd, h, 1),"),
    ("step_unit with the heads' order inverted", "return unit_step(q_group(qd, h, group),",
     "return unit_step(q_group(qd, spec.num_kv_heads - 1 - h, group),"),
    ("step_unit compacts the decoded keys", "decode(k_rows, spec.dtype), k_rows, v_rows,",
     "decode(k_rows, spec.dtype), decode(k_rows, spec.dtype), v_rows,"),
    ("shared layer: per-head keep", "keep = select_keep_shared(np.stack([h[2] for h in heads]), n, budget, window)",
     "keep = select_keep(heads[0][2], n, budget, window)"),
]

# Mathematically neutral edits: the pins must NOT reject these (softmax is
# invariant to a per-row or global shift; a mean over heads ranks as the sum).
NEUTRAL = {"max over the wrong axis", "rows reversed before the row mean",
           "shared: mean over heads"}


def _mutant(old, new):
    with open(SRC) as f:
        text = f.read()
    assert text.count(old) >= 1, f"mutation target vanished: {old!r}"
    text = text.replace(old, new, 1)
    mod = types.ModuleType("rkv_oracle_mutant")
    mod.__file__ = SRC
    exec(compile(text, SRC, "exec"), mod.__dict__)
    return mod


def _run_pins(mod):
    failed = []
    for pin in oracle_pins.ALL_PINS:
        try:
            pin(mod)
        except Exception as e:  # noqa: BLE001 - any failure counts as caught
            failed.append((pin.__name__, type(e).__name__))
    return failed


@pytest.mark.parametrize("name,old,new", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_mutant(name, old, new):
    failed = _run_pins(_mutant(old, new))
    if name in NEUTRAL:
        assert not failed, f"neutral edit rejected by {failed}"
    else:
        assert failed, f"mutant '{name}' survived every pin"
