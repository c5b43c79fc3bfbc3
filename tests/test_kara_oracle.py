"""The KARA-style window oracle against its pins, and planted mistakes in a
copy of it that the pins must catch (CPU only)."""
import os
import types

import pytest

import kara_pins
from oracle import kara_oracle

pytestmark = pytest.mark.cpu

SRC = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "oracle",
                   "kara_oracle.py")


@pytest.mark.parametrize("pin", kara_pins.ALL_PINS, ids=lambda f: f.__name__)
def test_pin(pin):
    pin(kara_oracle)


MUTANTS = [
    ("causal mask in the window", "    logits = logits - logits.max(axis=1, keepdims=True)\n",
     "    logits = logits + np.triu(np.full(logits.shape, -np.inf), 1)\n"
     "    logits = logits - logits.max(axis=1, keepdims=True)\n"),
    ("softmax over the rows", "p = p / p.sum(axis=1, keepdims=True)", "p = p / p.sum(axis=0, keepdims=True)"),
    ("sum instead of mean", "    return p.mean(axis=0)", "    return p.sum(axis=0)"),
    ("no 1/sqrt(d)", "logits = (q_rows @ k_window.T) / math.sqrt(d)", "logits = (q_rows @ k_window.T)"),
    ("anchors from the worst", "for a in order[:anchors]:", "for a in order[::-1][:anchors]:"),
    ("chunk one short on the right", "in_chunk[max(0, a - radius): min(w, a + radius + 1)] = True",
     "in_chunk[max(0, a - radius): min(w, a + radius)] = True"),
    ("chunk not clipped at 0", "in_chunk[max(0, a - radius): min(w, a + radius + 1)] = True",
     "in_chunk[a - radius: min(w, a + radius + 1)] = True"),
    ("fill ignores the chunk count", "kept[rest[: keep - int(in_chunk.sum())]] = True",
     "kept[rest[: keep]] = True"),
    ("fill may repeat chunk tokens", "rest = [int(j) for j in order if not in_chunk[j]]",
     "rest = [int(j) for j in order]"),
    ("ties keep the later position", "return np.lexsort((np.arange(len(s)), -s))",
     "return np.lexsort((-np.arange(len(s)), -s))"),
    ("trigger strict", "return int(n) - int(tail_start) >= int(window_len)",
     "return int(n) - int(tail_start) > int(window_len)"),
    ("new length drops the prefix", "return int(n) - int(window_len) + int(keep)", "return int(keep)"),
    ("free blocks floor", "first = -(-int(n_new) // block_size)", "first = int(n_new) // block_size"),
    ("window taken from the front", "kw, vw = k_rows[n - w:n], v_rows[n - w:n]", "kw, vw = k_rows[:w], v_rows[:w]"),
    ("GQA group ignored", "q = q_group_window(_decode(q_tail_sl, dtype), h, group)",
     "q = q_group_window(_decode(q_tail_sl, dtype), h, 1)"),
    ("bf16 decode without the 16-bit shift", "astype(np.uint32) << np.uint32(16)",
     "astype(np.uint32) << np.uint32(8)"),
    ("bf16 decode drops the sign", "w = np.asarray(x, dtype=np.uint16).astype(np.uint32) << np.uint32(16)",
     "w = (np.asarray(x, dtype=np.uint16).astype(np.uint32) & np.uint32(0x7FFF)) << np.uint32(16)"),
    ("bf16 decode with swapped bytes", "w = np.asarray(x, dtype=np.uint16).astype",
     "w = np.asarray(x, dtype=np.uint16).byteswap().astype"),
    ("f32 decode through half precision", "return np.asarray(x, dtype=np.float32).astype(np.float64)",
     "return np.asarray(x, dtype=np.float32).astype(np.float16).astype(np.float64)"),
    ("step_unit returns widened rows", "return unit_step(q, _decode(kw, dtype), kw, vw,",
     "return unit_step(q, _decode(kw, dtype), _decode(kw, dtype), vw,"),
]


def _mutant(old, new):
    text = open(SRC).read()
    assert text.count(old) == 1, f"mutation target: {old!r}"
    mod = types.ModuleType("kara_oracle_mutant")
    mod.__file__ = SRC
    exec(compile(text.replace(old, new), SRC, "exec"), mod.__dict__)
    return mod


@pytest.mark.parametrize("name,old,new", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_mutant_is_caught(name, old, new):
    mod = _mutant(old, new)
    failed = []
    for pin in kara_pins.ALL_PINS:
        try:
            pin(mod)
        except Exception as e:  # noqa: BLE001 - any failure counts as caught
            failed.append(pin.__name__)
    assert failed, f"mutant '{name}' survived every pin"
