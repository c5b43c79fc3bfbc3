"""The C ABI on a machine without a GPU: the library loads, exports every
function include/rkv.h declares, and rejects bad arguments before it touches
the device (no compute call is made here)."""
import ctypes
import math
import os
import re

import numpy as np
import pytest

from kv_cache_compression_decode_amd import binding as B

pytestmark = pytest.mark.cpu

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "rkv.h")


def header_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(rkv_[a-z_]+)\s*\(", text)))


def test_library_exports_every_declared_function():
    lib = B.load()
    declared = header_functions()
    assert declared, "no declarations parsed"
    assert set(declared) == set(B.EXPORTS)
    for name in declared:
        assert hasattr(lib, name), name


def test_header_constants_match_binding():
    text = open(HEADER).read()
    assert int(re.search(r"#define RKV_MAX_LEN (\d+)", text).group(1)) == B.RKV_MAX_LEN
    assert int(re.search(r"#define RKV_MAX_WINDOW_ROWS (\d+)", text).group(1)) == B.RKV_MAX_WINDOW_ROWS


def test_header_flag_constants_match_binding():
    text = open(HEADER).read()
    for name in ("RKV_DEVICE_SPAN_TIMEOUT", "RKV_DEVICE_BAD_BLOCK_ID"):
        assert int(re.search(rf"#define {name} (\d+)u", text).group(1)) == getattr(B, name)
    assert int(re.search(r"RKV_ERR_DEVICE_CHECK = (\d+)", text).group(1)) == B.RKV_ERR_DEVICE_CHECK


def test_struct_layouts(tmp_path):
    """The ctypes structures have the sizes and field offsets a C compiler
    gives the header's structures (gcc, host only)."""
    import subprocess
    fields = {"rkv_config": [f[0] for f in B.rkv_config._fields_],
              "rkv_cache": [f[0] for f in B.rkv_cache._fields_],
              "rkv_kara_config": [f[0] for f in B.rkv_kara_config._fields_]}
    lines = ['#include <stdio.h>', '#include <stddef.h>', '#include "rkv.h"', 'int main(void) {']
    for st, names in fields.items():
        lines.append(f'  printf("{st} size %zu\\n", sizeof({st}));')
        for f in names:
            lines.append(f'  printf("{st} {f} %zu\\n", offsetof({st}, {f}));')
    lines += ['  return 0;', '}']
    src = tmp_path / "layout.c"
    src.write_text("\n".join(lines) + "\n")
    exe = tmp_path / "layout"
    subprocess.run(["gcc", "-std=c99", "-I", os.path.join(ROOT, "include"), str(src), "-o", str(exe)],
                   check=True)
    out = subprocess.run([str(exe)], check=True, capture_output=True, text=True).stdout.split("\n")
    got = {tuple(l.split()[:2]): int(l.split()[2]) for l in out if l}
    for st, cls in (("rkv_config", B.rkv_config), ("rkv_cache", B.rkv_cache),
                    ("rkv_kara_config", B.rkv_kara_config)):
        assert got[(st, "size")] == ctypes.sizeof(cls), st
        for f in fields[st]:
            assert got[(st, f)] == getattr(cls, f).offset, (st, f)


def test_status_strings():
    for s, name in [(0, "RKV_OK"), (1, "RKV_ERR_INVALID_ARG"), (2, "RKV_ERR_UNSUPPORTED"),
                    (3, "RKV_ERR_WORKSPACE"), (4, "RKV_ERR_HIP"), (5, "RKV_ERR_DEVICE_CHECK")]:
        assert B.rkv_status_string(s) == name


def cfg(**kw):
    base = dict(num_layers=32, num_q_heads=32, num_kv_heads=8, head_dim=128, budget=1024,
                buffer=128, window=8, mix_lambda=0.1)
    base.update(kw)
    dtype = base.pop("dtype", "bf16")
    layout = base.pop("layout", "contiguous")
    bs = base.pop("block_size", 16)
    shared = base.pop("shared_selection", False)
    return B.make_config(**base, dtype=dtype, layout=layout, block_size=bs, shared_selection=shared)


FAKE = 1 << 20          # a 16-byte aligned, never dereferenced address


def cache(**kw):
    return B.make_cache(kw.get("k", FAKE), kw.get("v", FAKE), kw.get("capacity", 2048),
                        kw.get("num_blocks", 0), kw.get("block_table", None),
                        kw.get("max_blocks", 0), kw.get("layer_stride", 0))


def test_trigger_rule():
    c = cfg()
    assert B.rkv_is_triggered(c, 1151) == 0
    assert B.rkv_is_triggered(c, 1152) == 1
    assert B.rkv_is_triggered(c, 5000) == 1


def test_workspace_size_formula():
    c = cfg()
    # the 256-byte status block, then one record of 2*G*w + d floats per
    # (unit, 256-key chunk), 256-byte rounded
    n = B.rkv_workspace_size(c, 1, 1152)
    assert n == 256 + 1 * 32 * 8 * math.ceil(1152 / 256) * (2 * 4 * 8 + 128) * 4
    assert B.rkv_workspace_size(c, 200, 1152) == B.rkv_workspace_size(c, 128, 1152)
    assert B.rkv_workspace_size(cfg(head_dim=96), 1, 1152) == 0


def expect(status, fn, *a, **kw):
    with pytest.raises(B.RkvError) as e:
        fn(*a, **kw)
    assert e.value.status == status, e.value
    assert e.value.detail


def score(c, ca=None, lens=(1152,), q=FAKE, scores=FAKE, stride=1152, ws=FAKE * 4, wsb=1 << 30):
    B.rkv_score(c, cache() if ca is None else ca, q, len(lens), list(lens), scores, stride,
                None, None, ws, wsb, None)


@pytest.mark.parametrize("bad,status", [
    (dict(head_dim=96), B.RKV_ERR_UNSUPPORTED),
    (dict(num_q_heads=30), B.RKV_ERR_INVALID_ARG),
    (dict(budget=8), B.RKV_ERR_INVALID_ARG),
    (dict(window=0), B.RKV_ERR_INVALID_ARG),
    (dict(buffer=0), B.RKV_ERR_INVALID_ARG),
    (dict(mix_lambda=1.5), B.RKV_ERR_INVALID_ARG),
    (dict(mix_lambda=-0.1), B.RKV_ERR_INVALID_ARG),
    (dict(mix_lambda=float("nan")), B.RKV_ERR_INVALID_ARG),
    (dict(num_layers=0), B.RKV_ERR_INVALID_ARG),
    (dict(window=16, num_q_heads=80, num_kv_heads=8), B.RKV_ERR_UNSUPPORTED),
    (dict(layout="paged", block_size=24), B.RKV_ERR_UNSUPPORTED),
    (dict(budget=40000), B.RKV_ERR_UNSUPPORTED),
])
def test_config_rejected(bad, status):
    expect(status, score, cfg(**bad))


def test_shared_selection_flag_checked():
    c = cfg()
    c.shared_selection = 2
    expect(B.RKV_ERR_INVALID_ARG, score, c)
    assert B.make_config(1, 4, 1, 64, 128, 32, 8, 0.1, shared_selection=True).shared_selection == 1
    assert cfg().shared_selection == 0


def test_argument_errors():
    c = cfg()
    expect(B.RKV_ERR_INVALID_ARG, score, c, ca=cache(k=None))
    expect(B.RKV_ERR_INVALID_ARG, score, c, ca=cache(k=FAKE + 8))          # misaligned
    expect(B.RKV_ERR_INVALID_ARG, score, c, ca=cache(capacity=1000))       # len > capacity
    expect(B.RKV_ERR_INVALID_ARG, score, c, q=None)
    expect(B.RKV_ERR_INVALID_ARG, score, c, scores=None)
    expect(B.RKV_ERR_INVALID_ARG, score, c, stride=1000)
    expect(B.RKV_ERR_INVALID_ARG, score, c, lens=(1152, -1))
    expect(B.RKV_ERR_UNSUPPORTED, score, c, lens=(40000,), ca=cache(capacity=50000), stride=40000)
    expect(B.RKV_ERR_WORKSPACE, score, c, ws=None)
    expect(B.RKV_ERR_WORKSPACE, score, c, wsb=1000)
    expect(B.RKV_ERR_WORKSPACE, score, c, ws=FAKE * 4 + 16)               # misaligned
    expect(B.RKV_ERR_INVALID_ARG, B.rkv_select, c, 1, [1152], None, 1152, FAKE)
    expect(B.RKV_ERR_INVALID_ARG, B.rkv_select, c, 1, [1152], FAKE, 1152, None)
    expect(B.RKV_ERR_INVALID_ARG, B.rkv_select, c, 1, [1152], FAKE, 100, FAKE)
    lens = np.array([1152], np.int32)
    expect(B.RKV_ERR_INVALID_ARG, B.rkv_compact, c, cache(v=None), 1, lens, FAKE)
    expect(B.RKV_ERR_INVALID_ARG, B.rkv_compact, c, cache(), 1, lens, None)
    assert lens[0] == 1152, "failed call changed the lengths"
    pc = cfg(layout="paged")
    expect(B.RKV_ERR_INVALID_ARG, B.rkv_compact, pc, cache(num_blocks=100, max_blocks=72), 1, lens, FAKE)
    pca = cache(num_blocks=100, block_table=FAKE, max_blocks=72)
    # 1152 tokens -> 72 blocks, budget 1024 -> 64 blocks: 8 freed
    expect(B.RKV_ERR_INVALID_ARG, B.rkv_compact, pc, pca, 1, lens, FAKE, FAKE, 7)
    expect(B.RKV_ERR_INVALID_ARG, B.rkv_compact, pc, pca, 1, lens, FAKE, None, 8)
    expect(B.RKV_ERR_INVALID_ARG, B.rkv_compact, pc, cache(num_blocks=100, block_table=FAKE,
                                                             max_blocks=71), 1, lens, FAKE, FAKE, 8)


def test_nothing_triggered_is_a_no_op():
    """Below the trigger nothing is enqueued (safe without a GPU) and lengths stay."""
    c = cfg()
    lens = np.array([1151, 17, 0], np.int32)
    B.rkv_score(c, cache(), FAKE, 3, lens, FAKE, 1152, None, None, FAKE * 4, 1 << 30, None)
    B.rkv_select(c, 3, lens, FAKE, 1152, FAKE, None)
    counts = np.full(3, -1, np.int32)
    B.rkv_compact(c, cache(), 3, lens, FAKE, None, 0, counts, None)
    assert list(lens) == [1151, 17, 0]
    assert list(counts) == [0, 0, 0]
    B.rkv_score(c, cache(), None, 0, None, None, 0, None, None, None, 0, None)


def test_layer_stride_checked():
    """layer_stride: 0 (packed), or at least one packed layer and a multiple of
    16 bytes."""
    c = cfg()
    packed = 1 * 8 * 2048 * 128                      # S * Hkv * capacity * d
    expect(B.RKV_ERR_INVALID_ARG, score, c, ca=cache(layer_stride=-8))
    expect(B.RKV_ERR_INVALID_ARG, score, c, ca=cache(layer_stride=packed + 4))   # 8 bytes
    expect(B.RKV_ERR_INVALID_ARG, score, c, ca=cache(layer_stride=packed - 8))
    expect(B.RKV_ERR_INVALID_ARG, gram, c, ca=cache(layer_stride=packed - 8))
    lens = np.array([1152], np.int32)
    expect(B.RKV_ERR_INVALID_ARG, B.rkv_compact, c, cache(layer_stride=packed - 8), 1, lens, FAKE)
    expect(B.RKV_ERR_INVALID_ARG, B.rkv_step, c, cache(layer_stride=7), FAKE, 1, lens, FAKE, 1152,
           FAKE)
    fc = cfg(dtype="f32")
    expect(B.RKV_ERR_INVALID_ARG, score, fc, ca=cache(layer_stride=packed + 2))  # 8 bytes
    pc = cfg(layout="paged")
    ppacked = 100 * 8 * 16 * 128                     # num_blocks * Hkv * block_size * d
    expect(B.RKV_ERR_INVALID_ARG, score, pc, ca=cache(num_blocks=100, block_table=FAKE,
                                                       max_blocks=72, layer_stride=ppacked - 8))
    assert lens[0] == 1152


def test_check_block_table_flag():
    c = cfg(layout="paged")
    c.check_block_table = 2
    pca = cache(num_blocks=100, block_table=FAKE, max_blocks=72)
    expect(B.RKV_ERR_INVALID_ARG, score, c, ca=pca)
    c.check_block_table = 1
    lens = np.array([1152], np.int32)
    # the device check needs a workspace for its status word
    expect(B.RKV_ERR_WORKSPACE, B.rkv_step, c, pca, FAKE, 1, lens, FAKE, 1152, FAKE, FAKE, 8)
    expect(B.RKV_ERR_WORKSPACE, B.rkv_compact, c, pca, 1, lens, FAKE, FAKE, 8)
    assert lens[0] == 1152
    assert B.make_config(1, 4, 1, 64, 128, 32, 8, 0.1, layout="paged",
                         check_block_table=True).check_block_table == 1


def test_status_workspace_checked():
    """rkv_select and rkv_compact accept no workspace, or a 256-byte aligned
    one of at least 256 bytes; the status query needs one."""
    c = cfg()
    lens = np.array([1152], np.int32)
    expect(B.RKV_ERR_WORKSPACE, B.rkv_select, c, 1, lens, FAKE, 1152, FAKE, FAKE * 4 + 16, 4096)
    expect(B.RKV_ERR_WORKSPACE, B.rkv_select, c, 1, lens, FAKE, 1152, FAKE, FAKE * 4, 128)
    expect(B.RKV_ERR_WORKSPACE, B.rkv_compact, c, cache(), 1, lens, FAKE, None, 0, None,
           FAKE * 4 + 16, 4096)
    assert lens[0] == 1152


def test_span_wait_bound():
    prev = B.rkv_set_span_wait_us(0)
    try:
        assert prev == 1000000
        assert B.rkv_set_span_wait_us(-1) == -1
        assert B.rkv_set_span_wait_us(60000001) == -1
        assert B.rkv_set_span_wait_us(250) == 0
        assert B.rkv_set_span_wait_us(prev) == 250
    finally:
        B.rkv_set_span_wait_us(1000000)


def test_binding_requires_inplace_lengths():
    with pytest.raises(TypeError):
        B.rkv_compact(cfg(), cache(), 1, [1152], FAKE)


def step_dev(c, ca=None, n=1, lens=FAKE, max_len=1152, stride=1152, keep=FAKE, fb=None, cap=0,
             ws=FAKE * 4, wsb=1 << 30):
    B.rkv_step_device(c, cache() if ca is None else ca, FAKE, n, lens, max_len, FAKE, stride,
                      keep, fb, cap, None, ws, wsb, None)


def test_step_device_workspace_size():
    c = cfg()
    table = (1 + 3 * 4) * 4
    table = 256 + (table + 255) // 256 * 256     # the status block, then the table
    # fused at this shape (bf16, N <= 1280, G*w = 32): only the table
    assert B.rkv_step_device_workspace_size(c, 4, 1152) == table
    # not fused (N > 1280): plus one record per (unit, 256-key chunk) for every sequence
    rec = 4 * 32 * 8 * math.ceil(2000 / 256) * (2 * 4 * 8 + 128) * 4
    assert B.rkv_step_device_workspace_size(c, 4, 2000) == table + (rec + 255) // 256 * 256
    # head-shared selection never runs fused
    assert B.rkv_step_device_workspace_size(cfg(shared_selection=True), 4, 1152) > table
    assert B.rkv_step_device_workspace_size(c, 4, 40000) == 0


def test_step_device_argument_errors():
    """Every argument is checked on the host before anything is enqueued."""
    c = cfg()
    expect(B.RKV_ERR_INVALID_ARG, step_dev, c, lens=None)
    expect(B.RKV_ERR_INVALID_ARG, step_dev, c, max_len=-1)
    expect(B.RKV_ERR_UNSUPPORTED, step_dev, c, max_len=40000, ca=cache(capacity=50000), stride=40000)
    expect(B.RKV_ERR_INVALID_ARG, step_dev, c, max_len=3000)                 # > capacity 2048
    expect(B.RKV_ERR_INVALID_ARG, step_dev, c, stride=1000)
    expect(B.RKV_ERR_INVALID_ARG, step_dev, c, keep=None)
    expect(B.RKV_ERR_WORKSPACE, step_dev, c, ws=None)
    expect(B.RKV_ERR_WORKSPACE, step_dev, c, wsb=16)
    expect(B.RKV_ERR_WORKSPACE, step_dev, c, ws=FAKE * 4 + 16)
    pc = cfg(layout="paged")
    pca = cache(num_blocks=100, block_table=FAKE, max_blocks=72)
    # worst case: 2 sequences at 1152 tokens, 8 blocks freed each
    expect(B.RKV_ERR_INVALID_ARG, step_dev, pc, ca=pca, n=2, fb=FAKE, cap=15)
    expect(B.RKV_ERR_INVALID_ARG, step_dev, pc, ca=pca, n=2, fb=None, cap=16)
    expect(B.RKV_ERR_INVALID_ARG, step_dev, pc, ca=cache(num_blocks=100, block_table=FAKE,
                                                          max_blocks=71), n=2, fb=FAKE, cap=16)
    step_dev(c, n=0)   # no sequences: nothing to do, nothing enqueued


def gram(c, ca=None, lens=(1152,), red=FAKE, stride=1152):
    B.rkv_redundancy_gram(c, cache() if ca is None else ca, len(lens), list(lens), red, stride,
                          None)


def test_gram_argument_errors():
    c = cfg()
    expect(B.RKV_ERR_UNSUPPORTED, gram, cfg(dtype="f32"))
    expect(B.RKV_ERR_UNSUPPORTED, gram, cfg(head_dim=96))
    expect(B.RKV_ERR_INVALID_ARG, gram, c, ca=cache(k=None))
    expect(B.RKV_ERR_INVALID_ARG, gram, c, ca=cache(k=FAKE + 8))          # misaligned
    expect(B.RKV_ERR_INVALID_ARG, gram, c, ca=cache(capacity=1000))
    expect(B.RKV_ERR_INVALID_ARG, gram, c, red=None)
    expect(B.RKV_ERR_INVALID_ARG, gram, c, stride=1000)
    expect(B.RKV_ERR_INVALID_ARG, gram, c, lens=(1152, -1))
    expect(B.RKV_ERR_UNSUPPORTED, gram, c, lens=(40000,), ca=cache(capacity=50000), stride=40000)
    gram(c, lens=(1151, 9), red=None)   # nothing triggered: nothing enqueued


def wstore(c, layer0=0, count=32, q=FAKE, n=1, steps=FAKE, ring=FAKE * 4):
    B.rkv_window_store(c, layer0, count, q, n, steps, ring, None)


def test_window_store_argument_errors():
    c = cfg()
    expect(B.RKV_ERR_INVALID_ARG, wstore, c, layer0=-1)
    expect(B.RKV_ERR_INVALID_ARG, wstore, c, layer0=1, count=32)      # past the last layer
    expect(B.RKV_ERR_INVALID_ARG, wstore, c, count=-1)
    expect(B.RKV_ERR_INVALID_ARG, wstore, c, n=-1)
    expect(B.RKV_ERR_INVALID_ARG, wstore, c, q=None)
    expect(B.RKV_ERR_INVALID_ARG, wstore, c, steps=None)
    expect(B.RKV_ERR_INVALID_ARG, wstore, c, ring=None)
    expect(B.RKV_ERR_INVALID_ARG, wstore, c, q=FAKE + 8)              # misaligned
    expect(B.RKV_ERR_INVALID_ARG, wstore, c, ring=FAKE * 4 + 8)
    expect(B.RKV_ERR_INVALID_ARG, wstore, c, steps=FAKE + 2)
    expect(B.RKV_ERR_UNSUPPORTED, wstore, cfg(head_dim=96))
    wstore(c, n=0, q=None, steps=None, ring=None)                     # nothing to store
    wstore(c, count=0, q=None, steps=None, ring=None)


def test_membench_library_exports_its_header():
    """The measurement-only streaming kernels: librkv_membench.so exports what
    include/rkv_membench.h declares and rejects bad arguments before any launch."""
    path = os.path.join(ROOT, "kv_cache_compression_decode_amd", "librkv_membench.so")
    lib = ctypes.CDLL(path)
    text = re.sub(r"/\*.*?\*/", "", open(os.path.join(ROOT, "include", "rkv_membench.h")).read(),
                  flags=re.S)
    declared = sorted(set(re.findall(r"\b(rkv_[a-z_]+)\s*\(", text)))
    assert declared == ["rkv_membench_copy", "rkv_membench_read"]
    for name in declared:
        assert hasattr(lib, name)
    lib.rkv_membench_read.argtypes = [ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p,
                                      ctypes.c_int32, ctypes.c_void_p]
    lib.rkv_membench_copy.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_size_t,
                                      ctypes.c_int32, ctypes.c_void_p]
    assert lib.rkv_membench_read(None, 16, FAKE, 0, None) == -1
    assert lib.rkv_membench_read(FAKE + 4, 16, FAKE, 0, None) == -1
    assert lib.rkv_membench_read(FAKE, 17, FAKE, 0, None) == -1
    assert lib.rkv_membench_copy(FAKE, FAKE, 8, 0, None) == -1
    assert lib.rkv_membench_copy(FAKE, FAKE, 0, 0, None) == 0       # nothing to do


def kara(c, kc, ca=None, lens=(1152,), tails=(1024,), q=FAKE, scores=FAKE, keep=FAKE, fb=None, cap=0,
         ws=None, wsb=0):
    B.rkv_kara_step(c, kc, cache() if ca is None else ca, q, len(lens), np.array(lens, np.int32),
                    np.array(tails, np.int32), scores, keep, fb, cap, None, ws, wsb, None)


def test_kara_argument_errors():
    """rkv_kara_step checks everything before it enqueues anything."""
    c = cfg()
    good = B.rkv_kara_config(128, 32, 4, 2)
    expect(B.RKV_ERR_UNSUPPORTED, kara, cfg(dtype="f32"), good)
    expect(B.RKV_ERR_UNSUPPORTED, kara, c, B.rkv_kara_config(96, 32, 4, 2))
    expect(B.RKV_ERR_INVALID_ARG, kara, c, B.rkv_kara_config(128, 0, 0, 0))
    expect(B.RKV_ERR_INVALID_ARG, kara, c, B.rkv_kara_config(128, 129, 0, 0))
    expect(B.RKV_ERR_INVALID_ARG, kara, c, B.rkv_kara_config(128, 32, 4, 4))   # 4 * 9 > 32
    expect(B.RKV_ERR_INVALID_ARG, kara, c, B.rkv_kara_config(128, 32, -1, 0))
    expect(B.RKV_ERR_INVALID_ARG, kara, c, good, tails=(1200,))               # tail past the end
    expect(B.RKV_ERR_INVALID_ARG, kara, c, good, q=None)
    expect(B.RKV_ERR_INVALID_ARG, kara, c, good, keep=None)
    expect(B.RKV_ERR_INVALID_ARG, kara, c, good, ca=cache(capacity=1000))
    pc = cfg(layout="paged")
    pca = cache(num_blocks=100, block_table=FAKE, max_blocks=72)
    # 1152 -> 1056 tokens at bs 16: 72 -> 66 blocks, 6 freed
    expect(B.RKV_ERR_INVALID_ARG, kara, pc, good, ca=pca, fb=FAKE, cap=5)
    pc.check_block_table = 1
    expect(B.RKV_ERR_WORKSPACE, kara, pc, good, ca=pca, fb=FAKE, cap=6)
    # below the trigger nothing is enqueued and nothing changes
    lens = np.array([1151, 100], np.int32)
    tails = np.array([1024, 0], np.int32)
    B.rkv_kara_step(c, good, cache(), None, 2, lens, tails, None, None, None, 0, None, None, 0, None)
    assert list(lens) == [1151, 100] and list(tails) == [1024, 0]
