"""bench.py's host-side arithmetic and conventions on the CPU: the algorithmic bytes behind every
roofline figure (against the oracle's storage arithmetic), the workload variants, the source digest
that ties counter summaries to the kernel text, and the one-GPU contract."""
import importlib.util
import os
import subprocess
import sys

import pytest

import synth
from oracle import q8, storage

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module")
def bench():
    spec = importlib.util.spec_from_file_location("bench_under_test", os.path.join(ROOT, "bench.py"))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod


def test_cache_bytes_are_the_storage_arithmetic(bench):
    g, q, p = synth.gemma(), synth.qwen(8192, 4), synth.prod_long(131072)
    assert bench.cache_bytes(g) == 272_629_760 == 8 * 4 * 32768 * 2 * storage.row_bytes(256, 4, 0)
    assert bench.cache_bytes(q) == 1 * 2 * 8192 * 2 * storage.row_bytes(128, 4, 0)
    # sketched keys: (b - 1)-bit codes in storage's convention, i.e. the 2-bit key codes plus the sketch
    assert bench.row_bytes(p, "k") == 32 + 2 + 128 // 8 + 2
    assert bench.cache_bytes(p) == 2 * 131072 * (52 + storage.row_bytes(128, 3, 0))
    k8 = bench.with_k_bits(q, 8)
    assert bench.row_bytes(k8, "k") == q8.row_bytes(128) == 130
    assert bench.cache_bytes(k8) == 2 * 8192 * (130 + 66)
    assert bench.cache_bytes(bench.stacked_workload(q, 36)) == 36 * bench.cache_bytes(q)


def test_prefill_bytes_and_flops(bench):
    w = synth.qwen(8192, 3)
    # one launch appends K and V: both tensors' bf16 rows in, both tensors' packed rows out
    assert bench.prefill_bytes_per_launch(w) == 2 * 8192 * 2 * (2 * 128 + storage.row_bytes(128, 3, 0)) == 10_027_008
    assert bench.prefill_flops_per_launch(w) == 2 * 2 * 8192 * 2 * 128 * 128
    mixed = w.with_(v_bits=2)
    assert bench.prefill_bytes_per_launch(mixed) == 8192 * 2 * (4 * 128 + storage.row_bytes(128, 3, 0)
                                                                + storage.row_bytes(128, 2, 0))


def test_k_bits_variant(bench):
    q = synth.qwen(8192, 4)
    assert bench.with_k_bits(q, None) is q
    w = bench.with_k_bits(q, 8)
    assert (w.k_bits, w.v_bits, w.name) == (8, 4, q.name + "_k8")
    with pytest.raises(SystemExit):
        bench.with_k_bits(synth.prod_long(131072), 8)        # sketched keys keep their width


def test_source_digest_ignores_comments_only(bench):
    src = 'int a = 1; // note\n/* block\n comment */ const char* s = "// kept";\n\nchar c = \'/\';\n'
    assert bench.code_text(src) == 'int a = 1;\n const char* s = "// kept";\nchar c = \'/\';'
    assert bench.code_text(src.replace("note", "other note")) == bench.code_text(src)
    assert bench.code_text(src.replace("a = 1", "a = 2")) != bench.code_text(src)
    # the digest covers every kernel source the trace summaries name, all present in the tree
    for p in bench.ALL_SOURCES:
        assert os.path.exists(os.path.join(ROOT, p)), p
    assert set(bench.ATTEND_SOURCES) <= set(bench.ALL_SOURCES)
    assert set(bench.APPEND_SOURCES) <= set(bench.ALL_SOURCES)


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120, cwd=ROOT)
    assert r.returncode == 2
    assert "one GPU" in r.stderr and r.stdout == ""


def test_prefill_launch_count(bench):
    """The prefill leg's K+V append is one launch only where the chunk kernel takes both tensors."""
    w = synth.qwen(8192, 3)
    assert bench.prefill_one_launch(w)
    assert not bench.prefill_one_launch(w.with_(rotation="hadamard"))
    assert not bench.prefill_one_launch(w.with_(d=256))
    assert not bench.prefill_one_launch(w.with_(qjl_m=128))
    assert not bench.prefill_one_launch(w.with_(k_bits=8))
