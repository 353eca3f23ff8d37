"""bench.py on the CPU: the one-GPU rule and the algorithmic byte counts behind its
roofline.

The byte counts are fixed by what each call must move (the seam block's inputs
and outputs at hidden 5120, four streams, 24 logits): per token the residual
40,960 B and layer_input 10,240 B, the gates 96 B (pre-mix, post, comb) plus the
carried pre-mix 16 B when delayed; per call the float32 weight 1,966,080 B,
bias and alpha 108 B and the norm weight 10,240 B; the post stage reads y and x
and writes the next residual (92,160 B) plus its gates (80 B)."""
import os
import subprocess
import sys

import bench

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_exits_with_a_message():
    for n in (2, 8):
        r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", str(n)],
                           capture_output=True, text=True, cwd=ROOT, timeout=120)
        assert r.returncode == 2, r
        assert "one GPU only" in r.stderr
        assert r.stdout == ""


def test_algorithmic_bytes():
    # own pre-mix, no norm, 8 tokens
    assert bench.pre_bytes(8, norm=False, delayed=False) == 8 * 51_296 + 1_966_188 == 2_376_556
    # delayed with norm: decode and prefill sizes
    assert bench.pre_bytes(128) == 128 * 51_312 + 1_976_428 == 8_544_364
    assert bench.pre_bytes(16384) == 842_672_236
    # post stage
    assert bench.post_bytes(16384) == 16384 * 92_240 == 1_511_260_160
    # the seam as two calls, and as one: the fused call still writes the next
    # residual (the next seam reads it) but does not read it back (40,960 B per
    # token fewer: 143,552 -> 102,592 B per token)
    assert bench.pre_bytes(16384) + bench.post_bytes(16384) == 2_353_932_396
    assert bench.pre_bytes(16384) + bench.post_bytes(16384) - bench.fused_bytes(16384) == 16384 * 40_960
    assert bench.fused_bytes(16384) == 16384 * 102_592 + 1_976_428
    # entry: h in, four-stream residual, layer_input and gates out; the narrower weight
    assert bench.entry_bytes(1) == 10_240 + 40_960 + 10_240 + 96 + 491_520 + 108 + 10_240
    # other hidden sizes: 20 C + 192 bytes per token, 96 (4 C) + 108 + 2 C per call
    assert bench.fused_bytes(16384, 7168) == 16384 * 143_552 + 2_766_956
    assert bench.fused_bytes(16384, 4096) == 16384 * 82_112 + 1_581_164


def test_ceiling_probe_library_exports():
    """bench_ceilings.so (the benchmark's memory-ceiling probes, built by
    __graft_entry__.build()) loads and exports its two entry points; argument
    checks reject bad calls before any launch."""
    import ctypes
    path = os.path.join(ROOT, "bench_ceilings.so")
    if not os.path.exists(path):
        import pytest
        pytest.skip("bench_ceilings.so not built")
    L = ctypes.CDLL(path)
    P, I, Z = ctypes.c_void_p, ctypes.c_int, ctypes.c_size_t
    L.ceil_stream.argtypes = [I, P, P, Z, P, P]
    L.ceil_pattern_run.argtypes = [I, P, P, P, P, I, I, P]
    fake = ctypes.c_void_p(1 << 40)   # never dereferenced: every call below fails validation
    assert L.ceil_stream(3, fake, fake, 16, fake, None) == -1          # unknown kind
    assert L.ceil_stream(0, fake, fake, 15, fake, None) == -1          # not a multiple of 16
    assert L.ceil_stream(0, None, fake, 16, fake, None) == -1          # read needs a source
    assert L.ceil_stream(2, fake, None, 16, fake, None) == -1          # copy needs a destination
    assert L.ceil_stream(1, fake, fake, 16, None, None) == -1          # no sink
    assert L.ceil_pattern_run(1, fake, fake, fake, fake, 0, 16, None) == -1     # T < 1
    assert L.ceil_pattern_run(1, fake, fake, fake, fake, 64, 17, None) == -1    # too many groups
    assert L.ceil_pattern_run(1, fake, None, fake, fake, 64, 16, None) == -1    # fused needs y
