"""Host-side logic of bench.py: the code text that keys the committed traffic counters, the
algorithmic byte counts the roofline divides by, and the one-GPU contract."""
import subprocess
import sys
import os

import bench
from gated_deltanet_recurrent_02_amd import synth

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_code_text_drops_comments_and_keeps_literals():
    src = ('int a = 1; // one\n/* two\n   lines */ int b = 2;\n'
           'const char* s = "x // not a comment /* nor this */";\nchar c = \'/\';  int  d ;')
    assert bench.code_text(src) == ('int a = 1; int b = 2; const char* s = '
                                    '"x // not a comment /* nor this */"; char c = \'/\'; int d ;')


def test_code_text_sees_code_changes_only():
    a = "float f(float x) { return x * 2.0f; }  // doubles"
    assert bench.code_text(a) == bench.code_text("float f(float x) {\n  return x * 2.0f;\n}\n")
    assert bench.code_text(a) != bench.code_text("float f(float x) { return x * 3.0f; }")


def test_algorithmic_bytes_of_the_headline_workload():
    # B=256, H=48, D=128, T=1, fp32 state, bf16 q/k/v/o, fp32 alpha/beta: per head the state is
    # read and written once (2 * 64 KiB), q, k, v read once (3 * 256 B), alpha and beta (8 B),
    # o written (256 B).
    per_head = 2 * 128 * 128 * 4 + 3 * 128 * 2 + 8 + 128 * 2
    assert per_head == 132104
    spec = synth.WORKLOADS["decode_b256_h48_d128_t1"]
    assert bench.algorithmic_bytes(spec, "f32") == 256 * 48 * per_head == 1623293952


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120, cwd=ROOT)
    assert r.returncode != 0
    assert "one GPU" in (r.stdout + r.stderr)


def test_algorithmic_bytes_of_the_low_rank_workloads():
    # r = 16 slots, fp32 window, bf16 q/k/v/o, one token: per head the window is read once
    # (U and K: 2 * 16 * 128 * 4 B, weights 16 * 4 B, pos 4 B); the token's slot (U and K rows,
    # 2 * 128 * 4 B), every weight and pos are written; q, k, v, alpha, beta read, o written.
    read = 2 * 16 * 128 * 4 + 16 * 4 + 4
    write = 2 * 128 * 4 + 16 * 4 + 4
    token = 3 * 128 * 2 + 8 + 128 * 2
    assert read + write + token == 18576
    spec = synth.WORKLOADS["lowrank_b256_h48_d128_r16_t1"]
    assert bench.algorithmic_bytes(spec, "f32") == 256 * 48 * 18576 == 228261888
    # four tokens write four slots; a bf16 window halves the U and K bytes
    spec4 = synth.WORKLOADS["lowrank_b256_h48_d128_r16_t4"]
    read16 = 2 * 16 * 128 * 2 + 16 * 4 + 4
    write16 = 4 * 2 * 128 * 2 + 16 * 4 + 4
    assert bench.algorithmic_bytes(spec4, "bf16") == 256 * 48 * (read16 + write16 + 4 * token)
