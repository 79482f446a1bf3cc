"""bench.py's byte accounting and command line, without a GPU.

The algorithmic bytes that the bench divides by the kernel time are tied
here to the library's own record layout (gdn_records_bytes, a host call) and
to the tensor shapes of the workload, and the fused count to the two-call
count it replaces.
"""
import importlib.util
import os
import subprocess
import sys

import commit_gated_delta_amd as gdn

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _bench():
    spec = importlib.util.spec_from_file_location(
        "bench_under_test", os.path.join(ROOT, "bench.py"))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod


def test_window_bytes_follow_the_record_layout_and_shapes():
    b = _bench()
    dims = gdn.Dims.of(1, 1, b.HV, b.HK, b.DK, b.DV, 64)
    rec_tok = gdn.records_bytes(dims) / 64.0  # records of one token
    state = b.HV * b.DK * b.DV * 4
    inputs = 2 * b.HK * b.DK * 2 + b.HV * b.DV * 2 + 2 * b.HV * 4  # q k v, beta g
    out = b.HV * b.DV * 4                                        # o, f32
    per_tok = (b.alg_bytes_verify([2]) - b.alg_bytes_verify([1])) / b.NL
    # the library pads each record region to 256 bytes
    assert abs(per_tok - (inputs + out + rec_tok)) < 16
    assert b.alg_bytes_verify([0]) == b.NL * state


def test_kda_bytes_follow_the_kda_record_layout():
    b = _bench()
    dims = gdn.Dims.of(1, 1, b.HV, b.HK, b.DK, b.DV, 64)
    rec_tok = gdn.kda_records_bytes(dims) / 64.0
    inputs = (2 * b.HK * b.DK * 2 + b.HV * b.DV * 2 + b.HV * 4  # q k v, beta
              + b.HV * b.DK * 4)                                # per-channel g
    out = b.HV * b.DV * 4
    per_tok = (b.alg_bytes_kda_verify([2]) - b.alg_bytes_kda_verify([1])) / b.NL
    assert abs(per_tok - (inputs + out + rec_tok)) < 16
    per_rec = (b.alg_bytes_kda_commit([2]) - b.alg_bytes_kda_commit([1])) / b.NL
    assert abs(per_rec - rec_tok) < 16
    assert b.alg_bytes_kda_commit([1]) / b.NL > 2 * b.HV * b.DK * b.DV * 4


def test_verify_bytes_of_the_8_lane_t16_round():
    b = _bench()
    # 48 layers x 8 lanes: the 2 MiB state read plus 16 tokens of 57,856 B
    assert b.alg_bytes_verify([16] * 8) == 48 * 8 * (2 * 1024 * 1024 + 16 * 57856)


def test_fused_bytes_are_two_call_bytes_without_the_second_state_read():
    b = _bench()
    state = b.HV * b.DK * b.DV * 4
    t = [16, 3, 1, 16, 9, 12, 5, 16]
    m = [0, 3, 1, 16, 0, 7, 2, 11]
    committed = sum(1 for x in m if x > 0)
    assert b.alg_bytes_fused(t, m) == (b.alg_bytes_verify(t) + b.alg_bytes_commit(m)
                                       - b.NL * committed * state)
    assert b.alg_bytes_commit([0] * 8) == 0


def test_more_than_one_gpu_is_refused_with_a_message():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode != 0
    assert "one GPU" in r.stderr
