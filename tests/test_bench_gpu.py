"""bench.py on the GPU, shortened: its JSON line and its chained workloads.

* The bench with most legs left out prints exactly one JSON line. Its keys,
  types, units and roofline fields follow the bench contract, and `value`
  is the headline path's head-token updates over its step time.
* Each chained workload (one lane on four rotated state sets, eight ragged
  lanes, twelve lanes at T = 6) runs cut to a few rounds through the same
  code the bench uses:
  * the final commit of the sampled layer must equal, bit for bit, the
    debug state of a verify of its last window;
  * the fp64 oracle over the sampled chain must agree with the GPU's final
    state and last outputs within 2e-4.
"""
import importlib.util
import json
import os
import subprocess
import sys

import pytest

from tests.gpu_util import TOL

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():
    pytest.skip("no GPU", allow_module_level=True)

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def say(*a):
    print(*a, flush=True)


def _bench():
    spec = importlib.util.spec_from_file_location(
        "bench_under_test", os.path.join(ROOT, "bench.py"))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod


def test_bench_json_line_follows_the_contract():
    cmd = [sys.executable, os.path.join(ROOT, "bench.py"), "--steps", "3",
           "--warmup", "1", "--no-cpu", "--no-prefill", "--no-sweep",
           "--no-tree", "--no-kda", "--no-configs", "--no-general",
           "--no-token-verify", "--no-snapshot", "--no-clocks"]
    say("running", " ".join(cmd[1:]))
    r = subprocess.run(cmd, cwd=ROOT, capture_output=True, text=True,
                       timeout=240)
    assert r.returncode == 0, r.stderr[-2000:]
    lines = [x for x in r.stdout.splitlines() if x.startswith("{")]
    assert len(lines) == 1, r.stdout[-2000:]
    d = json.loads(lines[0])
    for key, typ in [("metric", str), ("value", float), ("unit", str),
                     ("n_gpus", int), ("steps", int), ("warmup", int),
                     ("ms_per_step", float), ("higher_is_better", bool),
                     ("scaling", str), ("dtype", str), ("data", str),
                     ("config", dict), ("roofline", dict)]:
        assert isinstance(d[key], typ), key
    b = _bench()
    assert d["metric"] == b.METRIC
    assert d["n_gpus"] == 1 and d["steps"] == 3 and d["warmup"] == 1
    assert d["higher_is_better"] is True and d["vs_baseline"] is None
    assert d["scaling"] in ("weak", "strong")
    assert "workload" in d["config"]
    upd = b.N * b.T * b.NL * b.HV
    assert abs(d["value"] - upd / (d["ms_per_step"] * 1e-3)) <= 1e-6 * d["value"]
    roof = d["roofline"]
    assert roof["bound"] == "hbm" and roof["unit"] == "GB/s"
    assert roof["peak"] == b.HBM_PEAK_GBS
    assert abs(roof["frac"] - roof["achieved"] / roof["peak"]) < 1e-12
    assert 0.0 < roof["frac"] < 1.0
    assert abs(roof["achieved"] - roof["alg_bytes_per_launch"]
               / (roof["avg_launch_ms"] * 1e-3) / 1e9) <= 1e-6 * roof["achieved"]
    say("  value %.4g, roofline frac %.3f" % (d["value"], roof["frac"]))


@pytest.mark.parametrize("name", ["one_lane_100_rounds", "eight_lanes_ragged",
                                  "twelve_lanes_t6_256_rounds"])
def test_chained_workload_short(name):
    b = _bench()
    cfg = dict(b.CHAIN_CONFIGS[name])
    cfg["rounds"] = 2 * cfg["n_sets"] + 1
    say("case", name, "rounds", cfg["rounds"])
    prev = torch.cuda.current_stream()
    torch.cuda.set_stream(torch.cuda.Stream())
    try:
        rec, sample = b.bench_chain(name, cfg, warmup=1)
    finally:
        torch.cuda.set_stream(prev)
    assert rec["bitexact_replay_sampled_layer"]
    par = b.oracle_chain_parity(sample)
    say("  S err %.2e  o err %.2e" % (par["max_rel_err_S"], par["max_rel_err_o"]))
    assert par["max_rel_err_S"] <= TOL and par["max_rel_err_o"] <= TOL
