"""Host-side logic of bench.py (CPU only): the per-expert byte count behind the
decode roofline and the rule that the stored HBM traffic figure is reported
only while the GEMM source it was measured on is unchanged."""

import importlib.util
import json
import os
import shutil

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _bench():
    spec = importlib.util.spec_from_file_location("bench_under_test", os.path.join(ROOT, "bench.py"))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod


def test_layer_bytes_at_gpt_oss_shapes():
    # H = I = 2880: w13 blocks 8,294,400 + scales 518,400 + bias 11,520 and w2
    # blocks 4,147,200 + scales 259,200 + bias 5,760 = 13,236,480 bytes per expert
    w13, w2 = _bench().layer_bytes(2880, 2880)
    assert (w13, w2) == (8_824_320, 4_412_160)
    assert w13 + w2 == 13_236_480
    # NVFP4: one E4M3 scale per 16 elements and a float32 second-level scale per tensor
    n13, n2 = _bench().layer_bytes(2880, 2880, nvfp4=True)
    assert (n13 - w13, n2 - w2) == (518_400 + 4, 259_200 + 4)


def test_traffic_reported_only_for_the_profiled_source(tmp_path):
    b = _bench()
    rec = json.load(open(os.path.join(ROOT, "profiles", "traffic.json")))
    key = "120b_prefill/gate_up_wide"
    assert b.measured_traffic("120b_prefill", "gate_up_wide") == float(rec["kernels"][key]["bytes"])
    assert b.measured_traffic("120b_prefill", "no_such_kernel") is None
    # the same record next to an edited copy of the source: no figure
    (tmp_path / "profiles").mkdir()
    shutil.copy(os.path.join(ROOT, "profiles", "traffic.json"), tmp_path / "profiles" / "traffic.json")
    src = tmp_path / rec["source"]
    src.parent.mkdir(parents=True)
    src.write_bytes(open(os.path.join(ROOT, rec["source"]), "rb").read() + b"\n// edited\n")
    b.ROOT = str(tmp_path)
    assert b.measured_traffic("120b_prefill", "gate_up_wide") is None
