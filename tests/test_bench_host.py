"""Host-side logic of bench.py (CPU only): the per-expert byte count behind the
decode roofline and the rule that the stored HBM traffic figure is reported
only while the GEMM source it was measured on is unchanged."""

import importlib.util
import json
import os

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
    # A counter record names the source it was measured on by its SHA-256: the
    # figure is reported while that source is unchanged, and dropped after an edit.
    import hashlib

    b = _bench()
    src = tmp_path / "pkg" / "kernels.hip"
    src.parent.mkdir(parents=True)
    src.write_bytes(b"// a kernel source\n")
    rec = {"source": "pkg/kernels.hip", "source_sha256": hashlib.sha256(src.read_bytes()).hexdigest(),
           "kernels": {"120b_prefill/gate_up_wide": {"bytes": 723238121.0}}}
    (tmp_path / "profiles").mkdir()
    (tmp_path / "profiles" / "traffic.json").write_text(json.dumps(rec))
    b.ROOT = str(tmp_path)
    assert b.measured_traffic("120b_prefill", "gate_up_wide") == 723238121.0
    assert b.measured_traffic("120b_prefill", "no_such_kernel") is None
    src.write_bytes(src.read_bytes() + b"// edited\n")
    assert b.measured_traffic("120b_prefill", "gate_up_wide") is None
    # the committed record, if any, has the same form
    committed = os.path.join(ROOT, "profiles", "traffic.json")
    if os.path.exists(committed):
        rec = json.load(open(committed))
        assert {"source", "source_sha256", "kernels"} <= set(rec)


def test_tile_kinds_follow_the_library_policy():
    # Full 128-pair tiles for experts with >= 128 pairs in large batches; mid
    # tiles for 5..127 pairs; one streaming tile for 1..4.  Batches of 5..256
    # tokens take no full tiles, and no streaming tiles when they average at
    # least 16 pairs per expert; NVFP4 needs H and I multiples of 64 for full tiles.
    tk = _bench().tile_kinds
    c = [200, 127, 5, 4, 0]
    assert tk(c, 4096, 2880, 2880, 128, 4) == (200, 132, 2)
    assert tk(c, 4096, 2880, 2880, 128, 4, act="mxfp8_split") == (200, 132, 2)
    assert tk(c, 4096, 96, 2880, 128, 4, nvfp4=True) == (0, 332, 3)
    assert tk(c, 4096, 128, 2880, 128, 4, nvfp4=True) == (200, 132, 2)
    # 256 tokens x 4 over 32 experts: 32 pairs per expert on average -> mid tiles only
    assert tk([130, 3, 0], 256, 2880, 2880, 32, 4) == (0, 133, 2)
    # the same batch over 128 experts: 8 per expert -> streaming tiles stay
    assert tk([130, 3, 0], 256, 2880, 2880, 128, 4) == (0, 130, 1)
    # with MXFP8 activations small batches keep the full-tile launch
    assert tk([130, 3, 0], 256, 2880, 2880, 32, 4, act="mxfp8") == (130, 0, 0)
    # decode: streaming tiles only
    assert tk([1, 2, 1], 4, 2880, 2880, 32, 4) == (0, 0, 0)
