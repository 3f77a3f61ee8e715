"""The shape-keyed tuning table: host-side behaviour (no GPU) and, on a GPU,
tuning a real call (every candidate bit-identical to the default; the
recorded choice is applied and survives a save / load round trip)."""

import json

import pytest
import torch

import microscaled_precision_gemm_amd as mx
from microscaled_precision_gemm_amd import tuning as T


def test_key_names_every_dimension():
    k = T.gemm_key(20480, 12288, 3072, "e2m3", "e2m3", "gelu_tanh", "mx", "e2m3", "dev0")
    assert k == "dev0|20480x12288x3072|a=e2m3|w=e2m3|epi=gelu_tanh|out=mx:e2m3"
    # the output element format only matters for MX outputs
    assert T.gemm_key(1, 2, 32, "e2m3", "e3m2", "none", "bf16", "e3m2", "d") == \
        T.gemm_key(1, 2, 32, "e2m3", "e3m2", "none", "bf16", "e2m3", "d")


def test_save_load_round_trip(tmp_path):
    t = T.TuningTable()
    key = T.gemm_key(256, 512, 1024, "e2m3", "e2m3", "none", "bf16", "e2m3", "devX")
    t.record(key, {"config": [8, 1, 128, 4], "us": 12.5, "default_us": 13.0,
                   "candidates": {"4,1,256,4": 13.0, "8,1,128,4": 12.5}})
    p = t.save(str(tmp_path / "sub" / "tuning.json"))
    u = T.TuningTable(p)
    assert u.lookup(256, 512, 1024, device="devX").key() == (8, 1, 128, 4)
    assert u.lookup(256, 512, 1024, device="other") is None  # entries are per device
    assert u.lookup(256, 512, 2048, device="devX") is None  # untuned shape: library default


def test_untuned_shape_takes_the_nearest_entry_of_the_same_gemm():
    """A call shape missing from the table takes the configuration of the
    tuned shape of the same GEMM (device, K, formats, epilogue, output) with
    the closest M x N, never one of another GEMM; with none, the library's
    shape rule applies (lookup returns None)."""
    t = T.TuningTable()
    dev = "devX"
    fc1 = dict(k=3072, epilogue="gelu_tanh", out_kind="mx")
    t.record(T.gemm_key(20480, 12288, 3072, "e2m3", "e2m3", "gelu_tanh", "mx", "e2m3", dev),
             {"config": [8, 1, 128, 4], "us": 1.0, "default_us": 1.0, "candidates": {}})
    t.record(T.gemm_key(512, 12288, 3072, "e2m3", "e2m3", "gelu_tanh", "mx", "e2m3", dev),
             {"config": [2, 1, 256, 8], "us": 1.0, "default_us": 1.0, "candidates": {}})
    t.record(T.gemm_key(2560, 12288, 3072, "e2m3", "e2m3", "none", "bf16", "e2m3", dev),
             {"config": [16, 0, 256, 4], "us": 1.0, "default_us": 1.0, "candidates": {}})
    # 2560 tokens: log2 distance 3 to 20480, 2.3 to 512 -> the 512 entry; 8192: the 20480 one
    assert t.source(2560, 12288, device=dev, **fc1).startswith(f"{dev}|512x")
    assert t.lookup(2560, 12288, device=dev, **fc1).key() == (2, 1, 256, 8)
    assert t.lookup(8192, 12288, device=dev, **fc1).key() == (8, 1, 128, 4)
    assert t.lookup(20480, 12288, device=dev, **fc1).key() == (8, 1, 128, 4)  # its own entry
    # another GEMM at the same M x N is never borrowed
    assert t.lookup(2560, 12288, 6144, epilogue="gelu_tanh", out_kind="mx", device=dev) is None  # other K
    assert t.lookup(2560, 12288, 3072, epilogue="gelu_tanh", out_kind="mx", out_fmt="e3m2", device=dev) is None
    assert t.lookup(2560, 12288, 3072, a_fmt="e3m2", epilogue="gelu_tanh", out_kind="mx", device=dev) is None
    assert t.lookup(2560, 12288, 3072, device=dev).key() == (16, 0, 256, 4)  # the bf16 GEMM's own entry
    assert t.lookup(2560, 12288, 3072, epilogue="gelu_tanh", out_kind="mx", device="devY") is None


def test_neighbours_change_one_knob():
    n = T.neighbours((8, 1, 128, 4), "e2m3", "e2m3", "gelu_tanh")
    assert set(n) == {(4, 1, 128, 4), (16, 1, 128, 4), (8, 0, 128, 4), (8, 1, 256, 4), (8, 1, 256, 8)}
    # FP8 operands have no 128-feature tiles; SwiGLU has every tile shape
    assert all(c[2] == 256 for c in T.neighbours((4, 1, 256, 4), "e4m3", "e4m3", "none"))
    assert {(c[2], c[3]) for c in T.neighbours((4, 1, 256, 4), "e2m3", "e2m3", "swiglu")} >= {(128, 4), (256, 8)}
    assert (1, 1, 256, 4) not in T.neighbours((1, 1, 256, 4), "e2m3", "e2m3", "none")


def test_library_shape_rule():
    """mx_gemm_select_config (what mx_gemm uses when given no configuration)
    picks the choices tuned on the workload shapes, and only configurations
    the call supports."""
    sel = mx.mx_gemm_select_config
    assert sel(20480, 12288, 3072, epilogue="gelu_tanh", out_kind="mx").key() == (8, 1, 256, 8)
    assert sel(2560, 12288, 3072, epilogue="none", out_kind="mx").key() == (8, 1, 256, 8)
    assert sel(20480, 3072, 12288, epilogue="none", out_kind="bf16").key() == (4, 1, 256, 8)
    assert sel(4096, 3072, 3072).key() == (4, 1, 256, 8)
    assert sel(20480, 12288, 3072, "e2m1", "e2m1").key() == (4, 1, 256, 8)
    assert sel(20480, 12288, 3072, "e4m3", "e4m3").key() == (4, 1, 256, 4)
    assert sel(20480, 16384, 3072, epilogue="swiglu", out_kind="mx").key() == (4, 1, 256, 8)
    assert sel(20480, 12288, 8192, epilogue="gelu_tanh", out_kind="mx").key() == (8, 1, 256, 8)
    assert mx.mx_gemm_default_config().key() == (4, 1, 256, 4)
    for af, wf in (("e2m3", "e2m3"), ("e3m2", "e2m3"), ("e2m1", "e2m1"), ("e5m2", "e4m3")):
        for epi, out in (("none", "bf16"), ("none", "f32"), ("gelu_tanh", "mx"), ("swiglu", "mx"), ("none", "mx")):
            for k in (128, 3072, 16384):
                if epi != "none" or out == "mx":
                    if af not in ("e2m3", "e3m2"):
                        continue
                assert T.supports(sel(4096, 4096, k, af, wf, epi, out).key(), af, wf, epi), (af, wf, epi, out, k)


def test_candidates_the_call_supports():
    # 128-feature tiles exist for the 6-bit pairs (every epilogue); 8 waves
    # for 256-feature tiles of every pair and epilogue
    assert T.supports((4, 1, 128, 4), "e2m3", "e3m2", "gelu_tanh")
    assert T.supports((4, 1, 128, 4), "e2m3", "e2m3", "swiglu")
    assert not T.supports((4, 1, 128, 4), "e4m3", "e4m3", "none")
    assert not T.supports((4, 1, 128, 8), "e2m3", "e2m3", "none")
    assert T.supports((4, 1, 256, 4), "e2m1", "e2m1", "none")
    assert T.supports((4, 1, 256, 8), "e4m3", "e5m2", "none")
    assert T.supports((4, 1, 256, 4), "e2m3", "e2m3", "swiglu")
    assert T.supports((4, 1, 256, 8), "e2m3", "e2m3", "swiglu")
    assert T.CANDIDATES[0] == (4, 1, 256, 4)
    assert {(c[2], c[3]) for c in T.CANDIDATES} == {(256, 4), (128, 4), (256, 8)}


def test_load_rejects_bad_entries(tmp_path):
    p = tmp_path / "bad.json"
    for cfg in ([0, 1, 256, 4], [4, 1, 64, 4], [4, 1, 256], [4, 1, 128, 8], [4, 1, 256, 6]):
        p.write_text(json.dumps({"format": T.FORMAT_VERSION, "entries": {"k": {"config": cfg}}}))
        with pytest.raises(ValueError):
            T.TuningTable(str(p))
    p.write_text(json.dumps({"format": 99, "entries": {}}))
    with pytest.raises(ValueError):
        T.TuningTable(str(p))


@pytest.mark.gpu
def test_tune_real_call_and_apply(tmp_path):
    from tests.parity import say
    torch.manual_seed(0)
    m, k, n = 2048, 512, 2048  # 8 x 8 tiles: the XCD remapping applies
    a = mx.mx_quantize(torch.randn(m, k, device="cuda").to(torch.bfloat16), "e2m3")
    w = mx.mx_quantize((torch.randn(n, k, device="cuda") * 0.05).to(torch.bfloat16), "e2m3")
    say("tuning 2048x512x2048 gelu->mx")
    table = T.TuningTable(str(tmp_path / "t.json"))
    entry = T.tune_gemm(table, a, w, out_kind="mx", epilogue="gelu_tanh", iters=3, rounds=2, warm_start=False)
    assert set(entry["candidates"]) >= {"4,1,256,4", "8,1,256,4", "1,1,256,4", "4,0,256,4", "4,1,128,4",
                                        "4,1,256,8"}
    cfg = table.lookup(m, n, k, epilogue="gelu_tanh", out_kind="mx")
    assert cfg is not None and cfg.key() == tuple(entry["config"])
    got = table.gemm(a, w, out_kind="mx", epilogue="gelu_tanh")
    ref = mx.mx_gemm(a, w, out_kind="mx", epilogue="gelu_tanh")
    torch.cuda.synchronize()
    assert torch.equal(got.codes, ref.codes) and torch.equal(got.scales, ref.scales)
    table.save()
    assert T.TuningTable(str(tmp_path / "t.json")).lookup(m, n, k, epilogue="gelu_tanh", out_kind="mx").key() == cfg.key()
    # a configuration outside the documented ranges is refused by the library
    with pytest.raises(mx.MXError):
        mx.mx_gemm(a, w, out_kind="bf16", config=(0, 1))
    with pytest.raises(mx.MXError):
        mx.mx_gemm(a, w, out_kind="bf16", config=(4, 2))
    with pytest.raises(mx.MXError):
        mx.mx_gemm(a, w, out_kind="bf16", config=(4, 1, 64))
    with pytest.raises(mx.MXError):
        mx.mx_gemm(a, w, out_kind="bf16", config=(4, 1, 128, 8))


def test_shipped_table_covers_the_workloads():
    """The table shipped with the package loads, is keyed for gfx950, and holds
    a valid configuration for every GEMM shape the bench runs."""
    t = T.TuningTable(T.SHIPPED_TABLE)
    dev = "gfx950/256cu"
    calls = [dict(m=20480, n=12288, k=3072, epilogue="gelu_tanh", out_kind="mx"),
             dict(m=20480, n=3072, k=12288),
             dict(m=20480, n=16384, k=3072, epilogue="swiglu", out_kind="mx"),
             dict(m=20480, n=3072, k=8192),
             dict(m=4096, n=3072, k=3072),
             dict(m=2560, n=12288, k=3072, epilogue="gelu_tanh", out_kind="mx"),
             dict(m=2560, n=3072, k=12288)]
    calls += [dict(m=20480, n=12288, k=3072, a_fmt=f, w_fmt=f) for f in ("e2m3", "e2m1", "e4m3")]
    for c in calls:
        cfg = t.lookup(device=dev, **c)
        assert cfg is not None, c
        af, wf, epi = c.get("a_fmt", "e2m3"), c.get("w_fmt", "e2m3"), c.get("epilogue", "none")
        assert T.supports(cfg.key(), af, wf, epi), (c, cfg.key())


@pytest.mark.gpu
def test_warm_start_for_an_untuned_token_count():
    """12288 tokens (a shorter sequence than the workload's 20480) is not in
    the shipped table.  lookup() gives it the configuration of the nearest
    tuned fc1 shape, the 20480-token entry (not the generic one), whose output
    is bit-identical to the generic configuration's and to the shape rule's; a
    warm-started tune starts from that entry and keeps a configuration no
    slower than the generic one."""
    from tests.parity import say
    torch.manual_seed(1)
    m, k, n = 12288, 3072, 12288
    shipped = T.TuningTable(T.SHIPPED_TABLE)
    dev = T.device_name()
    src = shipped.source(m, n, k, epilogue="gelu_tanh", out_kind="mx")
    if not dev.startswith("gfx950/"):
        pytest.skip(f"the shipped table is for gfx950, this is {dev}")
    assert src == T.gemm_key(20480, n, k, "e2m3", "e2m3", "gelu_tanh", "mx", "e2m3", dev)
    cfg = shipped.lookup(m, n, k, epilogue="gelu_tanh", out_kind="mx")
    assert cfg.key() != mx.mx_gemm_default_config().key()
    a = mx.mx_quantize(torch.randn(m, k, device="cuda").to(torch.bfloat16), "e2m3")
    w = mx.mx_quantize((torch.randn(n, k, device="cuda") * 0.02).to(torch.bfloat16), "e2m3")
    say("warm-started tuning 12288x3072x12288 gelu->mx")
    outs = [mx.mx_gemm(a, w, out_kind="mx", epilogue="gelu_tanh", config=c)
            for c in (cfg, mx.mx_gemm_default_config(), None)]
    torch.cuda.synchronize()
    for o in outs[1:]:
        assert torch.equal(o.codes, outs[0].codes) and torch.equal(o.scales, outs[0].scales)
    entry = T.tune_gemm(shipped, a, w, out_kind="mx", epilogue="gelu_tanh", iters=5, rounds=3)
    print("warm start", {k_: v for k_, v in entry.items()})
    assert entry["seeded_from"] == src
    assert ",".join(map(str, cfg.key())) in entry["candidates"]
    assert len(entry["candidates"]) < len(T.CANDIDATES)
    assert entry["us"] <= entry["default_us"]
    # the table-derived configuration itself is no slower than the generic one (5 % timing noise)
    assert entry["candidates"][",".join(map(str, cfg.key()))] <= 1.05 * entry["default_us"]
