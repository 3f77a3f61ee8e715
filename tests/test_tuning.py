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


def test_candidates_the_call_supports():
    # 128-feature tiles exist for the 6-bit pairs (every epilogue); 8 waves
    # for 256-feature tiles of every pair, without SwiGLU
    assert T.supports((4, 1, 128, 4), "e2m3", "e3m2", "gelu_tanh")
    assert T.supports((4, 1, 128, 4), "e2m3", "e2m3", "swiglu")
    assert not T.supports((4, 1, 128, 4), "e4m3", "e4m3", "none")
    assert not T.supports((4, 1, 128, 8), "e2m3", "e2m3", "none")
    assert T.supports((4, 1, 256, 4), "e2m1", "e2m1", "none")
    assert T.supports((4, 1, 256, 8), "e4m3", "e5m2", "none")
    assert T.supports((4, 1, 256, 4), "e2m3", "e2m3", "swiglu")
    assert not T.supports((4, 1, 256, 8), "e2m3", "e2m3", "swiglu")
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
    entry = T.tune_gemm(table, a, w, out_kind="mx", epilogue="gelu_tanh", iters=3, rounds=2)
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
             dict(m=4096, n=3072, k=3072)]
    calls += [dict(m=20480, n=12288, k=3072, a_fmt=f, w_fmt=f) for f in ("e2m3", "e2m1", "e4m3")]
    for c in calls:
        cfg = t.lookup(device=dev, **c)
        assert cfg is not None, c
        af, wf, epi = c.get("a_fmt", "e2m3"), c.get("w_fmt", "e2m3"), c.get("epilogue", "none")
        assert T.supports(cfg.key(), af, wf, epi), (c, cfg.key())
