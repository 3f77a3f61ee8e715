"""mx_quantize on the GPU against the oracle: codes and scales bit-exact."""

import numpy as np
import pytest
import torch

import microscaled_precision_gemm_amd as mx
from microscaled_precision_gemm_amd import synthetic as syn
from oracle import mx_oracle as O
from tests.parity import assert_mx_equal, say

pytestmark = pytest.mark.gpu

FMTS = ["e2m3", "e3m2", "e2m1", "e4m3", "e5m2"]
LAYOUTS = ["tiled", "rows"]


def _all_bf16_patterns() -> torch.Tensor:
    bits = torch.arange(65536, dtype=torch.int32).to(torch.int16)
    return bits.view(torch.bfloat16)


def _quantize_both(x_bf16_cpu: torch.Tensor, fmt: str, what: str, layout: str = "tiled"):
    say(f"quantize {what} {tuple(x_bf16_cpu.shape)} {fmt} {layout}")
    g = mx.mx_quantize(x_bf16_cpu.cuda(), fmt, layout)
    torch.cuda.synchronize()
    c, s = O.quantize(x_bf16_cpu.to(torch.float64).numpy(), fmt)
    assert_mx_equal(g, c, s, what)


@pytest.mark.parametrize("layout", LAYOUTS)
@pytest.mark.parametrize("fmt", FMTS)
def test_all_bf16_patterns_consecutive_blocks(fmt, layout):
    """All 65536 bf16 bit patterns, 32 consecutive patterns per block (shared
    sign and exponent: exercises the top binade, saturation, subnormal and
    zero blocks, and the Inf / NaN blocks)."""
    x = _all_bf16_patterns().reshape(2048, 32)
    _quantize_both(x, fmt, "all-bf16 consecutive", layout)
    # the same patterns as 128-wide rows (4 blocks per row), a ragged row count
    _quantize_both(x.reshape(512, 128)[:500], fmt, "all-bf16 rows of 128", layout)


@pytest.mark.parametrize("fmt", FMTS)
@pytest.mark.parametrize("shift", [0, 1, 2, 3, 4, 5, 6, 8, 12])
def test_all_bf16_patterns_fixed_scale_blocks(fmt, shift):
    """Every finite bf16 pattern lands in a block whose scale is fixed by an
    anchor 2**shift times the block's largest magnitude, so the elements fall
    `shift` binades below the top: every binade, subnormal and underflow case
    of the element rounding is swept."""
    pats = _all_bf16_patterns().to(torch.float32)
    pats = pats[torch.isfinite(pats)]
    n = pats.numel() // 31 * 31
    body = pats[:n].reshape(-1, 31)
    anchor = body.abs().amax(dim=1, keepdim=True) * (2.0 ** shift)
    anchor = torch.where(torch.isfinite(anchor), anchor, torch.full_like(anchor, 3.3895313892515355e38))
    x = torch.cat([anchor, body], dim=1).to(torch.bfloat16)
    _quantize_both(x, fmt, f"fixed-scale shift {shift}")


@pytest.mark.parametrize("layout", LAYOUTS)
@pytest.mark.parametrize("fmt", FMTS)
def test_f32_source_full_mantissa(fmt, layout):
    """fp32 sources (the fc1 epilogue's input type): random full-mantissa values
    over 200 binades, exact fp32 midpoints, subnormal and tiny blocks."""
    rng = np.random.default_rng(21)
    rows = 4096
    x = rng.standard_normal((rows, 64)).astype(np.float32)
    x *= np.exp2(rng.integers(-100, 100, size=(rows, 1))).astype(np.float32)
    # exact midpoints between E2M3 / E3M2 neighbours at the block scale (anchor 7.5 * 2^e)
    e = rng.integers(-60, 60, size=rows)
    x[:, 0] = np.ldexp(7.5, e).astype(np.float32)
    odd = rng.integers(0, 60, size=(rows, 8)) * 2 + 1
    x[:, 1:9] = np.ldexp(odd / 16.0, e[:, None]).astype(np.float32)
    x[::97] = (rng.standard_normal((len(x[::97]), 64)) * 2.0 ** -140).astype(np.float32)  # subnormal blocks
    x[::89, :32] = 0.0
    x[5, 3] = -0.0
    t = torch.from_numpy(x)
    say(f"quantize f32 {t.shape} {fmt} {layout}")
    g = mx.mx_quantize(t.cuda(), fmt, layout)
    torch.cuda.synchronize()
    c, s = O.quantize(x.astype(np.float64), fmt)
    assert_mx_equal(g, c, s, "f32 source")


@pytest.mark.parametrize("layout", LAYOUTS)
@pytest.mark.parametrize("fmt", FMTS)
def test_exact_ties_and_neighbours(fmt, layout):
    """Every midpoint between neighbouring magnitudes of the element type (the
    round-half-to-even cases), and the fp32 values just below and above it,
    in blocks whose scale an anchor at the largest magnitude fixes to 2**e,
    for scales across the E8M0 range; both signs; fp32 sources."""
    mags = O.magnitudes(fmt)
    mids = (mags[:-1] + mags[1:]) / 2
    rng = np.random.default_rng(len(mids))
    vals = np.concatenate([mids, np.nextafter(mids.astype(np.float32), np.float32(0)),
                           np.nextafter(mids.astype(np.float32), np.float32(np.inf)), mags]).astype(np.float32)
    vals = np.concatenate([vals, -vals])
    per = 31
    nblk = -(-len(vals) // per)
    vals = np.concatenate([vals, np.zeros(nblk * per - len(vals), np.float32)]).reshape(nblk, per)
    rows = []
    for e in (-120, -40, -3, 0, 5, 60, 100):
        blk = np.concatenate([np.full((nblk, 1), mags[-1], np.float32), vals], axis=1)
        rows.append(np.ldexp(blk.astype(np.float64), e).astype(np.float32))
    x = np.concatenate(rows)
    x = np.ascontiguousarray(x[:, rng.permutation(32)])  # the anchor anywhere in the block
    x = x.reshape(-1, 128) if x.shape[0] % 4 == 0 else x
    say(f"quantize ties {x.shape} {fmt} {layout}")
    g = mx.mx_quantize(torch.from_numpy(x).cuda(), fmt, layout)
    torch.cuda.synchronize()
    c, s = O.quantize(x.astype(np.float64), fmt)
    assert_mx_equal(g, c, s, "ties")


@pytest.mark.parametrize("fmt", FMTS)
def test_nonfinite_and_zero_blocks(fmt):
    x = torch.zeros(4, 96)
    x[0, 5] = float("inf")
    x[1, 40] = float("nan")
    x[2, 70] = -float("inf")
    x[3, :] = -0.0
    for dt in (torch.bfloat16, torch.float32):
      for layout in LAYOUTS:
        say(f"quantize non-finite {dt} {fmt} {layout}")
        g = mx.mx_quantize(x.to(dt).cuda(), fmt, layout)
        torch.cuda.synchronize()
        c, s = O.quantize(x.to(dt).to(torch.float64).numpy(), fmt)
        assert_mx_equal(g, c, s, f"non-finite {dt} {layout}")
        assert s[0, 0] == 0xFF and s[1, 1] == 0xFF and s[2, 2] == 0xFF and s[3, 0] == 0


def test_strided_rows_and_ragged_shapes():
    """Row stride > K, a single block, and a row count that is not a multiple
    of the launch granularity."""
    rng = np.random.default_rng(3)
    base = torch.from_numpy(rng.standard_normal((37, 200)).astype(np.float32)).to(torch.bfloat16)
    for k in (32, 96, 160):
        for layout in LAYOUTS:
            view = base.cuda()[:, :k]  # row stride 200 elements = 400 bytes (16-byte multiple)
            say(f"quantize strided k={k} {layout}")
            g = mx.mx_quantize(view, "e2m3", layout)
            torch.cuda.synchronize()
            c, s = O.quantize(base[:, :k].to(torch.float64).numpy(), "e2m3")
            assert_mx_equal(g, c, s, f"strided k={k} {layout}")


def test_empty_inputs_are_noops():
    for shape in ((0, 64), (5, 0)):
        for layout in LAYOUTS:
            say(f"quantize empty {shape} {layout}")
            g = mx.mx_quantize(torch.zeros(shape, dtype=torch.bfloat16, device="cuda"), "e2m3", layout)
            torch.cuda.synchronize()
            assert g.codes.numel() == 0 and g.scales.numel() == 0


@pytest.mark.parametrize("name", ["proj", "fc1", "fc2", "skinny"])
def test_workload_activations_and_weights(name):
    """The workloads' own activations and weights (full size on the GPU; the
    oracle checks a seeded sample of rows plus the first and last rows)."""
    w = syn.WORKLOADS[name]
    rng = np.random.default_rng(5)
    layout = "tiled"
    for which, fmt in (("a", "e2m3"), ("w", w.w_fmt)):
        t = syn.make_a(w) if which == "a" else syn.make_w(w)
        rows = np.unique(np.concatenate([[0, t.shape[0] - 1], rng.choice(t.shape[0], size=min(64, t.shape[0]), replace=False)]))
        say(f"quantize {name}.{which} {tuple(t.shape)} {fmt} {layout}")
        g = mx.mx_quantize(t.cuda(), fmt, layout)
        torch.cuda.synchronize()
        c, s = O.quantize(t[torch.from_numpy(rows)].to(torch.float64).numpy(), fmt)
        assert_mx_equal(g, c, s, f"{name}.{which}", rows=rows)
        del g, t
