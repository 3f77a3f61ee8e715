"""Shape-keyed tuning table for mx_gemm's launch configuration, persisted as JSON.

The Hedra post on Krea 3 (section "We tuned before writing custom kernels")
found library kernels falling back to a generic configuration for shapes
missing from their dispatch tables, and kept per-shape choices found by timing
candidates on real data.  This module does that for the knobs of mx_gemm that
are free to choose per shape (``MXGemmConfig``): the order in which output
tiles are handed to workgroups (group width and XCD remapping), which decides
which operand stages the tiles in flight share in each XCD's L2, and the tile
shape: 256 output features with 4 waves and one workgroup per CU, 128 with
two workgroups per CU (pays off where K is short and per-tile fixed costs
weigh more), or 256 with 8 waves, two per SIMD.

* ``tune_gemm`` times every candidate on the caller's own operands (HIP events
  on the current stream, after a warm-up), requires each candidate's output to
  be bit-identical to the default configuration's (neither the tile order nor
  the tile shape changes the arithmetic: each output takes the same matrix-core
  sequence over K; the check holds the library to that on the real data), and
  records the fastest, keeping the default unless a candidate beats
  it by more than ``margin``.
* ``TuningTable.lookup`` returns the recorded configuration for a call; for
  a shape never tuned, the configuration of the nearest tuned shape of the
  same GEMM (same device, K, element formats, epilogue and output kind; the
  closest M x N); with no such entry, None, and mx_gemm then applies the
  library's shape rule (``mx_gemm_select_config``), never the generic
  configuration blindly.
* ``tune_gemm`` warm-starts by default: the search starts from that nearest
  entry (the post tunes a new request size starting from the earlier
  optimizations of the same GEMM), or from the shape rule, and times that
  seed, the rule's pick, the generic configuration and the candidates one
  knob away from the seed, instead of every candidate.
* ``TuningTable.save`` / ``load`` persist the table as JSON; entries are keyed
  by the device's ISA name and compute-unit count, so a table carried to other
  hardware is not applied there.
* ``SHIPPED_TABLE`` is the table tuned on MI355X (gfx950, 256 CUs) for the
  workload shapes, shipped with the package so that a run uses the same
  configurations every time: several candidates are within run-to-run noise
  of each other on some shapes.
"""

from __future__ import annotations

import json
import math
import os
import tempfile

import torch

from .binding import MXGemmConfig, MXTensor, mx_gemm, mx_gemm_default_config, mx_gemm_select_config

# (group_m, xcd_remap, tile_n, waves)
CANDIDATES = ((4, 1, 256, 4), (2, 1, 256, 4), (8, 1, 256, 4), (16, 1, 256, 4), (1, 1, 256, 4), (4, 0, 256, 4),
              (8, 0, 256, 4),
              (4, 1, 128, 4), (2, 1, 128, 4), (8, 1, 128, 4), (16, 1, 128, 4),
              (4, 1, 256, 8), (2, 1, 256, 8), (8, 1, 256, 8))
FORMAT_VERSION = 3
SHIPPED_TABLE = os.path.join(os.path.dirname(os.path.abspath(__file__)), "tuned_gfx950.json")
FP6 = ("e2m3", "e3m2")


def supports(config: tuple[int, int, int, int], a_fmt: str, w_fmt: str, epilogue: str) -> bool:
    """Whether mx_gemm accepts this configuration for the call: 128-feature
    tiles take 6-bit operands (every epilogue) and 4 waves; 256-feature tiles
    take 4 or 8 waves (every pair and epilogue)."""
    _, _, tile_n, waves = config
    if tile_n == 128:
        return waves == 4 and a_fmt in FP6 and w_fmt in FP6
    return waves in (4, 8)


def device_name(device: torch.device | None = None) -> str:
    """The device part of a table key: the ISA name and the compute-unit count
    (the marketing name is generic on some boards and empty under some
    profilers)."""
    p = torch.cuda.get_device_properties(device)
    arch = (getattr(p, "gcnArchName", "") or "").split(":")[0]
    return f"{arch or p.name or 'gpu'}/{p.multi_processor_count}cu"


def gemm_key(m: int, n: int, k: int, a_fmt: str, w_fmt: str, epilogue: str, out_kind: str, out_fmt: str,
             device: str) -> str:
    """Table key of one mx_gemm call shape (output format only matters for MX outputs)."""
    of = out_fmt if out_kind == "mx" else "-"
    return f"{device}|{m}x{n}x{k}|a={a_fmt}|w={w_fmt}|epi={epilogue}|out={out_kind}:{of}"


def split_key(key: str) -> tuple[str, int, int, int, str]:
    """(device, m, n, k, the rest of the key) of a table key."""
    device, shape, rest = key.split("|", 2)
    m, n, k = (int(v) for v in shape.split("x"))
    return device, m, n, k, rest


def neighbours(config: tuple[int, int, int, int], a_fmt: str, w_fmt: str, epilogue: str) -> list:
    """The candidates one knob away from ``config``: the tile walk's group
    width halved or doubled, the XCD remapping flipped, or the other tile
    shapes with the same walk."""
    g, x, t, wv = config
    out = [(max(1, g // 2), x, t, wv), (min(16, g * 2), x, t, wv), (g, 1 - x, t, wv)]
    out += [(g, x, tt, ww) for tt, ww in ((256, 4), (128, 4), (256, 8)) if (tt, ww) != (t, wv)]
    return [c for c in dict.fromkeys(out) if c != config and supports(c, a_fmt, w_fmt, epilogue)]


class TuningTable:
    """Per-shape launch configurations of mx_gemm."""

    def __init__(self, path: str | None = None):
        self.path = path
        self.entries: dict[str, dict] = {}
        if path is not None and os.path.exists(path):
            self.load(path)

    def lookup(self, m, n, k, a_fmt="e2m3", w_fmt="e2m3", epilogue="none", out_kind="bf16", out_fmt="e2m3",
               device: str | None = None) -> MXGemmConfig | None:
        """The configuration for this call: its own entry, else the nearest
        tuned shape of the same GEMM, else None (the library's shape rule)."""
        key = self.source(m, n, k, a_fmt, w_fmt, epilogue, out_kind, out_fmt, device)
        return None if key is None else MXGemmConfig(*self.entries[key]["config"])

    def source(self, m, n, k, a_fmt="e2m3", w_fmt="e2m3", epilogue="none", out_kind="bf16", out_fmt="e2m3",
               device: str | None = None) -> str | None:
        """Key of the entry lookup() takes its configuration from: the call's
        own key, or the entry of the same device, K, formats, epilogue and
        output kind whose M x N is closest in log scale (ties: the closer N,
        then the key order), or None."""
        device = device or device_name()
        key = gemm_key(m, n, k, a_fmt, w_fmt, epilogue, out_kind, out_fmt, device)
        if key in self.entries:
            return key
        rest = split_key(key)[4]
        best, best_d = None, None
        for other in sorted(self.entries):
            dv, om, on, ok, orest = split_key(other)
            if dv != device or ok != k or orest != rest:
                continue
            d = (abs(math.log2(om * on) - math.log2(max(1, m * n))), abs(math.log2(on) - math.log2(max(1, n))))
            if best_d is None or d < best_d:
                best, best_d = other, d
        return best

    def record(self, key: str, entry: dict) -> None:
        self.entries[key] = entry

    def save(self, path: str | None = None) -> str:
        path = path or self.path
        if path is None:
            raise ValueError("no path to save the tuning table to")
        d = os.path.dirname(os.path.abspath(path))
        os.makedirs(d, exist_ok=True)
        fd, tmp = tempfile.mkstemp(dir=d, prefix=".tuning-", suffix=".json")
        with os.fdopen(fd, "w") as f:
            json.dump({"format": FORMAT_VERSION, "entries": self.entries}, f, indent=1, sort_keys=True)
        os.replace(tmp, path)
        return path

    def load(self, path: str) -> None:
        with open(path) as f:
            data = json.load(f)
        if data.get("format") != FORMAT_VERSION:
            raise ValueError(f"{path}: unknown tuning table format {data.get('format')!r}")
        for key, e in data["entries"].items():
            cfg = e.get("config")
            if not (isinstance(cfg, list) and len(cfg) == 4 and 1 <= cfg[0] <= 16 and cfg[1] in (0, 1)
                    and cfg[2] in (128, 256) and cfg[3] in (4, 8) and not (cfg[2] == 128 and cfg[3] == 8)):
                raise ValueError(f"{path}: bad entry {key!r}")
        self.entries.update(data["entries"])

    def gemm(self, a, w: MXTensor, out_kind: str = "bf16", epilogue: str = "none", out_fmt: str = "e2m3",
             a_fmt: str = "e2m3", **kw):
        """mx_gemm with this table's configuration for the call's shape (the
        library default when the shape was never tuned)."""
        m = a.rows if isinstance(a, MXTensor) else a.shape[0]
        af = a.fmt if isinstance(a, MXTensor) else a_fmt
        cfg = self.lookup(m, w.rows, w.k, af, w.fmt, epilogue, out_kind, out_fmt)
        return mx_gemm(a, w, out_kind=out_kind, epilogue=epilogue, out_fmt=out_fmt, a_fmt=a_fmt, config=cfg, **kw)


def _same(x, y) -> bool:
    if isinstance(x, MXTensor):
        return torch.equal(x.codes, y.codes) and torch.equal(x.scales, y.scales)
    return torch.equal(x, y)


def _time_us(fn, iters: int) -> float:
    start, stop = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    start.record()
    for _ in range(iters):
        fn()
    stop.record()
    torch.cuda.synchronize()
    return start.elapsed_time(stop) * 1e3 / iters


def tune_gemm(table: TuningTable, a: MXTensor, w: MXTensor, out_kind: str = "bf16", epilogue: str = "none",
              out_fmt: str = "e2m3", candidates=None, iters: int = 10, rounds: int = 3,
              margin: float = 0.01, warm_start: bool = True) -> dict:
    """Time the candidate configurations this call supports on these operands
    and record the fastest in ``table`` (see the module docstring).  With
    ``candidates`` None: a warm-started search (the seed, its neighbours, the
    shape rule's pick and the generic configuration) when ``warm_start``,
    else every candidate.  Returns the recorded entry; raises if a
    candidate's output differs from the generic configuration's."""
    default = mx_gemm_default_config().key()
    rule = mx_gemm_select_config(a.rows, w.rows, w.k, a.fmt, w.fmt, epilogue, out_kind).key()
    seed_key = table.source(a.rows, w.rows, w.k, a.fmt, w.fmt, epilogue, out_kind, out_fmt)
    if candidates is None and warm_start:
        seed = tuple(table.entries[seed_key]["config"]) if seed_key is not None else rule
        candidates = [seed, rule] + neighbours(seed, a.fmt, w.fmt, epilogue)
    elif candidates is None:
        candidates = CANDIDATES
    cands = [default] + [c for c in dict.fromkeys(map(tuple, candidates))
                         if c != default and supports(c, a.fmt, w.fmt, epilogue)]
    ref = mx_gemm(a, w, out_kind=out_kind, epilogue=epilogue, out_fmt=out_fmt, config=default)
    outs = {c: mx_gemm(a, w, out_kind=out_kind, epilogue=epilogue, out_fmt=out_fmt, config=c) for c in cands}
    torch.cuda.synchronize()
    for c, o in outs.items():
        if not _same(o, ref):
            raise RuntimeError(f"configuration {c} changed the result of mx_gemm; not recorded")
    for _ in range(3):  # warm-up, and let the clocks settle
        for c in cands:
            mx_gemm(a, w, out_kind=out_kind, epilogue=epilogue, out_fmt=out_fmt, out=outs[c], config=c)
    torch.cuda.synchronize()
    best = {c: float("inf") for c in cands}
    for _ in range(rounds):  # interleaved rounds: drifting clocks hit every candidate alike
        for c in cands:
            t = _time_us(lambda: mx_gemm(a, w, out_kind=out_kind, epilogue=epilogue, out_fmt=out_fmt, out=outs[c],
                                         config=c), iters)
            best[c] = min(best[c], t)
    pick = min(cands, key=lambda c: best[c])
    if best[pick] > best[default] * (1.0 - margin):
        pick = default
    entry = {"config": list(pick), "us": round(best[pick], 2), "default_us": round(best[default], 2),
             "candidates": {",".join(map(str, c)): round(t, 2) for c, t in best.items()},
             "seeded_from": seed_key if warm_start else None}
    key = gemm_key(a.rows, w.rows, w.k, a.fmt, w.fmt, epilogue, out_kind, out_fmt, device_name())
    table.record(key, entry)
    return entry
