"""Host-side pieces of bench.py's JSON line (no GPU): the timed kernels'
names follow the launch configuration, and the measured HBM traffic is
reported only for the kernel and the GEMM sources the committed counter
summary was taken of."""

import bench
from microscaled_precision_gemm_amd import tuning as T
from microscaled_precision_gemm_amd.binding import MXGemmConfig


def test_kernel_names_follow_the_configuration():
    assert bench.kernel_name("fc1", None) == "gemm_kernel<2, 2, 2, 1, 2, 256, 4>"
    assert bench.kernel_name("fc1", MXGemmConfig(8, 1, 128, 4)) == "gemm_kernel<2, 2, 2, 1, 2, 128, 4>"
    assert bench.kernel_name("fc2", MXGemmConfig(4, 1, 256, 8)) == "gemm_kernel<2, 2, 1, 0, 2, 256, 8>"


def test_traffic_only_for_the_profiled_kernel(monkeypatch):
    text = open(bench.TRAFFIC_FILE).read()
    recorded = {g: line.split(": ", 1)[1].strip() for g in ("fc1", "fc2")
                for line in text.splitlines() if line.startswith(f"{g}_kernel: ")}
    assert set(recorded) == {"fc1", "fc2"}
    for gemm, kernel in recorded.items():
        t = bench.measured_traffic(gemm, kernel)
        assert isinstance(t, int) and t > 0, (gemm, kernel)
        other = kernel.replace(", 4>", ", 8>") if kernel.endswith(", 4>") else kernel.replace(", 8>", ", 4>")
        assert bench.measured_traffic(gemm, other) is None
    # changed GEMM sources void the figure
    monkeypatch.setattr(bench, "gemm_sources_sha256", lambda: "0" * 64)
    assert bench.measured_traffic("fc1", recorded["fc1"]) is None


def test_profiled_kernels_are_the_shipped_table_choices():
    """The counter summary was taken of the kernels the shipped table picks for
    fc1 and fc2, so a default bench run reports traffic for them."""
    t = T.TuningTable(T.SHIPPED_TABLE)
    dev = "gfx950/256cu"
    cfg1 = t.lookup(20480, 12288, 3072, epilogue="gelu_tanh", out_kind="mx", device=dev)
    cfg2 = t.lookup(20480, 3072, 12288, device=dev)
    assert bench.measured_traffic("fc1", bench.kernel_name("fc1", cfg1)) is not None
    assert bench.measured_traffic("fc2", bench.kernel_name("fc2", cfg2)) is not None
