"""Host arithmetic of bench.py, on the CPU: the algorithmic bytes and flops
behind the roofline fractions, the W8A8 path choice, the percentile, the
dtype label and the counter records behind `roofline.traffic`. Each expected
value is written out here from the definitions of the kernels' work (weights
of the touched experts, their block scales, token rows in and h out), not
taken from bench.py."""
import json

import pytest

import bench
from synth import CONFIGS


def test_gate_up_work_w8a8_prefill_with_shared_expert():
    # DeepSeek-shaped prefill: 256 routed experts (all touched) and the shared
    # expert, all fp8 with fp32 scales per 128 x 128 block; the launch reads
    # E4M3 token rows and writes E4M3 h, each with fp32 scales per 128 columns
    cfg = CONFIGS["dsv3_prefill"]
    T, H, F, E, k = 4096, 7168, 2048, 256, 8
    assert (cfg.T, cfg.H, cfg.F, cfg.E, cfg.k, cfg.Fs) == (T, H, F, E, k, F)
    blocks = (H // 128) * (F // 128)
    routed = E * 2 * (H * F + 4 * blocks)          # W1 and W3 of every expert
    shared = 2 * (H * F + 4 * blocks)
    rows = T * k + T                                # routed rows + shared rows
    x_in = T * H + 4 * T * (H // 128)              # codes + scales
    h_out = rows * F + 4 * rows * (F // 128)
    nbytes, flops = bench.gate_up_work(cfg, E, a8=True)
    assert nbytes == routed + shared + x_in + h_out == 7_655_529_472
    assert flops == 4 * rows * H * F


def test_gate_up_work_bf16_decode_counts_touched_experts_only():
    cfg = CONFIGS["mixtral_decode"]
    T, H, F, k = 16, 4096, 14336, 2
    for touched in (1, 5, 8):
        nbytes, flops = bench.gate_up_work(cfg, touched, a8=False)
        assert nbytes == touched * 2 * H * F * 2 + T * H * 2 + T * k * F * 2
        assert flops == 4 * T * k * H * F


def test_gate_up_work_mxfp4_two_values_a_byte_and_byte_scales():
    cfg = CONFIGS["mixtral_decode_mxfp4"]
    T, H, F, k = 16, 4096, 14336, 2
    per_matrix = H * F // 2 + (H // 32) * F         # E2M1 codes + one E8M0 byte per 32 K rows
    nbytes, _ = bench.gate_up_work(cfg, 8, a8=False)
    assert nbytes == 8 * 2 * per_matrix + T * H * 2 + T * k * F * 2


def test_w8a8_path_choice():
    assert bench.uses_a8(CONFIGS["dsv3_prefill"], "auto")
    assert not bench.uses_a8(CONFIGS["dsv3_decode"], "auto")      # 64 x 8 assignments < 15 x 256
    assert bench.uses_a8(CONFIGS["dsv3_decode"], "tiled_a8")
    assert not bench.uses_a8(CONFIGS["mixtral_prefill"], "auto")   # bf16 weights


def test_dtype_is_the_gemm_arithmetic_type():
    assert bench.dtype_label(CONFIGS["dsv3_prefill"], True) == "fp8"
    assert bench.dtype_label(CONFIGS["dsv3_decode"], False) == "bf16"
    assert bench.dtype_label(CONFIGS["mixtral_decode_mxfp4"], False) == "bf16"
    assert bench.dtype_label(CONFIGS["toy_fp32"], False) == "f32"


@pytest.mark.parametrize("xs,q,want", [
    ([3.0], 0.95, 3.0),
    ([5.0, 1.0, 4.0, 2.0, 3.0], 0.5, 3.0),
    ([5.0, 1.0, 4.0, 2.0, 3.0], 0.95, 4.8),   # 0.95 x 4 = 3.8: 4 + 0.8 x (5 - 4)
    ([10.0, 20.0], 0.0, 10.0),
    ([10.0, 20.0], 1.0, 20.0),
])
def test_percentile_interpolates_linearly(xs, q, want):
    assert bench.percentile(xs, q) == pytest.approx(want, abs=1e-12)


def test_kernel_family_from_trace_names():
    assert bench.kernel_family("void moe::(anonymous namespace)::stream_gemm_kernel<1, true, true>(x)") == "stream"
    assert bench.kernel_family("void moe::tiled::(anonymous namespace)::tiled_a8_kernel<true, 4, 160, false>") == "a8"
    assert bench.kernel_family("moe::tiled::(anonymous namespace)::tiled_persist_kernel") == "persist"
    assert bench.kernel_family("void moe::tiled::tiled_gemm_kernel<1, true, 256, 2, false, 4>") == "tiled"


def _counter_csv(path, rows):
    path.mkdir(parents=True, exist_ok=True)
    lines = ["Dispatch_Id,Kernel_Name,Counter_Name,Counter_Value"]
    lines += [f'{d},"{k}",{c},{v}' for d, k, c, v in rows]
    (path / "run_counter_collection.csv").write_text("\n".join(lines) + "\n")


def test_counter_means_sum_rows_of_a_dispatch_then_average_dispatches(tmp_path):
    a, b = "void tiled_a8_kernel<true, 4, 160, false>(x)", "void other_kernel(x)"
    _counter_csv(tmp_path / "run", [
        (1, a, "FETCH_SIZE", 10.0), (1, a, "FETCH_SIZE", 20.0),   # two rows of one dispatch
        (2, a, "FETCH_SIZE", 40.0), (1, a, "WRITE_SIZE", 99.0),   # another dispatch; another counter
        (3, b, "FETCH_SIZE", 5.0),
    ])
    got = bench._pmc_means(str(tmp_path / "run"), "FETCH_SIZE")
    assert got == {a: (35.0, 2), b: (5.0, 1)}


def test_traffic_record_scales_each_counter_by_the_copy_calibration(tmp_path, monkeypatch):
    # a 1 GiB copy whose FETCH_SIZE reads half the bytes and whose WRITE_SIZE
    # reads them all: scales 2 and 1; the gate/up kernel reads 3000 KiB and
    # writes 500 KiB per dispatch
    n = bench.COPY_CALIBRATION_BYTES
    gu = "void moe::tiled::(anonymous namespace)::tiled_a8_kernel<true, 4, 160, false>(x)"
    dn = "void moe::tiled::(anonymous namespace)::tiled_a8_kernel<false, 4, 160, true>(x)"
    _counter_csv(tmp_path / "f", [(1, gu, "FETCH_SIZE", 3000.0), (2, dn, "FETCH_SIZE", 7.0)])
    _counter_csv(tmp_path / "w", [(1, gu, "WRITE_SIZE", 500.0), (2, dn, "WRITE_SIZE", 7.0)])
    _counter_csv(tmp_path / "cf", [(1, "copy", "FETCH_SIZE", n / 2048.0), (2, "fill", "FETCH_SIZE", 1.0)])
    _counter_csv(tmp_path / "cw", [(1, "copy", "WRITE_SIZE", n / 1024.0), (2, "fill", "WRITE_SIZE", n / 1024.0)])
    out = tmp_path / "profiles"
    out.mkdir()
    monkeypatch.setattr(bench, "PROFILE_DIR", str(out))

    class Args:
        pmc_fetch, pmc_write = str(tmp_path / "f"), str(tmp_path / "w")
        calib_fetch, calib_write = str(tmp_path / "cf"), str(tmp_path / "cw")
        workload, commands, pmc_kernel = "dsv3_prefill", ["cmd"], "gate_up"

    assert bench.record_traffic(Args) == 0
    rec = json.loads((out / "gate_up_swiglu_dsv3_prefill_pmc.json").read_text())
    assert rec["kernel"] == gu
    assert (rec["fetch_scale"], rec["write_scale"]) == (2.0, 1.0)
    assert rec["hbm_bytes_per_launch"] == 3000 * 1024 * 2 + 500 * 1024 * 1
