"""Host logic of the counter recorder in bench.py (no GPU): dispatch labels, the algorithmic
byte split of each counted kernel, and a record built from synthetic rocprofv3 CSV output."""
import csv
import json
import os
import shutil

import bench

PRE = "void kda::(anonymous namespace)::prefill_kernel<unsigned short, 128, 128, {}>(unsigned short const*)"
DEC = "void kda::decode_kernel<unsigned short, 128, 128, {}, {}, {}, {}>(unsigned short const*)"
EPI = "void kda::gate_rmsnorm_kernel<unsigned short, 128>(unsigned int __vector(4) const*)"
PRO = "void kda::(anonymous namespace)::prologue_kernel<unsigned short, 128>(kda::ProKernelArgs)"
PRO0 = "void kda::(anonymous namespace)::prologue_empty_kernel<unsigned short>(unsigned short const*)"
COPY = "__amd_rocclr_copyBuffer"
OTHER = "void at::native::vectorized_elementwise_kernel<4, at::native::bfloat16_copy_kernel_cuda>()"


def _sequence():
    """The kernels of one `bench.py --no-gated` step, in the order the benchmark launches them."""
    return [OTHER, PRE.format("false"), DEC.format("false", "false", "false", 1024), COPY,
            EPI, OTHER, PRE.format("true"), EPI, DEC.format("true", "true", "false", 1024),
            PRO, PRO0, PRO, PRO0, PRE.format("true"), EPI, DEC.format("true", "true", "true", 512)]


def test_labels_follow_kernel_and_position():
    labels = bench._label_dispatches([(n, {}) for n in _sequence()])
    assert labels == [None, "prefill", "decode", None, "epilogue", None, "prefill_gated",
                      "epilogue_after_prefill", "decode_epilogue", "prologue", None, None, None,
                      "prefill_gated", "epilogue_after_prefill", "decode_fused"]


def test_labels_refuse_a_run_with_the_split_timing():
    """The 12-head prefills of the split timing launch the headline prefill's kernel, so their
    counters would be averaged into it: such a run is refused."""
    import pytest
    scan = "void kda::(anonymous namespace)::split_scan_kernel<128, 128>(float*, float const*, float*, int, int)"
    with pytest.raises(SystemExit, match="--no-split"):
        bench._label_dispatches([(n, {}) for n in _sequence() + [PRE.format("false"), scan]])


def test_labels_refuse_one_kernel_on_two_grids():
    """The varlen timing launches the headline prefill's kernel on another grid; a run that
    includes it is refused, while one grid per label is accepted."""
    import pytest
    seq = _sequence()
    same = [(n, {"_grid": 98304.0} if "prefill_kernel" in n else {}) for n in seq]
    bench._label_dispatches(same)
    mixed = same + [(PRE.format("false"), {"_grid": 1572864.0})]
    with pytest.raises(SystemExit, match="--no-varlen"):
        bench._label_dispatches(mixed)


def test_algorithmic_bytes_match_the_per_launch_figures():
    r, w = bench.ALG_BYTES["prefill"]
    assert r + w == bench.T_PREFILL * bench.H * bench.PREFILL_BYTES_PER_TOKEN_HEAD + 2 * bench.H * bench.STATE_BYTES
    r, w = bench.ALG_BYTES["decode"]
    assert r + w == bench.N_DECODE * bench.H * bench.DECODE_BYTES_PER_PAIR
    r, w = bench.ALG_BYTES["prefill_gated"]
    assert r + w == bench.T_PREFILL * bench.H * bench.GATED_PREFILL_BYTES_PER_TOKEN_HEAD + 2 * bench.H * bench.STATE_BYTES
    r, w = bench.ALG_BYTES["decode_epilogue"]
    assert r + w == bench.N_DECODE * bench.H * bench.EPILOGUE_DECODE_BYTES_PER_PAIR
    r, w = bench.ALG_BYTES["decode_fused"]
    assert r + w == bench.N_DECODE * bench.H * bench.FUSED_DECODE_BYTES_PER_PAIR + bench.H * bench.CONV_C * 16
    r, w = bench.ALG_BYTES["epilogue"]
    assert r + w == bench.T_PREFILL * bench.H * bench.EPILOGUE_BYTES_PER_TOKEN_HEAD + bench.D * 4


def _write_pass(path, counters):
    os.makedirs(path, exist_ok=True)
    with open(os.path.join(path, "pmc_counter_collection.csv"), "w", newline="") as fh:
        w = csv.writer(fh)
        w.writerow(["Dispatch_Id", "Kernel_Name", "Counter_Name", "Counter_Value"])
        for i, name in enumerate(_sequence()):
            for cname, value in counters(name).items():
                # two instances per dispatch: the recorder sums them
                w.writerow([i + 1, name, cname, value / 2])
                w.writerow([i + 1, name, cname, value / 2])


def test_record_from_synthetic_passes(tmp_path, monkeypatch):
    gib = 4.0
    kib = gib * (1 << 30) / 1024
    alg = bench.ALG_BYTES

    def bytes_of(name, which):
        lab = {PRE.format("false"): "prefill", COPY: None}.get(name)
        if name == COPY:
            return kib * 1024
        return alg[lab][which] if lab else 1024.0

    # FETCH_SIZE reads half the bytes and WRITE_SIZE all of them, as on the GPU.
    _write_pass(tmp_path / "fetch", lambda n: {"FETCH_SIZE": bytes_of(n, 0) / 1024 * 0.5})
    _write_pass(tmp_path / "write", lambda n: {"WRITE_SIZE": bytes_of(n, 1) / 1024})
    _write_pass(tmp_path / "util", lambda n: {"MfmaUtil": 10.0, "VALUBusy": 40.0})
    # write into a scratch copy of the repository's profiles directory
    root = tmp_path / "root"
    (root / "profiles").mkdir(parents=True)
    for rel in {p for ps in bench.KERNEL_SOURCES.values() for p in ps}:
        os.makedirs(root / os.path.dirname(rel), exist_ok=True)
        shutil.copy(os.path.join(bench.ROOT, rel), root / rel)
    monkeypatch.setattr(bench, "ROOT", str(root))
    bench.record_counters(str(tmp_path), gib)
    rec = json.load(open(root / "profiles" / "hbm_traffic.json"))
    assert abs(rec["calibration"]["fetch_factor"] - 0.5) < 1e-12
    assert abs(rec["calibration"]["write_factor"] - 1.0) < 1e-12
    p = rec["prefill"]
    assert abs(p["hbm_bytes_read"] - alg["prefill"][0]) < 1.0
    assert abs(p["hbm_bytes_written"] - alg["prefill"][1]) < 1.0
    assert p["mfma_util_pct"] == 10.0 and p["valu_busy_pct"] == 40.0
    assert p["code_digest"] == bench.kernel_digest("prefill")
    assert set(rec) >= {"prefill", "decode", "epilogue", "epilogue_after_prefill", "prefill_gated",
                        "decode_epilogue", "prologue", "decode_fused", "calibration"}


def test_power_reading_parser(monkeypatch):
    """bench.py's amd-smi reading finds the socket power and the per-XCD shader
    clocks wherever the JSON nests them, and gives None when they are absent."""
    import subprocess

    def fake(out):
        class R:
            stdout = json.dumps(out)
        monkeypatch.setattr(subprocess, "run", lambda *a, **k: R())

    reading = {"gpu": 0, "power": {"socket_power": {"value": 1318, "unit": "W"}, "gfx_voltage": "N/A"},
               "clock": {"gfx_0": {"clk": {"value": 2352, "unit": "MHz"}}, "gfx_1": {"clk": {"value": 2309}},
                         "mem_0": {"clk": {"value": 1900}}, "fclk_0": {"clk": "N/A"}}}
    fake([reading])
    assert bench._smi_power_clocks() == (1318.0, [2352.0, 2309.0])
    fake({"gpu_data": [reading]})
    assert bench._smi_power_clocks() == (1318.0, [2352.0, 2309.0])
    fake({"other": 1})
    assert bench._smi_power_clocks() is None
