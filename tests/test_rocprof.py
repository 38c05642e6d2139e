"""The rocprofv3 reduction (memory_efficient_exact_amd/rocprof.py) on synthetic
CSV files shaped like rocprofv3's, with counter values chosen so that every
derived figure has a known answer. CPU only."""

import csv
import json
import os

import pytest

from memory_efficient_exact_amd import rocprof

BWD = "void mea::(anonymous namespace)::bwd_main_kernel<64, 8>(mea::(anonymous namespace)::BwdArgs)"
COPY = "__amd_rocclr_copyBuffer"


def write_csv(path, rows):
    os.makedirs(os.path.dirname(path), exist_ok=True)
    with open(path, "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=list(rows[0]))
        w.writeheader()
        w.writerows(rows)


def counter_rows(kernel, dispatch, values):
    return [{"Correlation_Id": dispatch, "Dispatch_Id": dispatch, "Agent_Id": 1, "Kernel_Name": kernel,
             "Counter_Name": c, "Counter_Value": v} for c, v in values.items()]


@pytest.fixture
def prof(tmp_path):
    d = tmp_path / "prof"
    # kernel trace: 4 dispatches of the backward (1, 2, 3, 4 ms), one copy
    trace = [{"Kind": "KERNEL_DISPATCH", "Dispatch_Id": i, "Kernel_Name": BWD,
              "Start_Timestamp": 1000 * i, "End_Timestamp": 1000 * i + 1_000_000 * i} for i in range(1, 5)]
    trace.append({"Kind": "KERNEL_DISPATCH", "Dispatch_Id": 9, "Kernel_Name": COPY,
                  "Start_Timestamp": 0, "End_Timestamp": 10})
    write_csv(str(d / "kt" / "host" / "run_kernel_trace.csv"), trace)
    # pass A: 2 dispatches averaging GRBM_GUI_ACTIVE = 8e6 (1e6 cycles per XCD);
    # busy cycles 5.12e8 = half of 1024 SIMDs x 1e6 cycles
    rows = counter_rows(BWD, 1, {"GRBM_GUI_ACTIVE": 7e6, "SQ_VALU_MFMA_BUSY_CYCLES": 5.12e8,
                                 "SQ_VALU_MFMA_COEXEC_CYCLES": 1.024e8, "SQ_INSTS_MFMA": 1.6e7,
                                 "SQ_WAVE_CYCLES": 1e9, "SQ_ACTIVE_INST_VALU": 2.5e8})
    rows += counter_rows(BWD, 2, {"GRBM_GUI_ACTIVE": 9e6, "SQ_VALU_MFMA_BUSY_CYCLES": 5.12e8,
                                  "SQ_VALU_MFMA_COEXEC_CYCLES": 1.024e8, "SQ_INSTS_MFMA": 1.6e7,
                                  "SQ_WAVE_CYCLES": 1e9, "SQ_ACTIVE_INST_VALU": 2.5e8})
    write_csv(str(d / "pmcA" / "run_counter_collection.csv"), rows)
    # pass B: per-instance rows of one counter are summed per dispatch
    # SQ_LDS_IDX_ACTIVE 6.4e7 = a quarter of 256 CUs x 1e6 cycles (the cycles of pass A)
    rows = counter_rows(BWD, 1, {"SQ_WAVE_CYCLES": 1e9, "SQ_WAIT_ANY": 4e8, "SQ_INSTS_LDS": 3.2e7,
                                 "SQ_LDS_IDX_ACTIVE": 6.4e7})
    rows += counter_rows(BWD, 1, {"SQ_LDS_BANK_CONFLICT": 1e6})
    rows += counter_rows(BWD, 1, {"SQ_LDS_BANK_CONFLICT": 2e6})
    write_csv(str(d / "pmcB" / "run_counter_collection.csv"), rows)
    # traffic: the 256 MiB copy reads 131072 KiB (factor 2) and writes 262144 KiB (factor 1)
    write_csv(str(d / "pmcF" / "run_counter_collection.csv"),
              counter_rows(COPY, 1, {"FETCH_SIZE": 131072.0}) + counter_rows(BWD, 2, {"FETCH_SIZE": 1024.0}))
    write_csv(str(d / "pmcW" / "run_counter_collection.csv"),
              counter_rows(COPY, 1, {"WRITE_SIZE": 262144.0}) + counter_rows(BWD, 2, {"WRITE_SIZE": 512.0}))
    return str(d)


def test_short_names():
    assert rocprof.short_name(BWD) == "bwd_main_kernel<64, 8>"
    assert rocprof.short_name("mea::(anonymous namespace)::fwd_bf16_kernel<64, 2, 128, false, 8>"
                              "(mea::(anonymous namespace)::FwdArgs)") == "fwd_bf16_kernel<64, 2, 128, false, 8>"
    assert rocprof.short_name(COPY) == COPY


def test_collect_and_derive(prof):
    s = rocprof.collect(prof, 256 << 20, timed=(1, 2))
    assert s["read_factor"] == pytest.approx(2.0) and s["write_factor"] == pytest.approx(1.0)
    e = s["kernels"]["bwd_main_kernel<64, 8>"]
    assert COPY not in s["kernels"]
    assert e["calls"] == 4 and e["avg_us"] == pytest.approx(2500.0)
    assert e["timed_avg_us"] == pytest.approx(2500.0)  # dispatches 2 and 3
    assert e["cycles_per_xcd"] == pytest.approx(1e6)
    assert e["mfma_busy"] == pytest.approx(0.5)
    assert e["mfma_valu_coissue"] == pytest.approx(0.1)
    assert e["busy_cycles_per_mfma"] == pytest.approx(32.0)
    assert e["valu_share"] == pytest.approx(0.25)
    assert e["wait_any_share"] == pytest.approx(0.4)
    assert e["lds_insts_per_mfma"] == pytest.approx(2.0)
    assert e["lds_bank_conflict_cycles"] == pytest.approx(3e6)
    assert e["lds_busy"] == pytest.approx(0.25)
    assert e["hbm_read_bytes"] == pytest.approx(2 * 1024 * 1024)
    assert e["hbm_write_bytes"] == pytest.approx(512 * 1024)
    assert e["hbm_gbs"] == pytest.approx(2.5 * 2 ** 20 / 2.5e-3 / 1e9)
    assert e["source_files"] == ["csrc/bwd_bf16.hip", "csrc/mea_device.h"]
    assert e["source_sha256"] == rocprof.source_hash("bwd_main_kernel<64, 8>")


def test_render_round_trip(prof, tmp_path):
    s = rocprof.collect(prof, 256 << 20)
    md = rocprof.render(s, "t", ["cmd a", "cmd b"])
    assert "| `bwd_main_kernel<64, 8>` |" in md and "50.0%" in md
    d = tmp_path / "profiles"
    d.mkdir()
    (d / "x.md").write_text(md)
    fig = rocprof.current_figures(str(d), "bwd_main_kernel<64, 8>")
    assert fig["mfma_busy"] == pytest.approx(0.5) and fig["profiles"] == ["x.md"]
    # a summary taken on other sources does not match
    s["kernels"]["bwd_main_kernel<64, 8>"]["source_sha256"] = "0" * 64
    (d / "x.md").write_text(rocprof.render(s, "t", []))
    assert rocprof.current_figures(str(d), "bwd_main_kernel<64, 8>") == {}


def test_plan_has_one_run_per_pass():
    cmds = rocprof.plan("/p", "prog")
    assert len(cmds) == 2 + len(rocprof.PASSES)
    for p, cs in rocprof.PASSES.items():
        line = [c for c in cmds if f"-d /p/{p} " in c]
        assert len(line) == 1 and " ".join(cs) in line[0] and line[0].startswith("timeout -s KILL")
        # the hardware limits of one pass: at most 8 SQ, 4 TCC-equivalent, 2 GRBM counters
        assert sum(c.startswith("SQ_") for c in cs) <= 8 and sum(c.startswith("GRBM_") for c in cs) <= 2


def test_mangled_library_names():
    # the profiler leaves some names mangled; bf16 parameters use a type code the
    # system demanglers do not read
    assert rocprof.short_name("_ZN3mea12_GLOBAL__N_115bwd_rows_kernelILi64EEEvPKDF16bS3_PKfS5_PfS6_l") \
        == "bwd_rows_kernel<64>"
    assert rocprof.short_name("_ZN3mea12_GLOBAL__N_117bwd_reduce_kernelILi128EDF16bEEvNS0_10ReduceArgsE") \
        == "bwd_reduce_kernel<128, __bf16>"
    assert rocprof.short_name("_ZN3mea12_GLOBAL__N_115fwd_bf16_kernelILi64ELi1ELi128ELb1ELi4EEEvNS0_7FwdArgsE") \
        == "fwd_bf16_kernel<64, 1, 128, true, 4>"


# ------------------------------------------------------------ probe derivation

def _probe(name, w, mfma_cyc, valu_cyc, mfma, valu):
    return {"probe": name, "waves_per_simd": w, "clock_mhz": 2000.0,
            "mfma_wave_cycles_per_iter": mfma_cyc, "valu_wave_cycles_per_iter": valu_cyc,
            "mfma_per_iter": mfma, "valu_per_iter": valu}


def test_probe_derivation_uses_the_register_only_mfma_time():
    import bench
    raw = {"probes": [
        _probe("mfma_32x32x16_bf16", 1, 128.0, 0.0, 4, 0),
        # an LDS-fed MFMA probe after it must not replace the MFMA-alone time
        _probe("mfma_fed_by_ds_read_b128", 1, 240.0, 0.0, 4, 0),
        _probe("v_fma_f32", 1, 0.0, 44.0, 0, 8),
        _probe("v_add_f32", 1, 0.0, 40.0, 0, 8),
        _probe("v_exp_f32", 1, 0.0, 72.0, 0, 8),
        _probe("v_exp_f32+v_add_f32", 1, 0.0, 56.0, 0, 8),
        _probe("one_wave:4mfma+8fma", 1, 135.0, 0.0, 4, 8),
        _probe("mfma_wave+exp_wave", 2, 160.0, 108.0, 4, 8),
    ], "atomic_dq": [{"mode": "atomic_add_f32", "ms": 4.0, "tb_per_s": 1.07}],
       "hbm_stream": [{"mode": "read_blocked_x4", "ms": 0.35, "bytes": 2147483648, "tb_per_s": 6.14}]}
    d = bench.derive_probes(raw)["derived"]
    assert d["hbm_stream"] == {"read_blocked_x4": {"tb_per_s": 6.14, "ms": 0.35}}
    from memory_efficient_exact_amd import rocprof
    md = rocprof.render_probes({"raw": raw, "derived": d})
    assert "| read_blocked_x4 | 0.350 | 2147483648 | 6.14 |" in md
    assert d["mfma_32x32x16_bf16 w1"]["simd_cycles_per_mfma"] == 32.0
    assert d["v_fma_f32 w1"]["wave_cycles_per_instr"] == 5.5
    assert d["v_fma_f32 w1"]["cost_vs_v_add_f32"] == 1.1
    # four exponentials (36 cycles) and four adds (20) alone: 56, so no overlap
    assert abs(d["v_exp_f32+v_add_f32 w1"]["time_vs_serial_sum"] - 1.0) < 1e-12
    mix = d["one_wave:4mfma+8fma"]
    assert mix["mfma_alone_cycles_per_iter"] == 128.0
    # 128 + 44 - 135 = 37 of the FMAs' 44 cycles ran under the MFMAs
    assert abs(mix["valu_hidden"] - 37.0 / 44.0) < 1e-12
    assert abs(mix["mfma_pipe_busy"] - 128.0 / 135.0) < 1e-12
    # an MFMA wave beside an exponential wave: each against its own time alone
    two = d["mfma_wave+exp_wave"]
    assert two["mfma_wave_slowdown"] == 160.0 / 128.0
    assert two["valu_wave_slowdown"] == 108.0 / 72.0
    assert abs(two["mfma_pipe_busy"] - 128.0 / 160.0) < 1e-12
