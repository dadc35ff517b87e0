"""bench.py's host logic, no GPU: the algorithmic byte model, the rotation
pool, the one-GPU contract and the counter-summary parser (on a synthetic
rocprofv3 counter CSV whose values are known)."""
import csv
import json

import pytest

import bench
import synthetic


def test_algorithmic_bytes():
    """One read per input element and one write per output element, FP32."""
    C = synthetic.Case
    assert bench.algo_split(C(2, "layernorm_residual", 1024, 4096, "uniform")) == (2 * 4 * 1024 * 4096, 4 * 1024 * 4096)
    assert bench.algo_bytes(C(2, "rmsnorm", 1024, 4096, "uniform")) == 8 * 1024 * 4096
    assert bench.algo_bytes(C(2, "softmax", 1024, 4096, "uniform")) == 33554432
    assert bench.algo_bytes(C(2, "layernorm_residual", 1024, 4096, "uniform")) == 50331648
    assert bench.algo_bytes(C(6, "layernorm", 16, 8, "uniform")) == 8 * 16 * 8
    assert bench.algo_split(C(7, "layernorm_affine", 16, 8, "uniform"))[1] == 4 * 16 * 8
    assert bench.algo_split(C(8, "row_sum", 16, 8, "uniform")) == (4 * 16 * 8, 4 * 16)
    assert bench.algo_split(C(8, "row_minmax", 16, 8, "uniform")) == (4 * 16 * 8, 8 * 16)


def test_rotation_pool_defeats_the_last_level_cache():
    for cfg in bench.WORKLOADS:
        for c in bench.WORKLOADS[cfg]:
            n = bench.rotation_sets(c)
            assert n >= 3 and n * bench.algo_bytes(c) >= 2 * 2 ** 30 > 256 * 2 ** 20


def test_default_workload_is_the_largest_single_gpu_one():
    """The default bench line times the wide-row configuration's three
    operators and the softmax stress configuration: the largest shapes that
    fit one GPU."""
    cases = bench.WORKLOADS[bench.LARGEST]
    assert [(c.op, c.rows, c.width) for c in cases] == [
        ("layernorm_residual", 16384, 8192), ("rmsnorm", 16384, 8192), ("softmax", 16384, 8192),
        ("softmax", 8192, 32768)]
    assert max(bench.algo_bytes(c) for c in cases) == max(bench.algo_bytes(c) for cfg in bench.CORE
                                                          for c in bench.WORKLOADS[cfg])
    name = bench.WORKLOAD_NAMES[bench.LARGEST]
    assert "16384x8192" in name and "8192x32768" in name


def test_more_than_one_gpu_is_refused(capsys):
    assert bench.main(["--gpus", "2"]) == 2
    msg = json.loads(capsys.readouterr().out.strip().splitlines()[-1])
    assert "one GPU" in msg["error"]


def _fake_counter_csv(path, ctr, per_case_kib, copy_kib):
    """One row per dispatch, in the order a `bench.py --pmc --all` pass makes
    them: per workload, for each case a flush fill then the library's kernel(s),
    and the calibration copy at the end."""
    rows, did = [], 0

    def add(name, value):
        nonlocal did
        rows.append({"Dispatch_Id": did, "Kernel_Name": name, "Counter_Name": ctr, "Counter_Value": value})
        did += 1

    for cfg in bench.PMC_CFGS:
        for c in bench.WORKLOADS[cfg]:
            add("void at::native::vectorized_elementwise_kernel<4, FillFunctor<float> >(int, ...)", 1.0)
            kib = per_case_kib(c)
            if cfg in bench.WS_WORKLOADS and c.width > 32768:
                # a two-dispatch call: both count
                add("void rowred::(anonymous namespace)::exchange_clear_kernel(unsigned long*, long)", 0.25 * kib)
                add("void rowred::(anonymous namespace)::seg_exchange_kernel<2, 8>(rowred::SegArgs)", 0.75 * kib)
            else:
                add("void rowred::(anonymous namespace)::rows_kernel<2, 8>(rowred::RowArgs)", kib)
        add("void rowred::(anonymous namespace)::copy_kernel(float4 const*, float4*, long)", copy_kib)
    with open(path, "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=["Dispatch_Id", "Kernel_Name", "Counter_Name", "Counter_Value"])
        w.writeheader()
        w.writerows(rows)


def test_traffic_summary_scales_by_the_copy(tmp_path):
    """Reads are FETCH_SIZE x (256 MiB / the copy's FETCH_SIZE); writes the
    same with WRITE_SIZE.  The fake counters read half the copy's bytes (as
    FETCH_SIZE does on this part) and exactly the algorithmic bytes after
    scaling: every ratio must come out 1."""
    copy_fetch, copy_write = 2 ** 28 / 1024 / 2, 2 ** 28 / 1024
    _fake_counter_csv(tmp_path / "f.csv", "FETCH_SIZE", lambda c: bench.algo_split(c)[0] / 1024 / 2, copy_fetch)
    _fake_counter_csv(tmp_path / "w.csv", "WRITE_SIZE", lambda c: bench.algo_split(c)[1] / 1024, copy_write)
    (tmp_path / "f.log").write_text("pmc kernel_source_hash abc\n")
    (tmp_path / "w.log").write_text("pmc kernel_source_hash abc\n")
    out = tmp_path / "profiles"
    out.mkdir()
    written = bench.traffic_summary(str(tmp_path / "f.csv"), str(tmp_path / "w.csv"), str(out),
                                    str(tmp_path / "f.log"), str(tmp_path / "w.log"))
    assert len(written) == len(bench.PMC_CFGS)
    for cfg in bench.PMC_CFGS:
        text = (out / f"pmc_traffic_cfg{cfg}.txt").read_text()
        assert "kernel_source_hash: abc" in text
        for c in bench.WORKLOADS[cfg]:
            key = f"{c.op} {c.rows}x{c.width}"
            line = next(l for l in text.splitlines() if l.startswith(f"read_bytes[{key}]"))
            assert "ratio 1.0000" in line, line
            line = next(l for l in text.splitlines() if l.startswith(f"write_bytes[{key}]"))
            assert "ratio 1.0000" in line, line
            total = int(next(l for l in text.splitlines() if l.startswith(f"traffic_bytes[{key}]")).split(":")[1])
            assert abs(total - bench.algo_bytes(c)) <= 1


def test_traffic_summary_counts_calls_exactly(tmp_path):
    """A pass with one call missing is refused rather than misattributed."""
    _fake_counter_csv(tmp_path / "f.csv", "FETCH_SIZE", lambda c: 1.0, 1.0)
    rows = list(csv.DictReader(open(tmp_path / "f.csv")))
    drop = next(i for i, r in enumerate(rows) if "rows_kernel" in r["Kernel_Name"])
    del rows[drop]
    with open(tmp_path / "g.csv", "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=list(rows[0].keys()))
        w.writeheader()
        w.writerows(rows)
    with pytest.raises(SystemExit):
        bench.traffic_summary(str(tmp_path / "g.csv"), str(tmp_path / "g.csv"), str(tmp_path))


def test_committed_traffic_is_used_only_on_matching_sources(tmp_path, monkeypatch):
    """roofline.traffic is read from the committed summary only when its
    kernel source hash matches the sources bench runs on."""
    case = bench.WORKLOADS[2][0]
    key = f"{case.op} {case.rows}x{case.width}"
    (tmp_path / "profiles").mkdir()
    summary = tmp_path / "profiles" / "pmc_traffic_cfg2.txt"
    summary.write_text(f"kernel_source_hash: {bench.kernel_source_hash()}\ntraffic_bytes[{key}]: 123\n")
    real_hash = bench.kernel_source_hash()
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    monkeypatch.setattr(bench, "kernel_source_hash", lambda: real_hash)
    assert bench.read_traffic(case) == 123
    monkeypatch.setattr(bench, "kernel_source_hash", lambda: "0" * 16)
    assert bench.read_traffic(case) is None


def test_short_names():
    n = "void rowred::(anonymous namespace)::ln_tail_kernel<2>(rowred::RowArgs)"
    assert bench.kernel_short_name(n) == "ln_tail_kernel<2>(rowred::RowArgs)"
    assert bench.is_library_reduction_kernel(n)
    assert not bench.is_library_reduction_kernel("void rowred::(anonymous namespace)::copy_kernel(float4 const*)")
    assert not bench.is_library_reduction_kernel("void at::native::fill_kernel<float>()")


def test_segments_summary_parses_a_counter_run(tmp_path):
    """The exchange segments summary groups each timed case's exchange
    dispatches in order (the first call of each untimed) and reports wave
    lifetime and waiting share from SQ counters."""
    import bench
    cases = list(bench.segment_cases())[:2]
    log = tmp_path / "log.txt"
    lines = ["segments kernel_source_hash abc123"]
    rows = []
    did = 0
    for k, (name, T, C, lds, S, r, w) in enumerate(cases):
        lines.append(json.dumps({"segments": S, "geometry": name, "rows": r, "width": w, "calls": 3,
                                 "us_per_call": 10.0 + k, "wait_status": 0}))
        for call in range(3):
            did += 1  # clear kernel, ignored
            rows.append((did, "rowred::(anonymous namespace)::exchange_clear_kernel", "SQ_WAVES", 1))
            did += 1
            kname = "void rowred::(anonymous namespace)::seg_exchange_kernel<2, 8>(rowred::SegArgs)"
            scale = 1 if call else 100  # the untimed call is dropped
            for ctr, v in (("SQ_WAVES", 1000), ("SQ_WAVE_CYCLES", 250 * (k + 1) * scale),
                           ("SQ_WAIT_ANY", 100 * (k + 1) * scale)):
                rows.append((did, kname, ctr, v))
    log.write_text("\n".join(lines) + "\n")
    csv_path = tmp_path / "c.csv"
    with open(csv_path, "w") as f:
        f.write('"Dispatch_Id","Kernel_Name","Counter_Name","Counter_Value"\n')
        for d, n, c, v in rows:
            f.write(f'{d},"{n}","{c}",{v}\n')
    out = tmp_path / "out.txt"
    bench.segments_summary(str(csv_path), str(log), str(out))
    body = [l for l in out.read_text().splitlines() if not l.startswith("#")]
    assert len(body) == 2 and body[0].split(" | ")[3] == "-"
    bench.segments_summary(str(csv_path), str(log), str(out), str(log))  # with the timing log
    body = [l for l in out.read_text().splitlines() if not l.startswith("#")]
    assert body[0].split(" | ")[3] == "10.0" and body[1].split(" | ")[3] == "11.0"
    # lifetime = 4 * 250 (k+1) / 1000 cycles; waiting share 100/250
    assert body[0].split(" | ")[5:] == ["1", "0.400"]
    assert body[1].split(" | ")[5:] == ["2", "0.400"]
    assert "abc123" in out.read_text()
