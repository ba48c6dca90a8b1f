"""Host-side logic of bench.py (no GPU): the attended-pair count behind every FLOP figure, and the counter
summary that turns rocprofv3 FETCH_SIZE / WRITE_SIZE readings into bytes per launch."""
import csv
import json
import os

import pytest

import bench


def brute_pairs(L, window):
    return sum(1 for i in range(L) for j in range(i + 1) if window < 0 or i - j <= window)


@pytest.mark.parametrize("L", [0, 1, 5, 128, 129, 130, 300])
@pytest.mark.parametrize("window", [-1, 0, 3, 128])
def test_pairs_per_head_matches_enumeration(L, window):
    assert bench.pairs_per_head([L], window) == brute_pairs(L, window)


def test_pairs_per_head_sums_sequences():
    assert bench.pairs_per_head([7, 0, 300], 128) == brute_pairs(7, 128) + brute_pairs(300, 128)


def _write_counters(d, counter, rows):
    os.makedirs(d, exist_ok=True)
    with open(os.path.join(d, "p_counter_collection.csv"), "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=["Dispatch_Id", "Kernel_Name", "Counter_Name", "Counter_Value"])
        w.writeheader()
        for i, (name, val) in enumerate(rows):
            # two rows per dispatch (as for a counter summed over several instances)
            w.writerow({"Dispatch_Id": i + 1, "Kernel_Name": name, "Counter_Name": counter, "Counter_Value": val / 2})
            w.writerow({"Dispatch_Id": i + 1, "Kernel_Name": name, "Counter_Name": counter, "Counter_Value": val / 2})


def test_traffic_summary_scales_by_copy(tmp_path, monkeypatch):
    fetch, write = str(tmp_path / "f"), str(tmp_path / "w")
    k = "void mimo::(anonymous namespace)::"
    gib_kib = bench.COPY_BYTES / 1024
    step = [(k + "kv_prep_kernel(...)", 100.0), (k + "attn_fwd_kernel<4, 8, true, true>(...)", 400.0)]
    # warm step, fill + copy, traced step
    _write_counters(fetch, "FETCH_SIZE", step + [("fill", 0.0), ("__amd_rocclr_copyBuffer", gib_kib / 2)] + step)
    _write_counters(write, "WRITE_SIZE", step + [("fill", gib_kib), ("__amd_rocclr_copyBuffer", gib_kib)] + step)
    with open(os.path.join(fetch, "traffic_order.json"), "w") as f:
        json.dump({"launches": ["kv_prep_swa", "attn_fwd_swa"]}, f)
    (tmp_path / "profiles").mkdir()
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    monkeypatch.setattr(bench, "kernel_source_hash", lambda: "h")
    bench.traffic_summary(fetch, write)
    out = json.load(open(tmp_path / "profiles" / "traffic.json"))
    assert out["fetch_size_scale"] == 2.0 and out["write_size_scale"] == 1.0
    assert out["kernels"]["attn_fwd_swa"] == {"fetch_bytes": 400 * 1024 * 2, "write_bytes": 400 * 1024,
                                              "bytes_per_launch": 400 * 1024 * 3}
    assert bench.measured_traffic("attn_fwd_swa") == 400 * 1024 * 3
    monkeypatch.setattr(bench, "kernel_source_hash", lambda: "changed")
    assert bench.measured_traffic("attn_fwd_swa") is None


def test_traffic_summary_rejects_misaligned_launches(tmp_path, monkeypatch):
    fetch, write = str(tmp_path / "f"), str(tmp_path / "w")
    k = "void mimo::(anonymous namespace)::"
    rows = [("__amd_rocclr_copyBuffer", bench.COPY_BYTES / 1024), (k + "bwd_dq_kernel<4, 8, false>(...)", 1.0)]
    _write_counters(fetch, "FETCH_SIZE", rows)
    _write_counters(write, "WRITE_SIZE", rows)
    with open(os.path.join(fetch, "traffic_order.json"), "w") as f:
        json.dump({"launches": ["bwd_dkdv_global"]}, f)
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    monkeypatch.setattr(bench, "kernel_source_hash", lambda: "h")
    with pytest.raises(SystemExit):
        bench.traffic_summary(fetch, write)


def test_cached_pairs_counts_visible_keys():
    """Pairs of a chunked prefill: brute force over key positions (cache rows precede the chunk)."""
    import bench

    def brute(chunks, rows, window):
        tot = 0
        for L, n in zip(chunks, rows):
            for i in range(L):
                p = n + i                          # the query's position when the cache starts at 0
                tot += sum(1 for j in range(n + i + 1) if window < 0 or j >= p - window)
        return tot
    for chunks, rows, window in [([3, 2, 0], [4, 0, 9], -1), ([5, 130], [200, 3], 128), ([7], [2], 0)]:
        assert bench.cached_pairs(chunks, rows, window) == brute(chunks, rows, window)


def test_kernel_hash_ignores_comments_only(tmp_path):
    """The traffic counters are tied to the kernels' code: a comment or whitespace edit keeps the hash, a code
    edit (even inside a line that also holds a comment, or in a string) changes it."""
    d = tmp_path / "csrc"
    d.mkdir()
    src = 'int f(int a) { // add one\n  return a + 1; /* done */ }\nconst char *s = "x // y";\n'
    (d / "k.hip").write_text(src)
    h0 = bench.kernel_source_hash(str(d))
    (d / "k.hip").write_text(src.replace("// add one", "// adds one to a").replace("  return", "\treturn"))
    assert bench.kernel_source_hash(str(d)) == h0
    (d / "k.hip").write_text(src.replace("a + 1", "a + 2"))
    assert bench.kernel_source_hash(str(d)) != h0
    (d / "k.hip").write_text(src.replace('"x // y"', '"x // z"'))
    assert bench.kernel_source_hash(str(d)) != h0
    (d / "notes.txt").write_text("not a source")
    (d / "k.hip").write_text(src)
    assert bench.kernel_source_hash(str(d)) == h0


def _write_trace(d, rows):
    """kernel_trace.csv with (dispatch id, kernel name, start ns, duration ns) rows."""
    os.makedirs(d, exist_ok=True)
    with open(os.path.join(d, "p_kernel_trace.csv"), "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=["Dispatch_Id", "Kernel_Name", "Start_Timestamp", "End_Timestamp"])
        w.writeheader()
        for i, name, t0, dt in rows:
            w.writerow({"Dispatch_Id": i, "Kernel_Name": name, "Start_Timestamp": t0, "End_Timestamp": t0 + dt})


def test_stats_summary_averages_the_timed_launches(tmp_path, capsys):
    k = "void mimo::(anonymous namespace)::bwd_dkdv_kernel<false>(mimo::BwdArgs)"
    # one cold warm-up launch of 9 us, then three timed launches of 6 us
    _write_trace(str(tmp_path), [(1, k, 0, 9000), (2, k, 20000, 6000), (3, k, 40000, 6000), (4, k, 60000, 6000)])
    bench.stats_summary(str(tmp_path), "t", "c", "3")
    line = [l for l in capsys.readouterr().out.splitlines() if l.startswith("bwd_dkdv_kernel")][0].split()
    assert line[1] == "4" and float(line[2]) == 6.8 and float(line[3]) == 6.0


def test_mfma_summary_rates_and_clock(tmp_path, capsys):
    d = str(tmp_path)
    k = "void mimo::(anonymous namespace)::bwd_dkdv_kernel<false>(mimo::BwdArgs)"
    with open(os.path.join(d, "traffic_order.json"), "w") as f:
        json.dump({"launches": ["bwd_dkdv_global"]}, f)
    with open(os.path.join(d, "p_counter_collection.csv"), "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=["Dispatch_Id", "Kernel_Name", "Counter_Name", "Counter_Value"])
        w.writeheader()
        # 2e12 flop executed (MOPS x 512) over two instances; 1700 cycles in a 1 us kernel (the counter sums the
        # 8 XCDs); busy 50% of 1024 SIMDs
        for part in (0.5, 0.5):
            w.writerow({"Dispatch_Id": 7, "Kernel_Name": k, "Counter_Name": "SQ_INSTS_VALU_MFMA_MOPS_BF16",
                        "Counter_Value": part * 2e12 / 512})
            w.writerow({"Dispatch_Id": 7, "Kernel_Name": k, "Counter_Name": "SQ_VALU_MFMA_BUSY_CYCLES",
                        "Counter_Value": part * 0.5 * 1700 * 1024})
            w.writerow({"Dispatch_Id": 7, "Kernel_Name": k, "Counter_Name": "GRBM_GUI_ACTIVE", "Counter_Value": 1700 * 8})
    _write_trace(d, [(7, k, 0, 1000)])
    bench.mfma_summary(d, "t", "c")
    line = [l for l in capsys.readouterr().out.splitlines() if l.startswith("bwd_dkdv_global")][0].split()
    assert float(line[3]) == 2.0 and float(line[4]) == 2e12 / 1e-6 / 1e12 and float(line[5]) == 50.0
    assert float(line[6]) == 1.7
