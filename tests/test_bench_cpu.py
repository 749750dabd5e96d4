"""Host logic of the benchmark (CPU): argument checks, the byte counts it
derives from rocprofv3 counter CSVs, and the committed traffic records it
reports beside the roofline.

The traffic figure is HBM bytes per launch from raw TCC request counters: a
read request of 32, 64 or 128 bytes and a write request of 64 bytes or
(the rest) 32 bytes. A plain copy of a known size must come out as exactly
its size, and a record taken on another version of a kernel's source must
not be reported.
"""
import csv
import json
import os
import shutil

import pytest

import bench

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_refuses_more_than_one_gpu(capsys):
    assert bench.main(["--gpus", "2"]) == 2
    assert "one GPU" in capsys.readouterr().err
    assert bench.main(["--gpus", "8"]) == 2


def test_refuses_empty_timed_region():
    assert bench.main(["--steps", "0"]) == 2
    assert bench.main(["--warmup", "-1"]) == 2


def test_decode_bytes_per_token_head():
    # state read and written in fp32, r w k v a b in, o out in fp32
    assert bench.decode_bytes_per_token_head(2) == 33792
    assert bench.decode_bytes_per_token_head(4) == 34560


def _write_csv(path, rows):
    with open(path, "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=["Dispatch_Id", "Kernel_Name",
                                          "Grid_Size", "Counter_Name",
                                          "Counter_Value"])
        w.writeheader()
        for r in rows:
            w.writerow(r)


def _rows(kernel, dispatch, grid, counters):
    return [{"Dispatch_Id": dispatch, "Kernel_Name": kernel, "Grid_Size": grid,
             "Counter_Name": c, "Counter_Value": v} for c, v in counters.items()]


def test_pmc_summary_counts_a_copy_of_known_size(tmp_path):
    """1 MiB read in 128-byte requests and written in 64-byte requests: 1 MiB
    each way, with no fitted factor."""
    mib = 2**20
    rd = {"TCC_EA0_RDREQ_sum": mib // 128, "TCC_EA0_RDREQ_32B_sum": 0,
          "TCC_EA0_RDREQ_64B_sum": 0, "TCC_EA0_RDREQ_128B_sum": mib // 128}
    wr = {"TCC_EA0_WRREQ_sum": mib // 64, "TCC_EA0_WRREQ_64B_sum": mib // 64}
    r, w = tmp_path / "r.csv", tmp_path / "w.csv"
    _write_csv(r, _rows("copy_kernel(uint4*)", 1, 4096, rd) +
               _rows("other_kernel", 2, 4096, {k: 7 for k in rd}))
    _write_csv(w, _rows("copy_kernel(uint4*)", 1, 4096, wr))
    m = bench.pmc_summary([str(r), str(w)], "copy_kernel")["grid4096"]
    assert m["read_bytes"] == mib
    assert m["write_bytes"] == mib
    assert m["dispatches"] == 1


def test_pmc_summary_mixed_request_sizes_and_grids(tmp_path):
    """Each request size counts its own bytes; writes that are not 64-byte
    requests count 32; dispatches are averaged per grid size."""
    p = tmp_path / "c.csv"
    rows = []
    # grid 1024: two dispatches, means 3x128 + 5x64 + 7x32 read,
    # 4x64 + 2x32 written
    for d, (a, b, c, w64, w32) in enumerate([(2, 4, 6, 3, 1), (4, 6, 8, 5, 3)]):
        rows += _rows("k<1>", d, 1024, {
            "TCC_EA0_RDREQ_sum": a + b + c, "TCC_EA0_RDREQ_128B_sum": a,
            "TCC_EA0_RDREQ_64B_sum": b, "TCC_EA0_RDREQ_32B_sum": c,
            "TCC_EA0_WRREQ_sum": w64 + w32, "TCC_EA0_WRREQ_64B_sum": w64})
    # grid 64: one dispatch, reads only
    rows += _rows("k<1>", 9, 64, {
        "TCC_EA0_RDREQ_sum": 1, "TCC_EA0_RDREQ_128B_sum": 1,
        "TCC_EA0_RDREQ_64B_sum": 0, "TCC_EA0_RDREQ_32B_sum": 0})
    _write_csv(p, rows)
    s = bench.pmc_summary([str(p)], "k<1>")
    g = s["grid1024"]
    assert g["dispatches"] == 2
    assert g["read_bytes"] == 3 * 128 + 5 * 64 + 7 * 32
    assert g["write_bytes"] == 4 * 64 + 2 * 32
    # per-dispatch values, as MiB to two decimals: two reads, two writes
    assert sum(g["per_dispatch_values"].values()) == 4
    assert s["grid64"]["read_bytes"] == 128
    assert "write_bytes" not in s["grid64"]


RECORDS = {
    # kind: algorithmic bytes per launch of the workload the record covers
    "decode": 256 * 32 * 33792,
    "decode_large": 1024 * 64 * 33792,
    "prefill": 8 * 4096 * 32 * (6 * 64 * 2 + 4 * 64) + 8 * 32 * 2 * 4 * 64 * 64,
    "prefill_f32": 8 * 4096 * 32 * (6 * 64 * 4 + 4 * 64) + 8 * 32 * 2 * 4 * 64 * 64,
}


@pytest.mark.parametrize("kind", sorted(RECORDS))
def test_committed_traffic_record_is_current(kind):
    """Every committed record was taken on the kernel source as it stands
    (else the benchmark reports its traffic as null) and moves the
    workload's algorithmic bytes to within 0.1%."""
    with open(os.path.join(ROOT, "profiles", f"{kind}_traffic.json")) as f:
        t = json.load(f)
    assert t["kernel_sha"] == bench.kernel_sha(t["kernel_src"]), (
        f"{kind}_traffic.json was taken on another version of "
        f"{t['kernel_src']}")
    got = bench.load_traffic(kind, RECORDS[kind])
    assert got == t["hbm_bytes_per_launch"]
    assert abs(got / RECORDS[kind] - 1) < 1e-3, (got, RECORDS[kind])


def test_stale_traffic_record_is_not_reported(tmp_path, monkeypatch):
    root = tmp_path / "repo"
    (root / "profiles").mkdir(parents=True)
    src = root / "linear_attention_rnn_amd" / "csrc"
    src.mkdir(parents=True)
    with open(os.path.join(ROOT, "profiles", "decode_traffic.json")) as f:
        t = json.load(f)
    for name in t["kernel_src"]:
        shutil.copy(os.path.join(ROOT, "linear_attention_rnn_amd", "csrc",
                                 name), src / name)
    shutil.copy(os.path.join(ROOT, "profiles", "decode_traffic.json"),
                root / "profiles" / "decode_traffic.json")
    monkeypatch.setattr(bench, "ROOT", str(root))
    assert bench.load_traffic("decode", 1.0) == t["hbm_bytes_per_launch"]
    with open(src / t["kernel_src"][-1], "a") as f:
        f.write("\n// edited\n")
    assert bench.load_traffic("decode", 1.0) is None
    assert bench.load_traffic("no_such_kernel", 1.0) is None
