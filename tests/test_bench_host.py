"""Host-side logic of bench.py (no GPU): the source digest that ties a
counter summary to the kernel code, the algorithmic byte counts, and the
traffic arithmetic from rocprofv3 counter tables."""
import os

import numpy as np

import bench
import synthetic as syn


def test_digest_ignores_comments_and_blank_lines():
    a = "int f(int x) {\n    return x + 1;  // one more\n}\n"
    b = "// a new header comment\n\nint f(int x) {\n    return x + 1;\n}\n\n"
    c = "int f(int x) {\n    return x + 2;\n}\n"
    assert bench._code_only(a) == bench._code_only(b)
    assert bench._code_only(a) != bench._code_only(c)


def test_committed_traffic_matches_or_is_withheld():
    """A counter summary counts only while its digest matches the current
    kernel code; otherwise read_traffic gives None (never stale numbers)."""
    for kernel in ("fwd", "bwd"):
        t = bench.read_traffic(kernel, "single_cell_b32h8d64_lognormal800")
        assert t is None or t > 0
        path = os.path.join(bench.PROFILES, f"traffic_{kernel}_single_cell_b32h8d64_lognormal800.txt")
        text = open(path).read()
        matches = f"source_sha256_16: {bench.source_digest(kernel)}" in text
        assert (t is not None) == matches


def test_algorithmic_bytes_by_hand():
    w = syn.make_workload("t", seed=1, B=3, H=2, d=64, lengths="uniform", lo=10, hi=50,
                          tensors=())
    valid = int(np.clip(w.seq_lens, 0, w.L).sum()) * w.H
    every = w.B * w.L * w.H
    row = 2 * w.d
    assert bench.algorithmic_bytes("fwd", w) == (3 * valid + every) * row
    assert bench.algorithmic_bytes("bwd", w) == (4 * valid + 3 * every) * row


def _counter_table(dirname, rows):
    os.makedirs(dirname, exist_ok=True)
    with open(os.path.join(dirname, "p_counter_collection.csv"), "w") as f:
        f.write("Dispatch_Id,Kernel_Name,Counter_Name,Counter_Value\n")
        for i, (kernel, counter, value) in enumerate(rows):
            f.write(f'{i},"{kernel}",{counter},{value}\n')


def test_traffic_scaled_by_the_copy_reference(tmp_path):
    """Counters read KiB per dispatch; each is scaled by the ratio between the
    true size of a plain copy and what the same counter reads for it."""
    sym = "void sigattn::fwd_kernel<64, 0, 4, 2, 0, 1>(sigattn::AttnParams)"
    _counter_table(tmp_path / "fetch", [(sym, "FETCH_SIZE", 1000.0), (sym, "FETCH_SIZE", 1200.0),
                                        ("other", "FETCH_SIZE", 9e9)])
    _counter_table(tmp_path / "write", [(sym, "WRITE_SIZE", 500.0)])
    _counter_table(tmp_path / "cf", [("copy", "FETCH_SIZE", 128 * 1024.0)])  # reads half
    _counter_table(tmp_path / "cw", [("copy", "WRITE_SIZE", 256 * 1024.0)])  # exact
    w = syn.make_workload("t", seed=1, B=2, H=1, d=64, lengths="uniform", lo=10, hi=20,
                          tensors=())
    text = bench.summarize_traffic("fwd", str(tmp_path / "fetch"), str(tmp_path / "write"),
                                   str(tmp_path / "cf"), str(tmp_path / "cw"), 256, w, "t")
    fields = dict(line.split(": ", 1) for line in text.splitlines() if ": " in line
                  and not line.startswith("#"))
    assert float(fields["fetch_scale"]) == 2.0 and float(fields["write_scale"]) == 1.0
    assert int(fields["hbm_bytes_per_launch"]) == int((1100.0 * 2.0 + 500.0) * 1024)
    assert fields["source_sha256_16"] == bench.source_digest("fwd")


def test_cpu_baseline_reports_all_threads_and_one(monkeypatch):
    """The oracle's host rate on every host thread (the reported value) and
    on one thread, with the thread count and CPU model, on a bounded sample."""
    monkeypatch.setenv("OMP_NUM_THREADS", "2")
    w = syn.make_workload("t", seed=3, B=4, H=2, d=64, lengths="uniform", lo=20, hi=60,
                          tensors=("q", "k", "v", "do"))
    res = bench.cpu_baseline(w, budget_all_s=0.5, budget_one_s=0.5)
    assert res["kind"] == "oracle" and res["unit"] == "TFLOP/s"
    assert res["cores"] == min(2, os.cpu_count()) and res["value"] > 0
    assert res["single_thread"]["cores"] == 1 and res["single_thread"]["value"] > 0
    assert isinstance(res["cpu_model"], str) and res["cpu_model"]
    assert res["host_cpus"] == os.cpu_count()


def test_pairs_within_budget():
    w = syn.make_workload("t", seed=3, B=8, H=4, d=64, lengths="uniform", lo=100, hi=100,
                          tensors=())
    # 1e-6 s per n^2 on one thread: each pair costs 0.01 s, so 0.05 s holds 5.
    pairs = bench._pairs_within(w, 1e-6, 0.05, 1)
    assert len(pairs) == 5 and len(set(pairs)) == 5
    assert len(bench._pairs_within(w, 1e-6, 0.05, 2)) == 10
    assert len(bench._pairs_within(w, 1.0, 0.0, 1)) == 1  # never empty


def test_parity_errors_attach_to_matching_suite_rows(tmp_path):
    import json
    log = tmp_path / "parity.jsonl"
    base = {"B": 32, "H": 8, "L": 1584, "d": 64, "variant": "sigmoid", "block": 128,
            "mask": "none"}
    recs = [dict(base, direction="fwd", output="O", max_abs=1e-3, rel_l2=2e-3),
            dict(base, direction="bwd", output="dQ", max_abs=4e-3, rel_l2=1e-3),
            dict(base, direction="bwd", output="dK", max_abs=2e-3, rel_l2=3e-3),
            dict(base, direction="bwd", output="dV", max_abs=1e-3, rel_l2=1e-3),
            dict(base, block=64, direction="fwd", output="O", max_abs=9e-3, rel_l2=9e-3)]
    log.write_text("".join(json.dumps(r) + "\n" for r in recs))
    rows = [dict(base, kernel="fwd"), dict(base, kernel="bwd"), dict(base, kernel="dkdv"),
            dict(base, kernel="blockmask"), dict(base, kernel="fwd", variant="softmax")]
    bench.attach_parity(rows, str(log))
    assert rows[0]["max_abs"] == 1e-3 and rows[0]["parity_outputs"] == ["O"]
    assert rows[1]["max_abs"] == 4e-3 and rows[1]["rel_l2"] == 3e-3
    assert rows[2]["parity_outputs"] == ["dK", "dV"] and rows[2]["max_abs"] == 2e-3
    assert "max_abs" not in rows[3] and "max_abs" not in rows[4]


def test_counter_summary_ratios(tmp_path):
    sym = "void sigattn::bwd_kernel<64, 4, 2, 0, 0, 1>(sigattn::AttnParams)"
    _counter_table(tmp_path / "a", [(sym, "SQ_VALU_MFMA_BUSY_CYCLES", 1024 * 500.0),
                                    (sym, "GRBM_GUI_ACTIVE", 8 * 1000.0),
                                    (sym, "SQ_INSTS_MFMA", 10.0),
                                    (sym, "SQ_INSTS_VALU_TRANS_F32", 25.0),
                                    ("other", "SQ_INSTS_MFMA", 99.0)])
    text = bench.summarize_counters("bwd", [str(tmp_path / "a")])
    assert "| SQ_INSTS_MFMA | 1 | 10 |" in text
    assert "SQ_VALU_MFMA_BUSY_CYCLES / (GRBM_GUI_ACTIVE / 8 XCDs x 1024 SIMDs) | 0.5 |" in text
    assert "SQ_INSTS_VALU_TRANS_F32 per MFMA instruction | 2.5 |" in text
