"""Host logic of bench.py (CPU): the HBM traffic it reports comes from a
committed rocprofv3 counter summary only while the kernel's source, and the
device headers every kernel includes, are unchanged since the counters were
taken; otherwise it reports none."""
import shutil

import pytest


@pytest.fixture
def fake_root(tmp_path, monkeypatch):
    import bench
    src = bench.ROOT / "mamba_ssd_scan_02_amd" / "csrc"
    csrc = tmp_path / "mamba_ssd_scan_02_amd" / "csrc"
    csrc.mkdir(parents=True)
    for f in ("chunk_scan.hip", "device_common.h", "lds_pipe.h"):
        shutil.copy(src / f, csrc / f)
    (tmp_path / "profiles").mkdir()
    monkeypatch.setattr(bench, "ROOT", tmp_path)
    return tmp_path


def _write_summary(root, kernel, workload, hbm_bytes, digest):
    (root / "profiles" / f"{kernel}_{workload}_counters.txt").write_text(
        f"# HBM traffic of {kernel} on {workload}\n"
        f"hbm_bytes_per_dispatch: {hbm_bytes:g}\n"
        f"source_sha256_16: {digest}\n")


def test_traffic_follows_the_source_hash(fake_root):
    import bench
    _write_summary(fake_root, "chunk_scan", "w", 8.77e8, bench.source_hash("chunk_scan"))
    assert bench.counter_traffic("chunk_scan", "w") == pytest.approx(8.77e8)
    # no summary for this workload, or a summary of other sources
    assert bench.counter_traffic("chunk_scan", "other") is None
    _write_summary(fake_root, "chunk_scan", "stale", 8.77e8, "0123456789abcdef")
    assert bench.counter_traffic("chunk_scan", "stale") is None


@pytest.mark.parametrize("changed", ["chunk_scan.hip", "device_common.h", "lds_pipe.h"])
def test_any_source_change_voids_the_traffic(fake_root, changed):
    import bench
    _write_summary(fake_root, "chunk_scan", "w", 8.77e8, bench.source_hash("chunk_scan"))
    f = fake_root / "mamba_ssd_scan_02_amd" / "csrc" / changed
    f.write_text(f.read_text() + "\n// edited\n")
    assert bench.counter_traffic("chunk_scan", "w") is None


def test_committed_summaries_name_their_kernels_and_commands():
    """Every committed counter summary carries its command, the copy-kernel
    calibration, its bytes and the hash it was taken against."""
    import bench
    files = sorted((bench.ROOT / "profiles").glob("*_counters.txt"))
    assert files
    for p in files:
        t = p.read_text()
        for key in ("command_fetch:", "command_write:", "calibration:", "hbm_bytes_per_dispatch:",
                    "algorithmic_bytes_per_dispatch:", "source_sha256_16:"):
            assert key in t, (p.name, key)


def test_kernel_names_map_to_the_stage_they_run():
    """Trace and counter summaries attribute each dispatch by its demangled
    name; every kernel of the forward's two paths and their gated forms must
    land under its own stage name."""
    import bench
    cases = {
        "void ssd::chunk_scan_paired_kernel<true, false>(ssd::bf16_t const*, int)": "chunk_scan_runs",
        "void ssd::chunk_scan_paired_kernel<true, true>(ssd::bf16_t const*, int)": "chunk_scan_runs_gated",
        "void ssd::chunk_scan_paired_kernel<false, false>(ssd::bf16_t const*, int)": "chunk_scan",
        "void ssd::chunk_scan_paired_kernel<false, true>(ssd::bf16_t const*, int)": "chunk_scan_gated",
        "void ssd::chunk_state_runs_kernel<256, 2>(ssd::bf16_t const*)": "chunk_state_runs",
        "void ssd::run_passing_kernel<ssd::bf16_t, 4, 4>(ssd::bf16_t const*)": "run_passing",
        "void ssd::chunk_state_mfmah_kernel<256, 2, true>(ssd::bf16_t const*)": "chunk_state_cumsum",
        "void ssd::chunk_state_mfmah_kernel<256, 2, false>(ssd::bf16_t const*)": "chunk_state",
        "void ssd::state_passing_kernel<ssd::bf16_t, 4, 4, true>(ssd::bf16_t const*)": "state_passing",
        "void ssd::state_walk_kernel<8>(ssd::bf16_t const*)": "state_scan",
        "__amd_rocclr_copyBuffer": "copy",
    }
    for name, want in cases.items():
        assert bench._short_kernel(name) == want, (name, bench._short_kernel(name))
