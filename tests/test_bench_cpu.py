"""bench.py's host-side contract, checked without a GPU.

A request for more than one GPU stops with a message before any device work; a
machine with no GPU gets an error, never a CPU fallback; and the HBM traffic
recorded under profiles/ is reported only when its kernel-source hash matches
the sources.
"""

import os

import bench

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_is_refused(capsys):
    assert bench.main(["--gpus", "2"]) == 2
    assert "one GPU" in capsys.readouterr().err


def test_no_gpu_is_an_error_not_a_fallback(capsys):
    import torch

    if torch.cuda.is_available():
        return  # on a GPU machine the bench runs; this case is for hosts without one
    assert bench.main(["--steps", "1", "--warmup", "0"]) == 1
    assert "needs a GPU" in capsys.readouterr().err


def _write_counters(root, workload, sha, traffic):
    os.makedirs(os.path.join(root, "profiles"), exist_ok=True)
    with open(os.path.join(root, "profiles", f"attn_kernel_{workload}_counters.txt"), "w") as fh:
        fh.write("# test file\n")
        fh.write(f"kernel_src_sha256 = {sha}\n")
        fh.write(f"traffic_bytes_per_launch = {traffic}\n")


def test_recorded_traffic_only_for_matching_sources(tmp_path, monkeypatch):
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    monkeypatch.setattr(bench, "kernel_sha", lambda: "0123456789abcdef")
    assert bench.read_counters("w") is None  # no file
    _write_counters(str(tmp_path), "w", "0123456789abcdef", 1234)
    assert bench.read_counters("w") == 1234.0
    _write_counters(str(tmp_path), "w", "fedcba9876543210", 1234)
    assert bench.read_counters("w") is None  # counters taken for other kernel sources


def test_kernel_sha_covers_the_attention_sources():
    # every file the hash covers exists, and the hash is the 16-hex-digit form
    for f in bench.KERNEL_SOURCES:
        assert os.path.exists(os.path.join(ROOT, "segmented_attention_paged_amd", "csrc", f))
    sha = bench.kernel_sha()
    assert len(sha) == 16 and int(sha, 16) >= 0
