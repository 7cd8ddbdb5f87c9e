"""Host-side logic of bench.py (no GPU): the one-GPU refusal, the algorithmic byte
count of a step and the gate on the measured-traffic summary."""
import subprocess
import sys

import pytest

import bench


def test_more_than_one_gpu_is_refused():
    res = subprocess.run([sys.executable, "bench.py", "--gpus", "2"], cwd=bench.ROOT,
                         capture_output=True, text=True, timeout=300)
    assert res.returncode == 2
    assert "one GPU" in res.stdout


@pytest.mark.parametrize("masked", [False, True])
@pytest.mark.parametrize("residual_bytes", [2, 4])
def test_algorithmic_bytes_counts_every_tensor_once_per_pass(masked, residual_bytes):
    B, N, H, D = 2, 96, 3, 32
    pair = B * N * N * H * D          # elements of q, k, v, o, dO and the gradients
    bias = B * H * N * N              # elements of bias, dbias and lse
    mask = B * N * N if masked else 0
    forward_reads = {"q": 2 * pair, "k": 2 * pair, "v": 2 * pair, "bias": 2 * bias, "mask": mask}
    forward_writes = {"o": 2 * pair, "residual": residual_bytes * pair, "lse": 4 * bias}
    backward_reads = {"q": 2 * pair, "k": 2 * pair, "v": 2 * pair, "o": 2 * pair,
                      "residual": residual_bytes * pair, "dO": 2 * pair, "lse": 4 * bias,
                      "bias": 2 * bias, "mask": mask}
    backward_writes = {"dq": 2 * pair, "dk": 2 * pair, "dv": 2 * pair, "dbias": 2 * bias}
    total = sum(sum(d.values()) for d in (forward_reads, forward_writes, backward_reads, backward_writes))
    assert bench.algorithmic_bytes(B, N, H, D, masked, residual_bytes) == total


def test_traffic_is_reported_only_for_a_matching_build(tmp_path, monkeypatch):
    prof = tmp_path / "profiles"
    prof.mkdir()
    monkeypatch.setattr(bench, "ROOT", tmp_path)
    assert bench.measured_traffic("crop768", False) is None          # no summary
    (prof / "traffic_bwd_main_crop768.md").write_text(
        f"traffic_bytes_per_launch: 123\nbuild_sha256: {bench.build_hash()}\n")
    assert bench.measured_traffic("crop768", False) == 123
    assert bench.measured_traffic("crop768", True) is None           # other orientation
    assert bench.measured_traffic("crop768", False, "bf16") is None  # other residual
    (prof / "traffic_bwd_main_crop768.md").write_text(
        "traffic_bytes_per_launch: 123\nbuild_sha256: " + "0" * 64 + "\n")
    assert bench.measured_traffic("crop768", False) is None          # other source or flags


def test_row_chunks_follow_one_round_of_workgroups():
    assert bench.row_chunks(48, 768) == 5     # crop768, H = 4: 240 of 256 compute units
    assert bench.row_chunks(384, 128) == 1    # more groups than compute units: one chunk
    assert bench.row_chunks(16, 64) == 16
    assert bench.row_chunks(2, 96) == 96      # never more chunks than rows
    assert bench.row_chunks(40, 640) == 6     # 107 rows per chunk: 6 chunks cover 640
    # 8 heads at D = 16: 96 groups; one round (2 chunks) would leave 64 of 256 CUs idle,
    # so three full rounds of 8 chunks of 96 rows
    assert bench.row_chunks(96, 768) == 8


def test_bias_dbias_bytes_at_crop768():
    d = bench.bias_dbias_bytes(1, 768, 4)
    nb = 4 * 768 * 768
    assert d["bias_tensor_bytes"] == 2 * nb
    assert d["bias_staged_bytes"] == 10 * 2 * nb        # five row chunks in each pass
    assert d["dbias_partial_bytes"] == 5 * 4 * nb
    assert d["dbias_reduction_bytes"] == 5 * 4 * nb + 2 * nb


@pytest.mark.parametrize("B,N,H,D", [(1, 768, 4, 32), (1, 640, 4, 32), (1, 384, 4, 32), (2, 352, 3, 32),
                                     (1, 768, 8, 16), (3, 128, 64, 32), (1, 96, 1, 16),
                                     (1, 768, 2, 64), (2, 96, 3, 64), (1, 256, 33, 64)])
def test_row_chunks_match_the_library_plan(B, N, H, D):
    """The library's backward workspace is the statistics, the dQ partials (one per
    key block: 64 keys, 32 at D = 64) and one fp32 dbias partial per row chunk, each 256-byte aligned:
    rebuilt from bench.row_chunks it must equal tri_attn_bwd_workspace_bytes."""
    import ctypes
    import triangle_attention_amd as ta
    lib = ta.load_library()
    got = lib.tri_attn_bwd_workspace_bytes(ctypes.byref(ta.make_problem(B, N, H, D)))

    def a256(x):
        return (x + 255) // 256 * 256
    T = -(-N // bench.block_size(D))
    C = bench.row_chunks(B * H * T, N)
    want = a256(B * N * H * 2 * N * 4) + a256(T * B * N * N * H * D * 2) + a256(C * B * H * N * N * 4)
    assert got == want
