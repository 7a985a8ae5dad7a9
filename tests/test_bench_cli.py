"""bench.py's command-line contract on the host: more than one GPU is refused with a message
and exit status 2 (this layer runs on one GPU), --help lists the sweep options, and the
sweep's shard block size follows the shard's own counts."""
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def run(*args):
    return subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), *args],
                          capture_output=True, text=True, timeout=120)


def test_more_than_one_gpu_is_refused():
    r = run("--gpus", "2")
    assert r.returncode == 2
    assert "one GPU" in r.stderr and r.stdout == ""


def test_help_lists_the_modes():
    r = run("--help")
    assert r.returncode == 0
    for opt in ("--sweep", "--sweep-block-m", "--routing", "--graph", "--dense-reference",
                "--copy-calibration", "--cpu-baseline"):
        assert opt in r.stdout


def test_shard_block_m_keys_on_local_counts():
    """The sweep's shard block size: the block-size rule of the slots a shard received per
    local expert that received any (a host function; no GPU)."""
    sys.path.insert(0, ROOT)
    import bench
    import routed_grouped_gemm_topk_amd as moe
    # 173 local slots on 10 active experts: 17.3 per expert -> 32-row blocks (the global mean
    # of the same 128-token batch, 4 per expert, would give 16)
    assert bench.shard_block_m(moe, 173, 10, "bf16", "bf16") == 32
    assert moe.moe_block_m_for(128 * 4 / 128, "bf16", "bf16") == 16
    assert bench.shard_block_m(moe, 0, 0, "bf16", "bf16") == 16           # nothing routed here
    assert bench.shard_block_m(moe, 41628, 16, "bf16", "bf16") == 256
    assert bench.shard_block_m(moe, 581, 13, "e4m3", "mxfp4") == 64       # 44.7 per expert
    assert bench.shard_block_m(moe, 41628, 16, "e4m3", "mxfp4") == 128
