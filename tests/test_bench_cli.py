"""bench.py's command-line contract on the host: more than one GPU is refused with a message
and exit status 2 (this layer runs on one GPU), --help lists the sweep options, the
sweep's shard block size follows the shard's own counts, and the parity record flags an output
or an alignment that differs from the oracle's."""
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


def test_parity_record_flags_planted_differences():
    """bench.py's parity record (host logic; no GPU): an output equal to the oracle's passes,
    one value moved past the tolerance fails, and an alignment that differs from the oracle's
    in one slot is not reported as bit-exact.  The 'GPU' buffers here are CPU tensors made
    from the oracle itself."""
    import numpy as np
    import torch
    sys.path.insert(0, ROOT)
    import bench
    import oracle
    from moe_inputs import get_config, make_case
    cfg = get_config("tiny_fp32")
    case = make_case(cfg, "cpu", seed=3)
    bm = 16
    _, ref, toks = bench.cpu_baseline(case, 16, case.ids_host, case.w_host)
    assert ref.shape == (16, cfg.H)
    o = oracle.align(case.ids_host, cfg.E, bm)

    def align_bufs():
        a = {k: torch.from_numpy(np.array(getattr(o, k))) for k in
             ("counts", "offsets", "sorted_slots", "slot_row", "tiles")}
        a["num_tiles"] = torch.tensor(o.num_tiles)
        return a

    out = torch.zeros((cfg.T, cfg.H), dtype=torch.float32)
    out[:16] = torch.from_numpy(ref)
    good = bench.parity_check(cfg, bm, out, align_bufs(), case.ids_host, ref, toks)
    assert good["within_tol"] and good["alignment_bit_exact"] and good["tokens_checked"] == 16

    bad_out = out.clone()
    bad_out[5, 7] += 2 * bench.PARITY_TOL["f32"] * float(np.abs(ref).max())
    r = bench.parity_check(cfg, bm, bad_out, align_bufs(), case.ids_host, ref, toks)
    assert not r["within_tol"] and r["alignment_bit_exact"]

    a = align_bufs()
    s0, s1 = int(a["sorted_slots"][0]), int(a["sorted_slots"][1])
    assert s0 != s1
    a["sorted_slots"][0], a["sorted_slots"][1] = s1, s0          # two slots swapped
    r = bench.parity_check(cfg, bm, out, a, case.ids_host, ref, toks)
    assert r["within_tol"] and not r["alignment_bit_exact"]
