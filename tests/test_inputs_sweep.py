"""Host logic of the batch-sweep workload: the 48 batch sizes and the production-like router
inputs ("MOE Bmm1 Fused Gather", the bench's batch sizes and prod-like logits)."""
import numpy as np

from moe_inputs import SWEEP_CONFIGS, get_config, make_logits, make_routing, make_x, sweep_batch_sizes
from moe_inputs import configs as C


def test_batch_sizes():
    b = sweep_batch_sizes(128, 4)
    assert len(b) == 48
    per = [v * 4 // 128 for v in b]
    assert per[:8] == [4, 5, 6, 7, 8, 10, 12, 14]
    assert per[8:16] == [16, 20, 24, 28, 32, 40, 48, 56]
    assert per[16:24] == [64, 80, 96, 112, 128, 160, 192, 224]
    assert per[24:] == list(range(256, 1024, 32))
    assert b[0] == 128 and b[-1] == 31744 == SWEEP_CONFIGS["gptoss_shard_bf16"].T
    assert all(x < y for x, y in zip(b, b[1:]))


def test_prefix_stable_inputs():
    small = get_config("gptoss_shard_bf16", T=96)
    big = get_config("gptoss_shard_bf16", T=640)
    assert np.array_equal(make_logits(small, 0), make_logits(big, 0)[:96])
    assert np.array_equal(make_x(small, 0), make_x(big, 0)[:96])


def test_prod_like_structure():
    """Without the per-token parts (cluster boost and Gumbel noise) the logits are the log
    Zipf popularity plus the batch-hot boost; the noise has the Gumbel(0, 0.75) mean."""
    cfg = get_config("gptoss_shard_bf16", T=4096)
    lg = make_logits(cfg, 0)
    base = np.median(lg, axis=0)                       # per-expert location
    # Zipf: the sorted per-expert locations fall by about 1.10 * log(rank) (cluster and hot
    # boosts perturb a few experts, so compare the slope over the long tail by least squares)
    srt = np.sort(base)[::-1]
    r = np.arange(1, 129)
    slope = np.polyfit(np.log(r[16:]), srt[16:], 1)[0]
    assert abs(slope + C.PROD_ZIPF_ALPHA) < 0.15, slope
    ids, w, _ = make_routing(cfg, 0)
    assert ids.min() >= 0 and ids.max() < 128
    assert all(len(set(row)) == 4 for row in ids.tolist())
    assert np.allclose(w.sum(axis=1), 1.0, atol=1e-6)
    counts = np.bincount(ids.reshape(-1), minlength=128)
    assert counts.max() > 0.5 * cfg.T                 # one expert takes most tokens
    assert (counts > 0).sum() > 64                     # and a long tail is still routed to
