"""Bookkeeping formulas against the numbers the pretraining page prints."""

import json
import os

from dense_pretraining_amd.config import Config, flops_per_token, param_count

GOLD = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "pages_numbers.json")))


def test_from_depth_matches_page_shape():
    c = Config.from_depth(GOLD["depth"])
    assert (c.d_model, c.n_head, c.head_dim) == (GOLD["d_model"], GOLD["n_head"], GOLD["head_dim"])
    assert c.batch * c.seq_len * GOLD["n_gpu"] == GOLD["tokens_per_step"]


def test_param_count_matches_page():
    # ~560M is the count with one KV head per query head (10 KV heads)
    c10 = Config.from_depth(20, n_kv_head=10)
    assert param_count(c10) == 560_988_160
    assert abs(param_count(c10) / GOLD["params_approx"] - 1) < 0.01
    assert param_count(Config.from_depth(20)) == 502_005_760
    assert param_count(Config.from_depth(30, batch=16)) == 1_372_323_840


def test_total_flops_and_steps_match_page():
    c10 = Config.from_depth(20, n_kv_head=10)
    tokens = 20 * GOLD["params_approx"]
    assert abs(tokens / GOLD["chinchilla_tokens_approx"] - 1) < 0.01
    assert abs(tokens / GOLD["tokens_per_step"] / GOLD["steps_approx"] - 1) < 0.01
    total = flops_per_token(c10, "palm") * GOLD["chinchilla_tokens_approx"]
    assert abs(total / GOLD["total_flops_approx"] - 1) < 0.1


def test_flops_per_token_values():
    c = Config.from_depth(20)
    assert flops_per_token(c, "causal") == 2_823_290_880
    assert flops_per_token(c, "palm") == 3_137_863_680
