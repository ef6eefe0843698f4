"""The layer shape the build computes reproduces the figures the pages print
(tests/golden/beam_page_figures.json, each entry citing its page)."""
import json
import os

from synth import BEAM

GOLD = json.load(open(os.path.join(os.path.dirname(__file__), "golden",
                                   "beam_page_figures.json")))


def _near(key, v):
    g = GOLD[key]
    assert abs(v - g["value"]) <= g.get("tol", 0), (key, v, g["value"])


def test_shape_matches_pages():
    _near("hidden_size", BEAM.hidden)
    _near("experts_per_layer", BEAM.n_experts)
    _near("experts_per_token", BEAM.top_k)
    _near("expert_intermediate", BEAM.intermediate)
    _near("groups", BEAM.n_groups)
    _near("experts_per_group", BEAM.group_size)
    _near("groups_kept", BEAM.topk_groups)
    _near("routed_scale", BEAM.routed_scale)


def test_parameter_closed_forms():
    per_expert = 3 * BEAM.hidden * BEAM.intermediate      # gate, up, down
    assert per_expert == 39_321_600
    _near("params_per_expert_approx", per_expert)
    moe_layers = GOLD["decoder_layers"]["value"] - GOLD["dense_layers"]["value"]
    assert moe_layers == 49
    experts = moe_layers * BEAM.n_experts * per_expert
    total = GOLD["total_params"]["value"]
    _near("expert_weight_share_percent", round(100 * experts / total, 1))
    rest = total - experts
    _near("replicated_params_under_ep", rest)
    active = moe_layers * BEAM.top_k * per_expert + rest
    _near("active_params_approx", active)
    _near("bf16_checkpoint_bytes_approx", 2 * total)
    # 8 H200s: replicated part on every card, experts split 8 ways
    _near("h200_bytes_per_card_8gpu", 2 * rest + 2 * experts / 8)
