"""Shapes read from user-supplied MoE model configs (the route by which a
model whose shapes are not built in, such as the Gemma-4-26B-A4B model the
PagedWeight pages evaluate on, becomes a workload).  Host-only checks of the
parser; the GPU parity of such a workload is in test_gpu_parity.py."""
import json
import os

import pytest

import pw_synth

HERE = os.path.dirname(os.path.abspath(__file__))
EXAMPLE = os.path.join(HERE, "configs", "example_moe_config.json")


def test_qwen2_moe_style_keys():
    shape, layers, _ = pw_synth.shape_from_model_config(dict(
        hidden_size=2048, intermediate_size=5632, moe_intermediate_size=1408, num_experts=60,
        num_experts_per_tok=4, shared_expert_intermediate_size=5632, num_hidden_layers=24))
    # the routed width is the MoE one, not the dense MLP's intermediate_size
    assert shape == pw_synth.CONFIGS[1].shape and layers == 24


def test_mixtral_style_keys():
    shape, layers, _ = pw_synth.shape_from_model_config(dict(
        hidden_size=4096, intermediate_size=14336, num_local_experts=8, num_experts_per_tok=2,
        num_hidden_layers=32))
    assert shape == pw_synth.CONFIGS[2].shape and layers == 32


def test_shared_experts_counted_in_routed_widths():
    shape, _, _ = pw_synth.shape_from_model_config(dict(
        hidden_size=2048, moe_intermediate_size=1408, n_routed_experts=64, num_experts_per_tok=6,
        n_shared_experts=2))
    assert (shape.E, shape.top_k, shape.I_shared) == (64, 6, 2 * 1408)


def test_example_file_nested_text_config():
    shape, layers, name = pw_synth.shape_from_model_config(EXAMPLE)
    assert shape == pw_synth.LayerShape(H=1120, I=352, E=24, top_k=6, I_shared=704)
    assert layers == 4 and name == "example-moe"
    spec = pw_synth.model_config_spec(EXAMPLE, tokens=(3,))
    assert spec.shape == shape and list(spec.tokens) == [3] and spec.extra["user_config"]


def test_direct_shape_keys_and_path_name(tmp_path):
    p = tmp_path / "tiny.json"
    p.write_text(json.dumps(dict(H=64, I=32, E=2, top_k=1)))
    shape, layers, name = pw_synth.shape_from_model_config(str(p))
    assert shape == pw_synth.LayerShape(H=64, I=32, E=2, top_k=1) and layers == 1 and name == "tiny"


@pytest.mark.parametrize("cfg, msg", [
    (dict(hidden_size=64, moe_intermediate_size=32, num_experts=4), "top_k"),
    (dict(hidden_size=100, moe_intermediate_size=32, num_experts=4, num_experts_per_tok=2), "multiples of 32"),
    (dict(hidden_size=64, moe_intermediate_size=48, num_experts=4, num_experts_per_tok=2), "multiples of 32"),
    (dict(hidden_size=64, moe_intermediate_size=32, num_experts=4, num_experts_per_tok=5), "top_k"),
    (dict(hidden_size=64, moe_intermediate_size=32, num_experts=4, num_experts_per_tok=2,
          shared_expert_intermediate_size=40), "multiples of 32"),
])
def test_rejected_configs(cfg, msg):
    with pytest.raises(ValueError, match=msg):
        pw_synth.shape_from_model_config(cfg)
