"""The random sweep's configurations are valid layers: the library's host checks accept
every one of them (workspace sizes for the forward and the backward), and they cover every
option value at least once."""
import os

import pytest

from mixture_experts_layer_group_amd import binding

import random_layers


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(binding.LIB_PATH):
        from mixture_experts_layer_group_amd import build
        build.build(verbose=False)
    return binding.load_library()


def test_random_configs_pass_host_checks(lib):
    for cfg in random_layers.CASES:
        assert binding.moe_workspace_size(cfg) > 0, cfg["name"]
        assert binding.moe_backward_workspace_size(cfg) > 0, cfg["name"]


def test_random_configs_cover_the_options():
    cases = random_layers.CASES
    for field, values in (("act", {0, 1, 2}), ("gate_norm", {0, 1, 2}), ("dtype", {0, 1}),
                          ("random_routing", {0, 1}), ("residual", {0, 1})):
        assert {c[field] for c in cases} == values, field
    assert any(c["n_shared"] > 0 for c in cases)
    assert any(c["topk_groups"] < c["expert_groups"] for c in cases)
    assert any(c["n_groups"] > 1 for c in cases)
    assert any(c["top_k"] > 2 for c in cases)
