"""Seeded input generators and the page facts they encode (CPU only)."""
import math
import os

import numpy as np
import pytest
import torch

from gdn_inputs import CHUNK_CONFIGS, DECODE_CONFIG, ChunkConfig, chunk_inputs, decode_inputs

HERE = os.path.dirname(os.path.abspath(__file__))


def _facts():
    out = {}
    with open(os.path.join(HERE, "golden", "page_facts.txt")) as f:
        for line in f:
            line = line.split("#", 1)[0].strip()
            if line:
                key, val = (x.strip() for x in line.split("="))
                out[key] = float(val)
    return out


FACTS = _facts()


def test_channel_gate_domain_matches_card():
    cap = FACTS["gate_cap_numerator"] / FACTS["gate_bs2"]
    assert cap == 5.0
    for name in ("channel_bf16", "channel_long"):
        assert CHUNK_CONFIGS[name].g_cap == cap
    assert DECODE_CONFIG.g_cap == cap
    cfg = CHUNK_CONFIGS["channel_bf16"].with_(B=2, H=2, T=300)
    d = chunk_inputs(cfg)
    g = d["g"]
    assert g.shape == (2, 300, 2, 128)
    assert float(g.min()) >= FACTS["gate_domain_lo"] and float(g.max()) <= FACTS["gate_domain_hi"]
    # the clamp is hit: softplus(N(0, 2^2)) exceeds 5 a few percent of the time
    assert float((g == -5).float().mean()) > 0.005
    alpha = torch.exp(g.double())
    assert float(alpha.min()) >= math.exp(-5) * (1 - 1e-7) and float(alpha.max()) <= 1


def test_long_prefill_state_is_three_mib_per_layer():
    cfg = CHUNK_CONFIGS["channel_long"]
    per_layer = cfg.H * cfg.K * cfg.V * 4
    assert per_layer == 3 * 2 ** 20
    total = FACTS["deltanet_layers"] * per_layer / 2 ** 20
    assert abs(total - FACTS["deltanet_state_total_mib_approx"]) < 1
    assert cfg.T == FACTS["native_context_tokens"]
    assert cfg.K == FACTS["bench_head_dim"]


@pytest.mark.parametrize("name", list(CHUNK_CONFIGS))
def test_config_shapes(name):
    cfg = CHUNK_CONFIGS[name]
    assert cfg.chunk == 64 and cfg.K in (64, 128) and cfg.V in (64, 128)


def test_chunk_inputs_properties_and_seed():
    cfg = ChunkConfig("t", B=2, H=3, T=70, K=64, V=32, dtype="bf16", gate="head")
    a = chunk_inputs(cfg)
    b = chunk_inputs(cfg)
    for key in ("q", "k", "v", "g", "beta"):
        assert torch.equal(a[key], b[key])
    assert a["S0"] is None
    assert a["q"].dtype == torch.bfloat16 and a["g"].dtype == torch.float32
    nq = a["q"].float().norm(dim=-1)
    assert float((nq - 1).abs().max()) < 1e-2  # unit norm up to bf16 rounding
    assert float(a["beta"].min()) > 0 and float(a["beta"].max()) < 1
    assert float(a["g"].max()) <= 0
    c = chunk_inputs(cfg, seed=1)
    assert not torch.equal(a["q"], c["q"])


def test_stress_gate_scaling():
    cfg = ChunkConfig("t", B=1, H=1, T=64, K=64, V=64, dtype="fp32", gate="head", g_scale=0.0)
    assert float(chunk_inputs(cfg)["g"].abs().max()) == 0.0


def test_decode_inputs_shapes():
    cfg = DECODE_CONFIG.with_(N=3, H=2, steps=4)
    d = decode_inputs(cfg)
    assert d["q"].shape == (4, 3, 2, 128) and d["g"].shape == (4, 3, 2, 128)
    assert d["S0"].shape == (3, 2, 128, 128) and d["S0"].dtype == torch.float32
    assert abs(float(d["S0"].std()) - 0.02) < 0.002
