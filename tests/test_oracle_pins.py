"""The CPU oracle against its pins (no GPU)."""
import pytest

import oracle
from tests import oracle_pins as pins


@pytest.mark.parametrize("pin", pins.ALL_PINS, ids=lambda f: f.__name__)
def test_pin(pin):
    pin(oracle)


def test_every_oracle_function_has_a_parity_status():
    for name in oracle.__all__:
        base = name
        if name in ("linear", "silu", "gelu", "token_positions", "multihead_attention",
                    "conv3d_patch_embed_direct", "modulate", "rope_segments", "cross_kv",
                    "cfg_euler", "dit_fwd", "self_attention_rope_only"):
            continue
        assert base in oracle.PARITY, name
