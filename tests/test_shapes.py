"""The layer shape used by the library, the oracle and the inputs, pinned to
the sizes the pages print (tests/golden/checkpoint_payloads.txt): the routed
expert weights of all MoE layers, in each format's stored size, must fit in
that format's checkpoint payload, and the layer and expert counts must agree
with the stated total.  A wrong width, expert width or expert count (or a
wrong bytes-per-weight of a format) breaks one of these."""
import os

from sparse_moe_routed_amd import synth

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "checkpoint_payloads.txt")


def _facts():
    facts, payload = {}, {}
    for line in open(GOLDEN):
        line = line.split("#")[0].split()
        if not line:
            continue
        if line[0] == "payload":
            payload[line[1]] = float(line[2]) * 1e9
        else:
            facts[line[0]] = int(line[1])
    return facts, payload


def test_layer_shape_matches_the_pages():
    facts, _ = _facts()
    d = synth.Dims()
    assert (d.hidden, d.ffn, d.n_experts, d.top_k) == (
        facts["hidden"], facts["ffn"], facts["experts"], facts["top_k"])
    assert synth.N_MOE_LAYERS == facts["moe_layers"]
    assert facts["moe_layers"] * facts["experts"] == facts["experts_total"]


def test_routed_experts_fit_each_checkpoint_payload():
    facts, payload = _facts()
    per_expert = 2 * facts["hidden"] * facts["ffn"]  # up and down projections
    n = facts["experts_total"]
    stored = {
        "bf16": 2.0,               # bf16 values
        "fp8": 1.0 + 4.0 / (per_expert / 2),     # E4M3 codes + one fp32 scale per projection
        "nvfp4": 0.5 + 1.0 / 16 + 4.0 / (per_expert / 2),  # E2M1 + E4M3 per 16 + fp32
    }
    expert_bytes = {f: n * per_expert * b for f, b in stored.items()}
    for f, b in expert_bytes.items():
        assert b < payload[f], (f, b, payload[f])
    # the rest of each folder (attention, Mamba-2, encoders, heads) is a
    # positive remainder, and the bf16 folder's routed experts are most of it
    assert 0.8 < expert_bytes["bf16"] / payload["bf16"] < 1.0
    # the bytes per weight order the folders the same way the payloads do
    assert expert_bytes["nvfp4"] < expert_bytes["fp8"] < expert_bytes["bf16"]
    assert payload["nvfp4"] < payload["fp8"] < payload["bf16"]
