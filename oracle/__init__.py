"""CPU oracle for the routed MoE layer -- TEST INFRASTRUCTURE ONLY.

A plain, slow, float64 (and, for quantiser decisions, IEEE float32) NumPy
implementation of what the layer computes.  It shares no code with the HIP
path in `sparse_moe_routed_amd` and imports nothing from it except the seeded
input generators (`sparse_moe_routed_amd.synth`, which hold none of the
layer's arithmetic).  Only `tests/`, `__graft_entry__.smoke()` and the
`cpu_baseline` leg of `bench.py` may import it; the product path never does.

Sources (pages about NVIDIA Nemotron 3.5 Transcribe 30B-A4B):
  * bloomery issue #967 "model: Nemotron 3.5 Transcribe from safetensors on x86
    cards and DGX Spark", section 2 "Checkpoint facts": 23 MoE layers, width
    2688, top-6 routing over 128 experts, ungated ReLU^2, expert width 1856;
    FP8 is scalar-scale E4M3 W8A8, NVFP4 experts are W4A4.
  * same issue, section 3 "Existing owners and gaps": the experts have only
    up and down parts (no gate matrix); K=1856 leaves a 64-value tail.
  * audio.cpp "NVIDIA Nemotron 3.5 Transcribe" port notes, section "CPU weight
    offload": routing weights and expert activation are fixed formulas;
    grouped expert matmul may change floating point rounding.
  * same notes, section "Q4_K, Q3_K and Q2_K expert profiles": zero padding of
    K with matching zero activations leaves outputs unchanged.

Parity status per function is listed in each module's header.
"""
