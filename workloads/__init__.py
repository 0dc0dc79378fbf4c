"""Seeded synthetic workloads (inputs only) shared by the oracle tests, the GPU tests and the benchmark."""
from .synth import (CONFIGS, MoEConfig, MoEInputs, generate, bf16_bits_from_f32, f32_from_bf16_bits,
                    random_logits, zipf_bias, FP8_MAX, BLOCK)
from .attn import QKConfig, QK_CONFIGS, QKInputs, generate_qk
