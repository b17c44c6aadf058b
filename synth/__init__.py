"""Seeded synthetic workloads shared by the tests, the smoke check and the bench."""
from .gen import (CONFIGS, Config, make_inputs, make_custom_ffn, make_custom_mmid,  # noqa: F401
                  f32_to_bf16_bits, bf16_bits_to_f32, draw_ids_uniform, draw_ids_zipf,
                  draw_route_w, draw_router_logits, zipf_popularity)
