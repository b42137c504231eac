"""fp64 CPU oracle for the Kimi-K3 attention-residual forward.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and
the CPU-baseline leg of ``bench.py`` may import this package.  It shares no
code with the GPU library (``kimi_k3_attention_amd``) and never imports it.
"""
from .oracle import (OracleResult, OracleTokens, attnres_oracle, attnres_oracle_tokens,
                     bf16_bits_to_f64, round_bf16_bits)

__all__ = ["OracleResult", "OracleTokens", "attnres_oracle", "attnres_oracle_tokens",
           "bf16_bits_to_f64", "round_bf16_bits"]
