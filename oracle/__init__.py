"""CPU float64 oracle for NSA selected attention.

Test infrastructure only: the tests, the smoke check and the benchmark's
CPU-baseline leg use it; the HIP path never imports it.
"""
from .fsa_oracle import build_index, key_indices, selected_attention, sequence_layout, valid_entries

__all__ = ["build_index", "key_indices", "selected_attention", "sequence_layout", "valid_entries"]
