"""Seeded synthetic inputs for the decoder-layer ops (no op arithmetic here)."""
from .configs import Layer, Workload, decode, prefill, prefill_positions, ragged, ragged_lengths, sweep, tiny
from .gen import normal, raw64, splitmix64_int, store, stream_key, uniform

__all__ = [
    "Layer", "Workload", "decode", "prefill", "prefill_positions", "ragged", "ragged_lengths",
    "sweep", "tiny", "normal", "raw64", "splitmix64_int", "store", "stream_key", "uniform",
]
