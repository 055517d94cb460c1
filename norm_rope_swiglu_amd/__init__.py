"""MI355X-native fused per-token decoder-layer ops (RMSNorm, residual-add +
RMSNorm, M-RoPE, SwiGLU; LayerNorm, M-RoPE + KV-cache append, softmax + top-k
sampling, RMSNorm fused into a Linear) as hand-written HIP kernels for gfx950 behind a C ABI
(include/nrs.h), with a thin torch-tensor binding."""
from ._native import NrsError, lib
from .ops import (Graph, add_layernorm, add_rmsnorm, decode_graph, layernorm, mrope,
                  mrope_kv_append, null_graph, rmsnorm, rmsnorm_linear, softmax_topk_sample, stream_probe,
                  swiglu)

__all__ = ["NrsError", "lib", "Graph", "add_layernorm", "add_rmsnorm", "decode_graph", "layernorm",
           "mrope", "mrope_kv_append", "null_graph", "rmsnorm", "rmsnorm_linear", "softmax_topk_sample",
           "stream_probe", "swiglu"]
