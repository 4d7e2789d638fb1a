"""Qwen2 decoder forward (prefill + greedy decode) for AMD Instinct MI355X.

The compute lives in libq2.so (hand-written HIP kernels for gfx950, C ABI in
include/q2.h); this package only marshals arguments.  Importing it fails if
the library has not been built.
"""
from ._lib import (Q2Error, Q2Tensor, Q2Config, header_functions, version, lib, LIB_PATH,
                   q2_embedding, q2_linear, q2_linear_noalloc, NOALLOC_SCRATCH_BYTES, q2_linear_workspace_bytes, q2_self_attention_workspace_bytes,
                   workspace, q2_rms_norm, q2_rope, q2_self_attention, q2_swiglu, q2_add,
                   q2_argmax, q2_rearrange, q2_model_create, q2_model_device_bytes, q2_model_load_weight,
                   q2_model_prefill, q2_model_prefill_embeds, q2_model_hidden_view, q2_model_decode, q2_model_generate, q2_model_continue, q2_model_kv_view, q2_model_kv_scale_view, q2_model_replay_stage, q2_model_seq_prefill, q2_model_seq_release, q2_model_seq_length,
                   q2_model_free_pages, STAGE_QKV, STAGE_ATTN, STAGE_O,
                   STAGE_GATE_UP, STAGE_DOWN, STAGE_ATTN_CORE, q2_kv_quantize, q2_kv_dequantize, q2_model_length,
                   q2_model_reset, q2_model_set_decode_path, q2_model_decode_path, q2_model_check,
                   q2_model_destroy)
from .model import Model, make_config, load_model, weight_tensor

__all__ = ["Q2Error", "Q2Tensor", "Q2Config", "header_functions", "version", "lib", "LIB_PATH",
           "q2_embedding", "q2_linear", "q2_linear_noalloc", "NOALLOC_SCRATCH_BYTES", "q2_linear_workspace_bytes", "q2_self_attention_workspace_bytes",
           "workspace", "q2_rms_norm", "q2_rope", "q2_self_attention", "q2_swiglu", "q2_add",
           "q2_argmax", "q2_rearrange", "q2_model_create", "q2_model_device_bytes", "q2_model_load_weight",
           "q2_model_prefill", "q2_model_prefill_embeds", "q2_model_hidden_view", "q2_model_decode", "q2_model_generate", "q2_model_continue", "q2_model_kv_view", "q2_model_kv_scale_view", "q2_model_replay_stage", "q2_model_seq_prefill", "q2_model_seq_release",
           "q2_model_seq_length", "q2_model_free_pages", "STAGE_QKV", "STAGE_ATTN",
           "STAGE_O", "STAGE_GATE_UP", "STAGE_DOWN", "STAGE_ATTN_CORE", "q2_kv_quantize", "q2_kv_dequantize", "q2_model_length",
           "q2_model_reset", "q2_model_set_decode_path", "q2_model_decode_path", "q2_model_check",
           "q2_model_destroy", "Model", "make_config", "load_model", "weight_tensor"]
