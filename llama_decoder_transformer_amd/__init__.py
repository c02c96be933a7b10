"""MI355X-native Llama-2/3 decoder forward pass (prefill + KV-cached greedy decode).

Submodules:
  inputs   -- seeded synthetic shapes, weights, token ids and cache contents
  binding  -- ctypes binding of the C ABI in include/llm.h (libllm.so)
  model    -- LlamaModel: torch-allocated buffers driving the C ABI
  build    -- hipcc build of libllm.so for gfx950

Importing the package loads nothing native; ``binding`` loads libllm.so on
first use and raises if it is missing.
"""
