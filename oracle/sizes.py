"""Per-token KV-cache size closed form.

Every token keeps one key and one value in every layer, so its cache takes
2 x hidden x layers x bytes-per-number (KV 缓存与分页注意力 §03, the OPT-13B
example; KV Cache从原理到实战 §2.2, the LLaMA-2 7B example).  For grouped or
multi-query attention the "hidden" that is cached is the KV width,
num_kv_heads x head_dim (KV 缓存与分页注意力 §11: Falcon-7B and Llama 2 70B).
"""


def kv_bytes_per_token(num_kv_heads: int, head_dim: int, num_layers: int, dtype_bytes: int) -> int:
    return 2 * (num_kv_heads * head_dim) * num_layers * dtype_bytes
