"""MI355X-native quantized-KV streaming decode attention.

The compute path lives in the HIP library ``libkvq.so`` (C ABI declared in
``include/kvq.h``); ``decode_attention_streaming_amd.kvq`` is its thin Python
binding and ``decode_attention_streaming_amd.synth`` the seeded workload
generator.
"""
