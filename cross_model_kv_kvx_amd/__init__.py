"""MI355X-native cross-model KV-cache translation.

``cross_model_kv_kvx_amd.kvx`` is the binding to the HIP library
(``libkvx.so``); ``cross_model_kv_kvx_amd.synth`` draws seeded inputs.
"""
