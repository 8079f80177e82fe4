"""MI355X-native sparse MoE FFN layer: a C-ABI HIP library plus a thin Python binding.

``synth`` (seeded inputs) imports nothing else; the binding in ``moe`` loads the built
``libsmoe.so`` and fails loudly when it is missing.
"""
