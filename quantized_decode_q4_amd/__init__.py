"""MI355X (gfx950) Q4_K decode path: C-ABI HIP library + thin Python binding.

``quantized_decode_q4_amd.q4k`` loads libq4k.so (and fails loudly when it is
missing); ``quantized_decode_q4_amd.inputs`` is the seeded synthetic-input
generator, importable without the library.
"""
