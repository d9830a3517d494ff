"""libdiffattn: causal differential attention on AMD MI355X (gfx950).

``differential_attention_causal_amd.diffattn`` is the ctypes binding of the C
library built from ``csrc/``; ``synth`` draws the seeded synthetic inputs.
Importing the binding loads the library lazily and raises if it is missing.
"""
