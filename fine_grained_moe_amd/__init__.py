"""MI355X-native fine-grained MoE FFN layer (dots.llm1 shapes) on gfx950.

Importing the package loads nothing native.  `fine_grained_moe_amd.moe`
loads the HIP library (libmoe.so) and raises if it is missing;
`fine_grained_moe_amd.synthetic` draws seeded inputs and needs no GPU.
"""
