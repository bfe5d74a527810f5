"""MI355X-native W4A16 grouped-quantized routed-MoE layer.

The compute path is the C-ABI library ``libmoe_w4a16.so`` (hand-written HIP
for gfx950); :mod:`w4a16_grouped_quantized_amd.binding` marshals arguments to
it.  :mod:`w4a16_grouped_quantized_amd.synth` holds the seeded input
generators.
"""
__all__ = ["synth"]
