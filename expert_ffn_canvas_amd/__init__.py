"""MI355X-native top-8-of-128 mixture-of-experts feed-forward layer (DiffusionGemma 26B-A4B shape).

The compute path lives in the HIP library libdgmoe.so behind the C ABI in include/dg_moe.h;
`expert_ffn_canvas_amd.dgmoe` is its ctypes binding (argument marshalling only) and
`expert_ffn_canvas_amd.synth` draws seeded synthetic inputs.
"""
__all__ = ["dgmoe", "synth"]
