"""Dory (looped normalized GPT) token forward on MI355X (gfx950).

The compute path is the HIP library ``libdory.so`` behind the C ABI declared in
``include/dory.h``; ``looped_normalized_gpt_amd.dory`` is its thin Python binding.
``looped_normalized_gpt_amd.synth`` draws the seeded synthetic inputs.
"""
