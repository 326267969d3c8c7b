"""MI355X-native joint audio-video DiT denoising step.

The compute path is the HIP library ``libavdit.so`` (C-ABI in ``include/avdit.h``), bound by
``audio_video_diffusion_dit_amd._native``. ``inputs`` draws the seeded synthetic workloads and
``device`` moves them into device memory.
"""

__all__ = ["inputs"]
