"""Locate (and if absent, build) libdit.so for the tests."""
import os

import diffusion_transformer_video_amd as dit


def ensure_built():
    if not os.path.exists(dit.LIB_PATH):
        from diffusion_transformer_video_amd import build
        build.build()
    return dit.lib()
