"""Layer-sliding offloaded fine-tuning hot path for AMD MI355X (gfx950).

libslide (HIP kernels + host runtime, C ABI in include/slide.h) does all the work; this package
holds its build script, a ctypes binding with the C names (binding), and the thread-based step
engine that drives the slot ring, the copy streams and the CPU optimizer (engine).
"""
from .binding import *  # noqa: F401,F403
from ._capi import LIB_PATH, SlideError, lib  # noqa: F401

__version__ = "0.1.0"
