"""Barrier-free small/medium-message AllReduce (sum) for N ranks emulated on one MI355X.

The compute path is the HIP library ``libar.so`` (sources in ``csrc/``, C ABI in
``include/ar.h``); :mod:`latency_collectives_amd._ar` is its ctypes binding. Nothing in this
package computes an AllReduce on the CPU.
"""

from ._ar import *  # noqa: F401,F403
from ._ar import ArError, lib  # noqa: F401
