"""MI355X-native prefill of the Qwen3-VL text decoder truncated at layer 50.

The compute path is the C-ABI library ``libmhe.so`` (hand-written HIP for
gfx950, built from ``csrc/``); ``binding`` wraps it with ctypes. Importing this
package loads nothing: the library is opened on first use of ``binding``.
"""

__all__ = ["binding", "synth"]
