"""MI355X-native Qwen Sparse Attention (QSA) hot path.

The compute runs in hand-written HIP kernels for gfx950 behind the C-ABI
library ``libqsa.so`` (declared in ``include/qsa.h``).  ``qsa`` is its thin
ctypes binding; ``synth`` draws the seeded synthetic inputs.  Importing the
package loads nothing: the library is opened on first use of ``qsa``.
"""
