"""MI355X-native salience/Hessian-weighted vector quantization of one weight matrix.

The package is a thin Python face over ``libvq.so`` (hand-written HIP kernels
for gfx950 behind a C ABI, declared in ``include/vq.h``).  Importing the
package loads nothing; ``hessian_weighted_vector_amd.vq`` loads the library on
first use and fails loudly when it is missing.
"""

__version__ = "0.1.0"
