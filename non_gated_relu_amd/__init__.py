"""Nemotron-H MoE layer forward on MI355X (gfx950): HIP kernels behind a C ABI.

``non_gated_relu_amd.binding`` is the Python face of libmoe.so (include/moe.h);
``non_gated_relu_amd.synthetic`` draws the seeded inputs.  Importing this
package loads nothing; the library loads on first use.
"""

__all__ = ["binding", "synthetic"]
