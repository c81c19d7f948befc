"""BitLinear forward of BitNet b1.58 on AMD MI355X (gfx950).

The compute path is the C-ABI library ``libbitlinear.so`` built from ``csrc/``;
``bitlinear`` is its thin ctypes binding (argument marshalling only).  Import
``ternary_weight_linear_forward_amd.bitlinear`` to load the library; importing
the package itself loads nothing, so the seeded input generators in ``synth``
can be used without a GPU.
"""
