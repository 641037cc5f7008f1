"""Forward implicit-GEMM convolution for MI355X (gfx950).

The binding to the C-ABI library lives in ``implicit_gemm_convolution_conv_amd.binding``;
importing this package loads nothing.
"""
