"""rotated_w4a4_quantized_amd -- the rotated low-bit quantized linear layer of
diffusion-transformer inference on AMD MI355X (gfx950).

    from rotated_w4a4_quantized_amd import rq
    rq.pack_weights(...)    # offline fold + quantize (librq host code)
    rq.rotate_quant(...)    # runtime: rotate + 4-bit quantize tokens (HIP)
    rq.w4a4_linear(...)     # runtime: low-bit GEMM + rescale (HIP)

The C ABI is include/rq.h; librq.so is built in-tree by
`python -m rotated_w4a4_quantized_amd.build`.  Importing the package does not
load the library; the first call does, and raises if it is missing.
"""
