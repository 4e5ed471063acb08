"""Seeded synthetic inputs for the structured-sparse weight GEMM.

This package only draws random numbers and shapes them into the workloads
that the tests, the smoke check and the bench feed to both sides (the HIP
library and the oracle).  It holds none of the GEMM or packing arithmetic.
The two synthetic pruners here stand in for training-time pruning, which the
pages describe but which needs data and training:

* 2:4 magnitude pruning (GPUSQ-ViT, "Boost Vision Transformer with
  GPU-Friendly Sparsity and Quantization", abstract): keep the two largest
  |w| of every four consecutive K entries of a column.
* tile-wise row/column pruning (Guo et al., "Accelerating Sparse DNN Models
  without Hardware-Support via Tile-Wise Sparsity", tile-wise pattern slide):
  each G-column tile keeps its own whole K-rows and N-columns.
"""

from .gen import (  # noqa: F401
    WORKLOAD_NAMES,
    make_workload,
    make_small_w24_f16,
    make_vit_base_fc1_i8,
    make_bert_base_fc1_tw,
    make_bert_base_fc1_tw_i8,
    make_bert_large_ffn_tw,
    vit_large_layers,
    VIT_LARGE_M,
    prune24_magnitude,
    prune_tilewise,
    prune_blockwise,
    prune_elementwise,
    tile_shape,
    f16_normal,
    f16_uniform,
    i8_uniform,
    i8_weights,
    f32_scales,
    random_24_f16,
    random_24_i8,
    random_tw_i8,
    random_tw_f16,
    exact_int_24_f16,
    exact_int_tw_f16,
    one_hot_24,
    device_int_matrix,
    one_hot_tw,
)
