"""Native-resolution ViT vision encoder (Qwen2-VL tower) for MI355X / gfx950.

The computation lives in libqv.so (hand-written HIP kernels behind the C ABI
of include/qv.h); this package only binds it to torch tensors and streams."""
from ._abi import QvError, header_functions, lib  # noqa: F401
from .encoder import (Encoder, KernelTimer, MergerConfig, MergerWeights, VisionConfig, VisionWeights,  # noqa: F401
                      fold_patch_weight, merge_workspace_size, pack_images, patch_merge, patch_opts, patch_width,
                      patchify, quantize_i8, seq_meta, smart_resize_grid, vision_forward,
                      vision_forward_noalloc,
                      vision_workspace_size)
