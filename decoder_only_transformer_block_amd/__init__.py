"""ncgpt: one-GPU MI355X (gfx950) forward + loss + backward of a nanochat-style
decoder-only Transformer stack, as hand-written HIP kernels behind a C ABI
(include/ncgpt.h).  `from decoder_only_transformer_block_amd import ncgpt`
loads the native library; importing the package itself loads nothing.
"""
