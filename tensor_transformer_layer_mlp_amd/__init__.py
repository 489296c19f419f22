"""One tensor-parallel rank's shard of a Megatron Transformer layer, native on MI355X (gfx950).

The compute lives in the C-ABI library `libtpshard.so` (hand-written HIP kernels); `binding`
marshals torch tensors into its entry points.  Importing the package does not load the library;
the first call does, and fails loudly if it has not been built.
"""
