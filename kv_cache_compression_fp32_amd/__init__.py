"""MI355X (gfx950) compressor of the DeepSeek-V4.1 compressed-attention KV cache.

The compute path is the C-ABI library libkvc.so (hand-written HIP kernels);
`kv_cache_compression_fp32_amd.kvc` is its thin Python binding. Importing this
package loads nothing: the library is loaded on first use of the binding.
"""
