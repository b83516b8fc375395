"""MI355X-native cluster-smoothed progressive residual KV-cache quantization.

A thin Python binding over the C-ABI library ``libqkv.so`` (include/qkv.h):
argument marshalling only.  Every step of the codec and of the attention read
runs in the library's HIP kernels; torch provides device memory and streams.
"""
from .binding import (QKV_BF16, QKV_F32, Codec, QkvError, config, lib, lib_path,
                      status_string, workspace_bytes)

__all__ = ["Codec", "QkvError", "config", "lib", "lib_path", "status_string", "workspace_bytes",
           "QKV_F32", "QKV_BF16"]
