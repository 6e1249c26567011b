"""MI355X (gfx950) batched conditional-flow-matching sampler.

The sampler is a HIP library with a C ABI (include/cfm.h); this package holds
its sources (csrc/), its build script and a thin ctypes binding. Importing the
package does not touch the GPU; creating a Sampler loads the library and fails
loudly if it has not been built.
"""
from ._lib import (CfmError, Sampler, adaln, attention_bf16, attention_bf16_noalloc, cfg_euler, check_sample_args,
                   config_from_shape, gemm_bf16, load, make_config, pack_weights, weight_manifest,
                   weights_bytes, workspace_bytes,
                   LIB_PATH, EXPORTS, KERNEL_CLASSES)

__all__ = ["CfmError", "Sampler", "adaln", "attention_bf16", "attention_bf16_noalloc", "cfg_euler", "check_sample_args",
           "config_from_shape", "gemm_bf16", "load",
           "make_config", "pack_weights", "weight_manifest", "weights_bytes", "workspace_bytes",
           "LIB_PATH", "EXPORTS", "KERNEL_CLASSES"]
