"""SwitchSD copy-speculation hot path on MI355X (gfx950).

The compute lives in libswitchsd.so (HIP kernels behind the C ABI declared in
include/switchsd.h).  This package holds its sources (csrc/), the build script
(build.py) and a thin ctypes binding (binding.py) with the ABI's names.
"""
from .binding import (SSD_BF16, SSD_F32, PackedWeight, SwitchSDError, abi_version, accept_longest,
                      accept_sample, blocktri_verify, blocktri_verify_accept, blocktri_verify_noalloc,
                      blocktri_verify_sample, calibrate, calibrate_workspace_bytes, commit_accepted,
                      copy_labels, copy_labels_workspace_bytes, kgram_retrieve, load, pack_gate_up,
                      pack_gate_up_bytes, pack_layer, pack_weight, pack_weight_bytes,
                      probe_kgram_retrieve, probe_logits, probe_score, verify_forward,
                      verify_forward_workspace_bytes, verify_workspace_bytes)

__all__ = ["SSD_BF16", "SSD_F32", "PackedWeight", "SwitchSDError", "abi_version", "accept_longest",
           "accept_sample", "blocktri_verify", "blocktri_verify_accept", "blocktri_verify_noalloc",
           "blocktri_verify_sample", "calibrate", "calibrate_workspace_bytes", "commit_accepted",
           "copy_labels", "copy_labels_workspace_bytes", "kgram_retrieve", "load", "pack_gate_up",
           "pack_gate_up_bytes", "pack_layer", "pack_weight", "pack_weight_bytes",
           "probe_kgram_retrieve", "probe_logits", "probe_score", "verify_forward",
           "verify_forward_workspace_bytes", "verify_workspace_bytes"]
