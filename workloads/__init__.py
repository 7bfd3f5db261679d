"""Seeded synthetic inputs for the SwitchSD copy-speculation step.

This module is the one piece both the HIP path's tests/bench and the CPU oracle
read.  It holds none of the method's arithmetic: it draws token ids (Zipf
vocabulary draws with planted verbatim repeats), the anchor's hidden state and
the probe vector, query/key/value tensors and LM-head weights — nothing is
matched, scored, softmaxed or accepted here.

Workload shapes follow the pages' experimental setups (SwitchSD paper §4.1 and
the write-up's §3.1: Llama-3.1-8B, Qwen3-8B and Llama-3.3-70B targets, T = 0,
kappa = 5, W = 10, D = 20, tau ~ 0.4).  The copy-heavy / medium / light mix of
the write-up's CopyDiversity table (§2.2: 10.6 / 11.7 / 77.7 %) and the copy
trigger rates of its Table 1 set the planted-repeat densities; no dataset item
of any benchmark is used.
"""
from .gen import (CALIB_CONFIGS, CONFIGS, FWD_CONFIGS, SCAN_N, SCAN_SIZES, CalibWorkload,
                  FwdWorkload, Workload, device_tensors, f32_to_bf16_bits, generate, generate_calibration,
                  generate_forward, generate_with_ids, scan_ids_device, scan_ids_planted, spec,
                  to_torch)

__all__ = ["CALIB_CONFIGS", "CONFIGS", "FWD_CONFIGS", "CalibWorkload", "FwdWorkload", "Workload",
           "device_tensors",
           "f32_to_bf16_bits", "generate", "generate_calibration", "generate_forward",
           "generate_with_ids", "SCAN_N", "SCAN_SIZES", "scan_ids_device", "scan_ids_planted",
           "spec", "to_torch"]
