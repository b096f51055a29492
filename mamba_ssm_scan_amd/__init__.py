"""Mamba-3 SSM core recurrence on AMD MI355X (gfx950): HIP kernels behind a C ABI.

The compute lives in `libm3.so` (HIP kernels + C entry points declared in
include/m3.h); `mamba_ssm_scan_amd.binding` marshals torch tensors into those
calls. `mamba_ssm_scan_amd.inputs` draws the seeded synthetic workloads.
"""
