"""Seeded synthetic inputs and the workload list for the small-M GEMM.

This package holds no arithmetic of the GEMM itself: it only draws and
encodes inputs.  Both the CPU oracle's tests and the HIP path's tests and
benchmark take their inputs from here.
"""
