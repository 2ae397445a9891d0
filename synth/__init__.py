"""Seeded synthetic inputs shared by the CPU oracle and the GPU path.

``synth.gen`` (NumPy) and ``synth.device`` (HIP, via ctypes) implement one
counter-based generator; ``synth.workloads`` holds the workload sizes and
bucket schedules.  Nothing here computes any part of the ZeRO method.
"""
