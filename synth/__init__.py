"""Seeded synthetic inputs shared by the CPU oracle and the GPU path.

``synth.gen`` (NumPy) and ``synth.device`` (HIP, via ctypes) implement one
counter-based generator; ``synth.workloads`` holds the workload sizes and
bucket schedules; ``synth.probe`` streams plain reads, writes and copies whose
rates the bench reports as the box's practical HBM ceilings.  Nothing here
computes any part of the ZeRO method.
"""
