"""fp64 CPU oracle for the rotated W4A16 linear -- test infrastructure only.

Only tests/, the smoke check and the benchmark's CPU-baseline leg import this
package.  It shares no code with the GPU library (rotation_int4_weight_amd).
"""
