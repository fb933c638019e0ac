"""CPU oracle for the ConvRot quantized linear layer -- test infrastructure only.

Only the tests, the package smoke check and the benchmark's CPU-baseline leg may import it.
"""
