"""CPU oracle for the causal GQA attention forward: TEST INFRASTRUCTURE ONLY.

Only tests/, the package smoke check and the bench's CPU-baseline leg may
import this package.  It shares no code with the GPU path.
"""
