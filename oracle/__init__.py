"""CPU oracle of the LatentMoE layer forward: test infrastructure only.

Only the tests, the package smoke check and the benchmark's CPU-baseline leg
import this package.  The HIP library neither imports nor links it.
"""
