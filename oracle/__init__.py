"""Plain CPU oracle of the predictor-gated sparse FFN -- test infrastructure only.

Only tests, the package smoke check and the benchmark's CPU-baseline leg may
import this package.  It shares no code with the GPU library.
"""
