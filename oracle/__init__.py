"""CPU oracle of the device-split all-to-all-v (test infrastructure only).

Only the tests, the smoke check and the benchmark's CPU-baseline leg may
import this package. The product path (``embeddings_a2av_virtual_amd``) never
does, and shares no code with it.
"""
