"""CPU oracle of the block-drafter path (float64 NumPy).

TEST INFRASTRUCTURE ONLY: imported by the tests, the smoke check and the
benchmark's CPU-baseline leg; never by the product path."""
