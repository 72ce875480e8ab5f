"""Float64 CPU oracle of the Muon step.  Test infrastructure only: used by
tests/, the smoke entry point and the benchmark's CPU-baseline leg; never by
the product path."""
