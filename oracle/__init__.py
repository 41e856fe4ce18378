"""The CPU oracle of the Dory token forward: test infrastructure only (tests,
the smoke check and the benchmark's CPU-baseline leg)."""
