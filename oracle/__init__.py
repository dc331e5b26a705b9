"""CPU oracle of the MoE layer: test infrastructure only.  Imported by the
tests, the package smoke check and the CPU-baseline leg of the benchmark;
never by the product path."""
