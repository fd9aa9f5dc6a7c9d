"""CPU oracle for the quantized linear path.  Test infrastructure only: the
tests, the smoke check and the benchmark's CPU-baseline leg import it; the
product path never does."""
