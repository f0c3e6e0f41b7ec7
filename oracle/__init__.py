"""fp64 CPU oracle for the KDA recurrence.  Test infrastructure only: imported by
the test suite, the smoke check and the benchmark's CPU-baseline leg, never by
the product path."""
