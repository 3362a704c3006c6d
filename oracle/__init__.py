"""Test infrastructure: the fp64 CPU oracle.  Not part of the product path;
only tests, the smoke check and the bench's CPU-baseline leg use it."""
