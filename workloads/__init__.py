"""Seeded synthetic inputs shared by the tests, the smoke check and the benchmark.

Holds none of the method's arithmetic: random numbers, routing tables and row
bookkeeping only.  Neither the oracle nor the HIP library is imported here.
"""
