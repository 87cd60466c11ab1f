"""CPU oracle of the GPT-2 training step: test infrastructure only.

Imported by the tests, the smoke check and the benchmark's CPU-baseline leg;
never by the product library.
"""
