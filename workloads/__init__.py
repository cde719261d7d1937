"""Seeded synthetic inputs for the paged GQA attention path.

This package draws random numbers and nothing else: request lengths, token ids,
page permutations and N(0,1) query/key/value values (rounded to bf16 storage
where the workload is bf16).  It contains none of the method's arithmetic (no
rotation, no attention, no page-table construction), so both the CPU oracle and
the GPU path can take their inputs from it without sharing any computation.
"""

from .gen import Case, make_case, CASE_IDS  # noqa: F401
