"""Request-length generator of the ai-infra-handbooks "Paged KV cache" page.

Section "Why paging" draws 200 (prompt, output) pairs with Python's ``random``
seeded with 0, prompt uniform on the integers 100..2000 and output uniform on
20..1500 (both ends included), and prints the memory utilization that results;
the tests pin this generator to those printed percentages.  The decode
workloads take the first pairs of the same stream: context = prompt + output.
"""
from __future__ import annotations

import random

PROMPT_RANGE = (100, 2000)
OUTPUT_RANGE = (20, 1500)


def p2_length_pairs(n: int, seed: int = 0) -> list[tuple[int, int]]:
    """First ``n`` (prompt, output) pairs of the seeded stream, drawn prompt-then-output."""
    rng = random.Random(seed)
    return [(rng.randint(*PROMPT_RANGE), rng.randint(*OUTPUT_RANGE)) for _ in range(n)]


def p2_context_lens(n: int, seed: int = 0) -> list[int]:
    return [p + o for p, o in p2_length_pairs(n, seed)]
