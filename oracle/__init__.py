"""Plain float64 CPU oracle of the speculative-decoding verification step.

Test infrastructure only; see ``svo.h`` and ``svo.py``.
"""
