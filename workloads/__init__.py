"""Seeded synthetic inputs (shapes and random bytes only) for the verify step."""
from .configs import (ALL, BY_NAME, DENSE_BF16, LONG_FP8, PAGE, PAGED_BF16, RAGGED_MIXED,
                      SPARSE_BF16, SUB_PAGE, TINY_FP32, VerifyWorkload)
from .gen import (DTYPE_NAME, AcceptCase, DenseCase, Lengths, SparseCase, draw_lengths,
                  make_accept_case, make_dense_case, make_sparse_case, raw_numpy, seed_for)
