"""fp64 CPU oracle (test infrastructure only; see kl_oracle.py)."""
from .kl_oracle import (teacher_distribution, teacher_on_vocab, student_log_softmax,
                        kl_dense, kl_sparse, kl_chunked, kl_loops, kl_logits, topk_rows)

__all__ = ["teacher_distribution", "teacher_on_vocab", "student_log_softmax",
           "kl_dense", "kl_sparse", "kl_chunked", "kl_loops", "kl_logits", "topk_rows"]
