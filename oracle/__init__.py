"""fp64 CPU oracle (test infrastructure only; never imported by the product path)."""
from .lca_oracle import *  # noqa: F401,F403
from .lca_oracle import plan, kept_fraction, summary_query, importance_scores, softmax  # noqa: F401
