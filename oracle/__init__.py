"""fp64 CPU oracle for MiniMax Sparse Attention: test infrastructure only."""
