"""CPU oracle (fp64 NumPy) for the MLA decode step. Test infrastructure only."""
