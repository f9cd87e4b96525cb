"""CPU oracle of the XPress Jacobi pass (test infrastructure; never imported by the product)."""
