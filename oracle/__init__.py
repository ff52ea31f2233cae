"""CPU oracle (test infrastructure only): see msa_ref for the definition it computes."""
