"""CPU oracle of the Lighthouse Attention layer (test infrastructure only;
see oracle.lighthouse)."""
