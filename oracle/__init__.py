"""CPU oracle of the Veda hot path: test infrastructure, never the product path."""
