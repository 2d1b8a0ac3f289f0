"""CPU oracle of the OmniKVQuant hot path: test infrastructure only (see omnikv_oracle)."""
