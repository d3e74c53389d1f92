"""Oracle package: test infrastructure only (see mtp_oracle)."""
