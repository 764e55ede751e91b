"""CPU oracle (test infrastructure only; see ``oracle.sad_oracle``)."""
