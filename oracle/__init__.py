"""CPU oracle (test infrastructure only): see kvs_oracle.py."""
