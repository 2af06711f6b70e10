"""CPU oracle for the NVFP4 weight-only linear.  Test infrastructure only: see nvfp4_oracle."""
