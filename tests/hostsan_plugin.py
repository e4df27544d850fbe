"""pytest plugin for test_host_sanitize.py: load the host-sanitized library
(its path in DSPARK_HOSTSAN_LIB) before any test module asks for libdspark.so."""
import os

import draft_verify_sampling_markov_amd as dv

dv.load_library(os.environ["DSPARK_HOSTSAN_LIB"])
