"""Measurement-only helpers: the streaming-rate reference kernels and the
clock-stamp breakdown of the headline decode kernel.  Nothing in the decode
path imports this package."""
