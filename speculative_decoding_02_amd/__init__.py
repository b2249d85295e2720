"""Medusa decode step for one AMD Instinct MI355X (gfx950).

The compute lives in ``libmedusa.so`` (HIP kernels behind the C ABI of
``include/medusa.h``); ``speculative_decoding_02_amd.medusa`` is its thin
Python binding and ``speculative_decoding_02_amd.decoder`` drives a full
Medusa decode loop through it.  Importing the package itself loads nothing.
"""
