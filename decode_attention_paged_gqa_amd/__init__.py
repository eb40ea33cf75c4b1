"""Paged GQA decode attention for MI355X (gfx950): HIP kernels behind a C ABI.

The binding loads ``libdecode_attn.so`` on first use and raises if it is
missing; there is no fallback path.
"""
