"""MI355X-native multi-row sparse-attention decode core.

The compute path is the HIP library `libds_rows.so` (built from `csrc/`),
reached through the thin ctypes binding in `ds_rows.py`. Importing the package
does not load the library; `ds_rows.load()` does, and fails loudly when it is
missing.
"""
