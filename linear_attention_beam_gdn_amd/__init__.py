"""GDN large-beam decode on MI355X (gfx950).

The hot path lives in the HIP library ``libgdnbeam.so`` behind the C ABI of
``include/gdn_beam.h``; ``binding`` is its thin ctypes wrapper.  Importing
the package does not load the library; ``binding.lib()`` does, and raises if
the library has not been built.
"""
