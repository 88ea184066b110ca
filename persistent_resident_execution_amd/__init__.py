"""MI355X-native persistent decode engine.

The decode step runs in HIP kernels behind a C-ABI library
(``include/pre.h``); ``engine`` binds it with ctypes.  ``synth`` builds the
seeded synthetic inputs.  Importing the package loads nothing native; the
binding loads the library on first use and raises if it has not been built.
"""
