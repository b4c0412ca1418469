"""CommunityKV sparse decode step for AMD MI355X (gfx950).

The HIP library (libckv.so) holds every kernel of the decode path; the
``ckv`` submodule is its ctypes binding and ``synth`` draws seeded synthetic
workloads.  Importing the package loads nothing; ``ckv`` loads the library
on first import and raises if it has not been built.
"""
