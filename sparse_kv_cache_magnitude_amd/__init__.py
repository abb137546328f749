"""Hierarchical semi-structured sparse KV attention for MI355X (gfx950).

The compute path is the HIP library libhierasparse.so (C ABI in include/hierasparse.h); this
package is its thin Python binding (argument marshalling only) plus the seeded input generators.
Importing the package loads nothing; the first call into the binding loads the library and fails
loudly if it is missing.
"""
