"""MI355X-native Shannonic codec for 8-bit quantised tensors.

The codec lives in the HIP library libshannonic.so (C ABI: include/shannonic.h);
``codec`` is its Python binding and ``datagen`` draws the seeded synthetic workloads.
Importing the package loads nothing; the library is loaded on first use and every call
raises if it has not been built.
"""
__all__ = ["codec", "datagen", "build"]
