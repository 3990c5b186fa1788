"""Packed-tree SSD (Mamba2) speculative verification and commit on AMD MI355X.

``binding`` is the Python face of the C-ABI HIP library (``libtree_ssd.so``);
``workloads`` holds the seeded synthetic inputs. Importing the package does
not load the HIP library; ``binding`` does, and fails loudly if it is absent.
"""
__all__ = ["binding", "workloads"]
