"""MI355X-native fp8 paged MQA logits + per-row top-k (the sparse-MLA decode indexer).

The HIP library (``libmqa.so``) holds every step of the computation. The
``mqa`` submodule binds its C-ABI; ``workloads`` draws seeded synthetic inputs.
Importing the package itself loads nothing, so input generation works on
machines without the built library.
"""
__all__ = ["mqa", "workloads"]
