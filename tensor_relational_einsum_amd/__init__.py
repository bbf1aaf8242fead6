"""jagg: join-agg einsum executor for AMD MI355X (gfx950).

The binding (``tensor_relational_einsum_amd.jagg``) loads ``libjagg.so``
lazily, so importing the package, or its input generators, needs no GPU.
"""
__all__ = ["jagg", "inputs", "build"]
