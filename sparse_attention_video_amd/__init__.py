"""SVG-EAR sparse-attention hot path for AMD MI355X (gfx950).

The compute lives in the in-tree HIP library ``libsvgear.so`` (C ABI:
include/svgear.h); ``svgear`` is its thin Python binding."""
from . import svgear  # noqa: F401
from .svgear import (Layer, centroid_variances, centroids, kmeans, kmeanspp, load, quantize_fp8, route,  # noqa: F401
                     route_topp, sparse_attn, sparse_attn_fp8, sparse_attn_noalloc, version)
