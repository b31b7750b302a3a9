"""MI355X-native (gfx950) hybrid compressed attention (CSA / HCA) layer: a C-ABI HIP library (liblca.so) and its
Python binding.  See include/lca.h for the calls."""
from . import lca  # noqa: F401  (raises ImportError when liblca.so is not built)
