"""fp64 CPU oracle of the GDN decode step. Test infrastructure only: the HIP
library and its Python binding never import this package."""
