"""MI355X-native GDN decode path: a C-ABI HIP library (libgdn.so) and its thin
Python binding. ``inputs`` holds the seeded synthetic workloads."""
