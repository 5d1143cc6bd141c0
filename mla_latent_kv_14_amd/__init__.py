"""libmla: absorbed Multi-Head Latent Attention decode over a paged latent cache, for MI355X (gfx950).

The compute path is the C-ABI library ``libmla.so`` (hand-written HIP kernels);
``mla_latent_kv_14_amd.binding`` is its thin ctypes binding.  Importing the
package does not load the library; ``inputs`` holds the seeded workload
generator.
"""
