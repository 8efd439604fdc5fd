"""MoE token dispatch and combine for AMD Instinct MI355X (gfx950).

* ``combine_topk_ids_amd.moe``       -- ctypes binding of libmoe (HIP kernels)
* ``combine_topk_ids_amd.workloads`` -- seeded synthetic inputs
* ``combine_topk_ids_amd._build``    -- hipcc build of libmoe.so

Importing the package loads nothing; importing ``.moe`` loads libmoe.so and
raises if it is missing.
"""
