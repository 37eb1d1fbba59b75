"""MI355X-native SparseGemv: N:M-sparse INT4 weight-only GEMV in 2bit-CSR form.

The package is a thin ctypes binding over the in-tree C-ABI library
``_lib/libsgemv.so`` (host packer + gfx950 HIP kernels). Every step of the
computation runs in that library; Python only marshals arguments, and
PyTorch only supplies device memory and streams.
"""
from .sgemv import (  # noqa: F401
    SgemvError, Desc, Plan, lib, lib_path, describe, select_groups, prune, pack, layout, run, plan, strerror,
    SparseGemvLayer, algorithmic_bytes, Task, MAX_GROUP, run_group, plan_group,
    describe_fp16, pack_fp16, layout_fp16, f64_to_f16, probe_read, probe_empty,
    LIST_MAX, run_list, plan_list, LIST_TABLE_MAX, ListLaunch, list_table, run_list_table,
)
