"""FlashAttention forward pass for AMD Instinct MI355X (gfx950).

``io_aware_tiled_04_amd.fa`` binds the C ABI of ``libfa.so`` (include/fa.h);
``io_aware_tiled_04_amd.workloads`` draws the seeded synthetic inputs;
``io_aware_tiled_04_amd.build`` compiles the HIP sources with hipcc.
The binding is imported on first use so that the input generators can be used
without loading the GPU library.
"""


def __getattr__(name):
    if name in ("fwd", "fwd_splitkv", "fwd_dropout", "fwd_kvouter", "bwd", "fa_fwd_kvouter",
                "fa_fwd_kvouter_workspace_size", "fa_fwd", "fa_fwd_f32", "fa_fwd_splitkv",
                "fa_fwd_splitkv_workspace_size", "fa_fwd_dropout", "fa_bwd", "fa_bwd_dropout",
                "fa_bwd_workspace_size",
                "fa_status_string", "FaError"):
        from . import fa
        return getattr(fa, name)
    raise AttributeError(name)
