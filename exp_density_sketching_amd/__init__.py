"""MI355X-native polynomial-method streaming sketch of the exp kernel, with the
exact streaming attention path beside it.

The compute lives in hand-written HIP kernels for gfx950 behind a C ABI
(include/expsketch.h, built into libexpsketch.so); this package is the thin
Python binding with the same call names.  Source of the method: "Rumo a Limites
Estritos para Atenção em Streaming" (gist.science, pt), sections "Definição do
Problema" and "Metodologia" (pillar "O Método Polinomial", Merge-and-Reduce).
"""

from ._binding import (LIB_PATH, EXPORTED, LAYOUTS, Sketch, SketchError, sketch_create,
                       sketch_layout, sketch_update_path, UPDATE_KERNELS, sketch_destroy, sketch_reset, sketch_update, sketch_merge,
                       sketch_query, sketch_step, sketch_set_center, sketch_set_staging,
                       sketch_export, sketch_state, sketch_timing,
                       sketch_kernel_times, exact_attend, exact_attend_noalloc,
                       exact_release_workspaces, exact_timing, exact_kernel_times, raw,
                       Coreset, coreset_create,
                       coreset_reset, coreset_update, coreset_merge, coreset_query,
                       coreset_export)

__all__ = ["LIB_PATH", "EXPORTED", "LAYOUTS", "Sketch", "SketchError", "sketch_create",
           "sketch_layout", "sketch_update_path", "UPDATE_KERNELS",
           "sketch_destroy", "sketch_reset", "sketch_update", "sketch_merge",
           "sketch_query", "sketch_step", "sketch_set_center", "sketch_set_staging",
           "sketch_export", "sketch_state", "sketch_timing",
           "sketch_kernel_times", "exact_attend", "exact_attend_noalloc", "exact_release_workspaces",
           "exact_timing", "exact_kernel_times", "raw",
           "Coreset", "coreset_create", "coreset_reset", "coreset_update", "coreset_merge",
           "coreset_query", "coreset_export"]
