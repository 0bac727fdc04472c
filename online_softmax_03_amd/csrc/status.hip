// fa_strerror (include/fa.h): the text of every fa_status value. Kept apart
// from the kernels' host code so that a change of wording touches no kernel
// source.
#include "fa.h"

extern "C" {

const char* fa_strerror(int status) {
    switch (status) {
        case FA_OK: return "ok";
        case FA_ERR_NULL: return "a required pointer is NULL";
        case FA_ERR_SHAPE: return "B, H and N must be positive and the sizes must fit";
        case FA_ERR_HEADDIM: return "head dimension must be 64 or 128";
        case FA_ERR_DTYPE: return "unsupported (in_dtype, out_dtype) pair";
        case FA_ERR_SCALE: return "scale must be positive and finite";
        case FA_ERR_ALIGN: return "q, k, v, o must be 16-byte aligned and lse 4-byte aligned";
        case FA_ERR_TILE: return "no kernel for the requested tile shape";
        case FA_ERR_LAUNCH: return "kernel launch failed";
        case FA_ERR_SPLITS: return "num_splits must be in [1, FA_MAX_SPLITS]";
        case FA_ERR_WORKSPACE: return "workspace is NULL, not 16-byte aligned, or too small";
        case FA_ERR_OFFSET: return "max_offset must be 0 or 8";
        case FA_ERR_SCRATCH: return "split partials exceed the fixed scratch (FA_NOALLOC_SCRATCH_BYTES)";
        default: return "unknown status";
    }
}

}  // extern "C"
