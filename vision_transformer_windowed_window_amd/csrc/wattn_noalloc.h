// wattn_noalloc.h -- the library-held backward scratch (wattn_noalloc.hip), shared with the
// host API.
#pragma once

#include <hip/hip_runtime_api.h>

// Size of the library-held scratch on each device: 64 MiB, room for the backward pass of up to
// (64 MiB - 16 KiB H) / 136 query rows (B * Hgrid * Wgrid * H): 493327 with one head.
#define WATTN_NOALLOC_SCRATCH_BYTES (64u << 20)

hipError_t wattn_noalloc_scratch(hipStream_t stream, void** out);
