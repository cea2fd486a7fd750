// Internal interface of the device self-check (selfcheck.cpp), shared by
// rgg_selfcheck (caller workspace) and rgg_selfcheck_noalloc (noalloc.hip).
#pragma once

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

namespace rgg {

// Bytes of device staging the self-check uses (inputs and outputs of every
// check, laid out in selfcheck.cpp), and of each host image.
constexpr size_t kSelfcheckBytes = 827392;

// Runs the checks selected by `checks` (bits 0-6, as in rgg.h) over device
// staging `ws` (kSelfcheckBytes, 256-byte aligned) on `stream`, with host
// images `in` and `out` of kSelfcheckBytes each; waits for the stream.
// Returns RGG_OK, RGG_ERR_SELFCHECK (bits in *failed) or the status of a
// failing call.
int selfcheck_run(uint8_t *ws, hipStream_t stream, uint32_t checks, uint32_t *failed, uint8_t *in,
                  uint8_t *out);

// Looks up this device's self-check scratch array once (noalloc.hip).
int noalloc_prepare(int device);

}  // namespace rgg
