// qrs_window.h -- the per-window update record of qrs_window.hip, shared with
// the API layer that sizes the caller's buffer.  Internal to the library.
#pragma once

namespace qrs {

// Bytes of one record: GDN k, v FP16 + beta, alpha FP32 (528); KDA k, v and
// the decay factors exp(g) FP16 + beta FP32, padded to 16 bytes (784), so
// records stage into LDS in 16-byte pieces.
__host__ __device__ constexpr int window_record_bytes(int kind) { return kind == 0 ? 528 : 784; }

}  // namespace qrs
