// bf16 split-K paged flash-decode: design notes and helpers of the decode
// statements in decode_body.inc, which the decode kernel and the fused
// selection + decode kernel both compile.  The method is described in
// decode.hip.
#pragma once
#include "common.h"

namespace sa {

// The list, block table, lengths and counts arrive as restrict kernel
// arguments: the kernel never writes them, so their wave-uniform reads compile
// to scalar loads, which complete on their own counter and never wait behind
// the K/V vector loads in flight.
// STAGED (d 128, per-KV-head lists): each wave copies its next 64-token
// chunk (K rows and V^T rows, 32 KiB) into its own LDS area with non-temporal
// load-to-LDS instructions of 1 KiB contiguous each, and reads the MFMA
// operands from there.  Streaming reads whose instructions cover whole cache
// lines run at ~6.1-6.4 TB/s on this HBM against ~5.4-6.0 TB/s for the
// operand-shaped register loads (16 rows x 64 B per instruction), which
// cannot use the non-temporal hint.  Every page of a per-KV-head list is read
// by one workgroup only, so nothing is lost by not keeping it in L2.
// LDS rows are XOR-swizzled so the operand reads are free of bank conflicts
// (gfx950 16-byte reads: four cycles per 64 lanes, lanes of a cycle by
// half-wave and the parity of lane bits 2..4, distinct 16-byte slots modulo
// 256 bytes):
//   K row r (256 B):   16-byte chunk c sits at slot c ^ (2 (r & 3) + 8 ((r >> 3) & 1))
//   V^T row d (128 B): token chunk c sits at slot c ^ (d & 6)
__device__ __forceinline__ int stg_kswz(int r) { return 2 * (r & 3) + 8 * ((r >> 3) & 1); }
__device__ __forceinline__ int stg_vswz(int d) { return d & 6; }

// Workgroup barriers the decode statements execute, each on every path
// (after the chunk loop when STAGED, then before the 4 waves' partials are
// combined).  A workgroup whose other waves skip the decode has them execute
// the same number of barriers, so every barrier is met by every wave.
constexpr int decode_body_barriers(bool staged) { return staged ? 2 : 1; }

}  // namespace sa
