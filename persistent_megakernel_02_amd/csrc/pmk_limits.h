// Limits shared by the schedule builder / validator and the kernels (plain C++, no HIP types).
#pragma once

namespace pmk {

// Largest weight tile (bytes) one GEMV task may cover: tiles are addressed through a buffer
// resource with 32-bit offsets, and offsets at or past this bound read as zeros.
constexpr long long kMaxTileBytes = 0x7FFFFFF0ll;

// Positions one attention task holds: 8 waves x 2 matrix-core blocks of 32 positions; splits are
// whole 32-position blocks.
constexpr int kAttnMaxChunk = 512;

// Weight bytes a GEMV workgroup loads before its dependency wait (8 waves x 10 x 1 KiB).
constexpr long long kPrefetchBytes = 8 * 10 * 1024;

}  // namespace pmk
