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

// Linear-weight formats (pmk_dtype values): bits per element, elements per 16-byte chunk (the
// GEMV's load unit per lane), row bytes, and the scale element of the scaled formats (fp8: one
// fp32 per 128x128 block; int8 / int4: one bf16 per row and 128-column group).
constexpr int weight_bits(int wdt) { return wdt == 2 || wdt == 3 ? 8 : wdt == 4 ? 4 : 16; }
constexpr int weight_epl(int wdt) { return 128 / weight_bits(wdt); }
constexpr long long weight_row_bytes(int wdt, long long K) { return K * weight_bits(wdt) / 8; }
constexpr bool weight_is_int(int wdt) { return wdt == 3 || wdt == 4; }
constexpr int weight_scale_bytes(int wdt) { return wdt == 2 ? 4 : weight_is_int(wdt) ? 2 : 0; }

}  // namespace pmk
