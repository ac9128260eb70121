// Chunk kernels: one variant per stack depth up to kChunkRegLayers (layers in
// registers) plus one for any depth, each in four modes (see fi_tables.h).
#include <array>
#include <utility>

#include "fi_tables.h"
#include "fi_chunk.h"

namespace fi {

namespace {
template <int... I>
constexpr std::array<ChunkK, 4 * sizeof...(I)> chunk_table(std::integer_sequence<int, I...>) {
    return {{&k_chunk<I / 4, I % 4>...}};
}
constexpr auto kChunkKernels = chunk_table(std::make_integer_sequence<int, 4 * (kChunkRegLayers + 1)>{});
}  // namespace

ChunkK chunk_k(int mt, int mode) {
    if (mt < 0 || mt > kChunkRegLayers || mode < 0 || mode > 3) return nullptr;
    return kChunkKernels[4 * mt + mode];
}

}  // namespace fi
