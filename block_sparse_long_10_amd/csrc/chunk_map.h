// Device side of ChunkMap: where a prefill tile of a (possibly batched) call
// lives.
#pragma once

#include "msa_launch.h"

namespace msa {

struct TileLoc {
  int seq, tile, prior, chunk, q0;  // sequence, local tile, lengths, first chunk row
};

// Tile u of the call (wave-uniform).
__device__ __forceinline__ TileLoc locate_tile(const ChunkMap& m, int u) {
  if (m.tile_seq == nullptr) return TileLoc{0, u, m.prior_len, m.chunk_len, 0};
  const int s = m.tile_seq[u];
  return TileLoc{s, u - m.tile_start[s], m.prior_lens[s], m.chunk_lens[s], m.q_start[s]};
}

}  // namespace msa
