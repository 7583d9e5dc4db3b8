// Constants shared by host planning and device kernels (no HIP dependency).
#pragma once

namespace muon {
constexpr int kChunkElemsHost = 32768;  // elements per momentum chunk
}  // namespace muon
