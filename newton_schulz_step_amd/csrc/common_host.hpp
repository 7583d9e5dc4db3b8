// Constants shared by host planning and device kernels (no HIP dependency).
#pragma once

namespace muon {
constexpr int kMomThreads = 256;                 // threads per momentum block
constexpr int kMomChunk = kMomThreads * 4;       // elements per momentum block (4 per thread)
}  // namespace muon
