// nf4_internal.h -- the device-side layer table and the tile constants shared
// by the kernels and the C entry points (not part of the public ABI).  The
// launchers are declared in nf4_launch.h.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace nf4k {

// One tile = one double-quantisation group = 256 blocks of 64 elements.
constexpr int kTileElems = 16384;
constexpr int kTileShift = 14;
constexpr int kThreads = 256;
constexpr int kPartsPerTile = 4;   // fp64 squared-error partials per tile (one per wave)

// Device copy of one nf4_layer plus the running tile count: tiles of all
// layers form one flat index space, layer l owning [tile_end - tiles(n), tile_end).
struct LayerDesc {
    const void* w;
    uint8_t* codes;
    float* absmax;
    int8_t* qabsmax;
    float* scale2;
    void* out;
    int64_t n;
    int64_t tile_end;
};
static_assert(sizeof(LayerDesc) == 64, "layer table entry is 64 bytes");

__host__ __device__ inline int64_t tiles_of(int64_t n) { return (n + kTileElems - 1) >> kTileShift; }

}  // namespace nf4k
